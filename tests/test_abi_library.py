"""The C-ABI library loads on the CPU and exports every symbol include/*.h
declares (no compute calls: there is no GPU here)."""

import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "precision_mxfp4_producers_amd", "libmxfp4.so")


def declared_functions():
    names = set()
    for hdr in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(hdr).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*[A-Za-z_][\w\s\*]*?\b(fp4_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


def test_header_declares_the_hot_path_calls():
    names = declared_functions()
    for n in ("fp4_quantize_rows", "fp4_quantize_cols", "fp4_quantize_dual", "fp4_quantize_w2d32", "fp4_gemm",
              "fp4_gemm_pair", "fp4_gemm_grouped",
              "fp4_swiglu_producer", "fp4_swiglu_backward", "fp4_swiglu_backward_producer",
              "fp4_gemm_swiglu_backward_producer", "fp4_nv_quantize_rows", "fp4_nv_quantize_w2d16", "fp4_nv_gemm"):
        assert n in names


def test_library_exports_every_declared_symbol():
    if not os.path.exists(LIB):
        pytest.fail("libmxfp4.so is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_binding_signatures_cover_the_header():
    import precision_mxfp4_producers_amd as mx
    assert set(mx.EXPORTS) == declared_functions()


def test_host_only_calls():
    import numpy as np
    import precision_mxfp4_producers_amd as mx
    from oracle import philox as P
    lib = mx.load(LIB)
    assert lib.fp4_abi_version() >> 16 == 1
    assert lib.fp4_abi_version() & 0xFFFF >= 4      # fp4_gemm_pair, fp4_quantize_dual, the fp4_nv_* calls, fp4_gemm_grouped
    # the library's host sign-mask helper agrees with the oracle's generator
    for seed in (0, 1, 2 ** 40 + 7):
        assert mx.fp4_sign_mask_from_seed(seed) == P.sign_mask_from_seed(seed)


def test_argument_errors_are_reported_without_gpu_work():
    import precision_mxfp4_producers_amd as mx
    lib = mx.load(LIB)
    v = ctypes.c_void_p
    # null pointers -> FP4_EINVAL; bad shape -> FP4_ESHAPE; misalignment -> FP4_EALIGN
    assert lib.fp4_quantize_rows(None, 32, 32, 32, None, None, 0, 0, 0, None) == 1
    assert lib.fp4_quantize_rows(v(4096), 32, 33, 40, v(4096), v(4096), 0, 0, 0, None) == 2
    assert lib.fp4_quantize_rows(v(4098), 32, 32, 32, v(4096), v(4096), 0, 0, 0, None) == 3
    assert lib.fp4_quantize_rows(v(4096), 32, 32, 32, v(4096), v(4096), 7, 0, 0, None) == 1
    assert lib.fp4_quantize_cols(v(4096), 48, 32, 32, v(4096), v(4096), 0, 0, None) == 2
    assert lib.fp4_quantize_cols(v(4096), 32, 32, 32, v(4096), v(4096), 16, 0, None) == 1
    u64 = ctypes.c_uint64
    d4 = [v(4096)] * 2
    assert lib.fp4_quantize_dual(v(4096), 48, 32, 32, *d4, 1, u64(0), u64(0), *d4, 32, 0, None) == 2
    assert lib.fp4_quantize_dual(v(4096), 32, 32, 32, *d4, 3, u64(0), u64(0), *d4, 32, 0, None) == 1
    assert lib.fp4_quantize_dual(v(4096), 32, 32, 32, *d4, 1, u64(0), u64(0), *d4, 16, 0, None) == 1
    assert lib.fp4_quantize_dual(v(4096), 32, 32, 32, v(4096), v(4096), 1, u64(0), u64(0), None, v(4096), 32, 0,
                                 None) == 1
    assert lib.fp4_quantize_dual(v(4098), 32, 32, 32, *d4, 1, u64(0), u64(0), *d4, 32, 0, None) == 3
    assert lib.fp4_quantize_w2d32(v(4096), 32, 32, 16, v(4096), v(4096), v(4096), v(4096),
                                  ctypes.c_float(0.87), None) == 2
    assert lib.fp4_gemm(32, 32, 48, v(4096), v(4096), v(4096), v(4096), v(4096), 32, 0, None) == 2
    assert lib.fp4_gemm(32, 32, 32, v(4096), v(4096), v(4096), v(4096), v(4096), 32, 2, None) == 1
    pair = [v(4096)] * 8
    assert lib.fp4_gemm_pair(32, 32, 48, *pair, v(4096), 32, 0, None) == 2
    assert lib.fp4_gemm_pair(32, 32, 32, *pair, v(4096), 32, 2, None) == 1
    assert lib.fp4_gemm_pair(32, 32, 32, *pair[:7], None, v(4096), 32, 0, None) == 1
    assert lib.fp4_gemm_pair(32, 32, 32, *pair[:5], v(4100), *pair[6:], v(4096), 32, 0, None) == 3
    assert lib.fp4_swiglu_producer(32, 32, 32, v(4096), v(4096), v(4096), v(4096), v(4096), v(4096),
                                   v(4096), v(4096), v(4096), None, 0, None) == 1
    assert lib.fp4_swiglu_backward(32, 32, v(4096), 16, v(4096), v(4096), v(4096), v(4096), None) == 2
    u64 = ctypes.c_uint64
    bufs = [v(4096)] * 8
    assert lib.fp4_swiglu_backward_producer(32, 48, v(4096), 48, v(4096), v(4096), u64(0), u64(0), u64(1),
                                            0, *bufs, None) == 2
    assert lib.fp4_swiglu_backward_producer(32, 32, v(4096), 32, v(4096), None, u64(0), u64(0), u64(1),
                                            0, *bufs, None) == 1
    assert lib.fp4_swiglu_backward_producer(32, 32, v(4100), 32, v(4096), v(4096), u64(0), u64(0), u64(1),
                                            0, *bufs, None) == 3
    # dh row pitch of 2^23 floats or more: the kernel's 32-bit buffer offsets would overflow
    assert lib.fp4_swiglu_backward_producer(32, 32, v(4096), 1 << 23, v(4096), v(4096), u64(0), u64(0), u64(1),
                                            0, *bufs, None) == 2


def test_size_limit_errors_are_reported_without_gpu_work():
    """The launch-shape limits each declaration states come back as
    FP4_ESHAPE from the host checks (no pointer is dereferenced)."""
    import precision_mxfp4_producers_amd as mx
    lib = mx.load(LIB)
    v, u64 = ctypes.c_void_p, ctypes.c_uint64
    d4 = [v(4096)] * 2
    big_rows = 65536 * 128                                 # 65536 tiles of 128 tokens
    assert lib.fp4_quantize_cols(v(4096), big_rows, 32, 32, v(4096), v(4096), 32, 0, None) == 2
    assert lib.fp4_quantize_dual(v(4096), big_rows, 32, 32, *d4, 1, u64(0), u64(0), *d4, 32, 0, None) == 2
    assert lib.fp4_quantize_w2d32(v(4096), big_rows, 32, 32, v(4096), v(4096), v(4096), v(4096),
                                  ctypes.c_float(0.87), None) == 2
    assert lib.fp4_quantize_w2d32(v(4096), 32, 32, 1 << 22, v(4096), v(4096), v(4096), v(4096),
                                  ctypes.c_float(0.87), None) == 2
    assert lib.fp4_quantize_w2d32(v(4096), 32, 32, 32, v(4096), v(4096), v(4096), v(4096),
                                  ctypes.c_float(1.5), None) == 1
    huge = 1 << 40                                         # (2^32)^2 tiles of 256 x 256
    assert lib.fp4_gemm(huge, huge, 32, v(4096), v(4096), v(4096), v(4096), v(4096), huge, 0, None) == 2
    assert lib.fp4_gemm_pair(huge, huge, 256, *([v(4096)] * 8), v(4096), huge, 0, None) == 2
    assert lib.fp4_swiglu_producer(huge, huge, 32, *([v(4096)] * 10), 0, None) == 2
    fb = [v(4096)] * 8
    assert lib.fp4_gemm_swiglu_backward_producer(32, 32, 288, *([v(4096)] * 6), u64(0), u64(0), u64(1), 0, *fb,
                                                 None) == 2                     # d not a multiple of 256
    assert lib.fp4_gemm_swiglu_backward_producer(32, 1 << 22, 256, *([v(4096)] * 6), u64(0), u64(0), u64(1), 0,
                                                 *fb, None) == 2                # f beyond the 32-bit panel offsets
    assert lib.fp4_gemm_swiglu_backward_producer(32, 32, 256, *([v(4096)] * 5), None, u64(0), u64(0), u64(1), 0,
                                                 *fb, None) == 1
    assert lib.fp4_gemm_swiglu_backward_producer(32, 32, 256, *([v(4096)] * 6), u64(0), u64(0), u64(1), 0,
                                                 *fb[:6], v(4100), fb[7], None) == 3   # misaligned dbt_codes
    assert lib.fp4_gemm_swiglu_backward_producer(0, 64, 256, *([None] * 6), u64(0), u64(0), u64(1), 0,
                                                 *([None] * 8), None) == 0      # empty
    # just inside the limits the checks pass on to the (here absent) alignment check
    assert lib.fp4_quantize_cols(v(4098), big_rows - 128, 32, 32, v(4096), v(4096), 32, 0, None) == 3
    assert lib.fp4_quantize_w2d32(v(4098), 32, 32, (1 << 22) - 8, v(4096), v(4096), v(4096), v(4096),
                                  ctypes.c_float(0.87), None) == 3


def test_nvfp4_argument_errors_without_gpu_work():
    """The CTA-local NVFP4 calls: bad enums, shapes, limits, alignment, empty
    outputs -- all answered by the host checks."""
    import precision_mxfp4_producers_amd as mx
    lib = mx.load(LIB)
    v, u64 = ctypes.c_void_p, ctypes.c_uint64
    p = v(4096)
    assert lib.fp4_nv_quantize_rows(p, 32, 32, 32, p, p, p, p, 2, u64(0), u64(0), None) == 1
    assert lib.fp4_nv_quantize_rows(p, 32, 48, 48, p, p, p, p, 0, u64(0), u64(0), None) == 2
    assert lib.fp4_nv_quantize_rows(p, 65536 * 32, 32, 32, p, p, p, p, 0, u64(0), u64(0), None) == 2
    assert lib.fp4_nv_quantize_rows(p, 65535 * 32, 32, 32, v(4098), p, p, p, 0, u64(0), u64(0), None) == 3
    assert lib.fp4_nv_quantize_rows(p, 32, 32, 32, p, p, None, p, 0, u64(0), u64(0), None) == 1
    assert lib.fp4_nv_quantize_rows(None, 0, 64, 64, None, None, None, None, 1, u64(0), u64(0), None) == 0
    assert lib.fp4_nv_quantize_w2d16(p, 32, 48, 48, p, p, p, p, p, p, None) == 2
    assert lib.fp4_nv_quantize_w2d16(p, 32, 32, 32, p, p, p, p, None, p, None) == 1
    assert lib.fp4_nv_quantize_w2d16(p, 32, 32, 32, p, p, v(4100), p, p, p, None) == 3
    assert lib.fp4_nv_quantize_w2d16(None, 0, 32, 32, None, None, None, None, None, None, None) == 0
    assert lib.fp4_nv_gemm(32, 32, 32, p, p, p, 1, p, p, p, 0, p, 32, 0, None) == 2          # k % 64
    assert lib.fp4_nv_gemm(32, 32, 1 << 24, p, p, p, 1, p, p, p, 0, p, 32, 0, None) == 2
    assert lib.fp4_nv_gemm(32, 32, 64, p, p, p, -1, p, p, p, 0, p, 32, 0, None) == 1
    assert lib.fp4_nv_gemm(32, 32, 64, p, p, p, 1, p, p, p, 0, p, 32, 2, None) == 1
    assert lib.fp4_nv_gemm(32, 32, 64, p, p, p, 1, p, p, None, 0, p, 32, 0, None) == 1
    assert lib.fp4_nv_gemm(1 << 40, 1 << 40, 64, p, p, p, 1, p, p, p, 0, p, 1 << 40, 0, None) == 2
    assert lib.fp4_nv_gemm(32, 32, 64, p, p, p, 1, p, p, p, 0, p, 34, 0, None) == 3
    assert lib.fp4_nv_gemm(64, 64, 0, None, None, None, 1, None, None, None, 0, p, 64, 1, None) == 0
    assert lib.fp4_nv_gemm(0, 64, 64, None, None, None, 1, None, None, None, 0, None, 64, 0, None) == 0


def test_empty_calls_are_noops_without_gpu_work():
    """An output with no elements: FP4_OK, NULL pointers allowed, no device call."""
    import precision_mxfp4_producers_amd as mx
    lib = mx.load(LIB)
    u64 = ctypes.c_uint64
    assert lib.fp4_quantize_rows(None, 0, 64, 64, None, None, 1, 0, 0, None) == 0
    assert lib.fp4_quantize_rows(None, 5, 0, 0, None, None, 0, 0, 0, None) == 0
    assert lib.fp4_quantize_cols(None, 0, 64, 64, None, None, 32, 0, None) == 0
    assert lib.fp4_quantize_cols(None, 64, 0, 0, None, None, 0, 0, None) == 0
    assert lib.fp4_quantize_dual(None, 0, 64, 64, None, None, 1, u64(0), u64(0), None, None, 32, 0, None) == 0
    assert lib.fp4_quantize_w2d32(None, 0, 64, 64, None, None, None, None, ctypes.c_float(0.87), None) == 0
    assert lib.fp4_gemm(0, 64, 64, None, None, None, None, None, 64, 0, None) == 0
    assert lib.fp4_gemm(64, 0, 64, None, None, None, None, None, 0, 1, None) == 0
    assert lib.fp4_gemm_pair(0, 64, 64, *([None] * 8), None, 64, 0, None) == 0
    # k = 0 accumulating: C unchanged, no device work (C itself must still be given)
    assert lib.fp4_gemm_pair(64, 64, 0, *([None] * 8), ctypes.c_void_p(4096), 64, 1, None) == 0
    assert lib.fp4_swiglu_producer(0, 64, 64, None, None, None, None, None, None, None, None, None, None, 0, None) == 0
    assert lib.fp4_swiglu_backward(0, 64, None, 64, None, None, None, None, None) == 0
    assert lib.fp4_swiglu_backward_producer(64, 0, None, 0, None, None, u64(0), u64(0), u64(1), 0,
                                            *([None] * 8), None) == 0
    # negative sizes and bad enums are still rejected
    assert lib.fp4_quantize_rows(None, -1, 64, 64, None, None, 0, 0, 0, None) == 2
    assert lib.fp4_quantize_rows(None, 0, 64, 64, None, None, 5, 0, 0, None) == 1
    assert lib.fp4_gemm(-32, 64, 64, None, None, None, None, None, 64, 0, None) == 2


def test_grouped_gemm_checks_every_problem_before_any_launch():
    """fp4_gemm_grouped answers bad counts and each problem's errors on the
    host, and checks all problems before it enqueues anything: a valid first
    problem beside an invalid second one gives the second one's error, not a
    launch failure (there is no GPU here)."""
    import precision_mxfp4_producers_amd as mx
    lib = mx.load(LIB)
    P = mx._GemmProblem
    v = ctypes.c_void_p
    p = v(4096)

    def call(*probs, count=None):
        arr = (P * max(1, len(probs)))(*probs)
        return lib.fp4_gemm_grouped(ctypes.cast(arr, v), len(probs) if count is None else count, None)

    good = P(256, 256, 256, p, p, p, p, None, None, None, None, p, 256, 0)
    assert lib.fp4_gemm_grouped(None, 0, None) == 0
    assert lib.fp4_gemm_grouped(None, 1, None) == 1
    assert call(good, count=-1) == 1
    assert call(good, count=5) == 1
    assert call(good, P(256, 256, 48, p, p, p, p, None, None, None, None, p, 256, 0)) == 2       # k % 32
    assert call(good, P(256, 256, 256, p, p, p, p, None, None, None, None, p, 255, 0)) == 2      # ldc < n
    assert call(good, P(256, 256, 256, p, p, p, p, None, None, None, None, p, 256, 2)) == 1      # accumulate
    assert call(good, P(256, 256, 256, p, p, p, None, None, None, None, None, p, 256, 0)) == 1   # b_scales
    assert call(good, P(256, 256, 256, p, p, p, p, p, p, p, None, p, 256, 0)) == 1               # pair, 3 of 4
    assert call(good, P(256, 256, 256, p, p, p, p, p, p, p, v(4100), p, 256, 0)) == 3            # pair alignment
    assert call(good, P(256, 256, 256, p, p, p, p, None, None, None, None, v(4100), 256, 0)) == 3
    huge = 1 << 40
    assert call(good, P(huge, huge, 256, p, p, p, p, None, None, None, None, p, huge, 0)) == 2
    # together above 2^31 - 1 tiles, each alone below
    half = 256 * 32768                                     # 2^30 tiles each
    big = P(half, half, 256, p, p, p, p, None, None, None, None, p, half, 0)
    assert call(big, big) == 2
    # empty products, and K = 0 accumulating, need no device work
    assert call(P(0, 256, 256, None, None, None, None, None, None, None, None, None, 256, 0),
                P(256, 256, 0, None, None, None, None, None, None, None, None, p, 256, 1)) == 0


def test_header_compiles_and_links_as_plain_c(tmp_path):
    """include/mxfp4.h is a C header: a C11 program built with gcc against it
    links to the library and gets the documented host-check answers."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = tmp_path / "c_abi.c"
    src.write_text(r'''
#include <stdio.h>
#include "mxfp4.h"
int main(void) {
  int fails = 0;
  if (fp4_abi_version() >> 16 != 1) ++fails;
  if (fp4_sign_mask_from_seed(7) > 0xFFFFu) ++fails;
  /* a bad rounding mode and an empty call, answered on the host */
  if (fp4_quantize_rows((const uint16_t*)4096, 32, 32, 32, (uint8_t*)4096, (uint8_t*)4096, (fp4_round)5, 0, 0, NULL)
      != FP4_EINVAL) ++fails;
  if (fp4_nv_gemm(0, 64, 64, NULL, NULL, NULL, 1, NULL, NULL, NULL, 0, NULL, 64, 0, NULL) != FP4_OK) ++fails;
  {
    fp4_gemm_problem g[2] = {{0, 64, 64, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 64, 0},
                             {64, 64, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, (float*)4096, 64, 1}};
    if (fp4_gemm_grouped(g, 2, NULL) != FP4_OK) ++fails;
    if (fp4_gemm_grouped(g, FP4_GEMM_GROUP_MAX + 1, NULL) != FP4_EINVAL) ++fails;
  }
  printf("c_abi: %d failure(s)\n", fails);
  return fails;
}
''')
    exe = tmp_path / "c_abi"
    libdir = os.path.dirname(LIB)
    cmd = [gcc, "-std=c11", "-Wall", "-Werror=implicit-function-declaration", "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", str(src), "-L", libdir, "-lmxfp4",
           "-Wl,-rpath," + libdir, "-o", str(exe)]
    b = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=120)
    assert b.returncode == 0, b.stdout.decode()[-3000:]
    r = subprocess.run([str(exe)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=60)
    assert r.returncode == 0 and b"0 failure(s)" in r.stdout, r.stdout.decode()[-2000:]
