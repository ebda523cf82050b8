"""Build libmxfp4.so for gfx950 with hipcc (in-tree, next to this file).

    python -m precision_mxfp4_producers_amd.build

Every HIP source is compiled with
  -O3 --offload-arch=gfx950 -ffp-contract=off
  -Xclang -target-feature -Xclang -packed-fp32-ops
no fused multiply-add contraction (the producers' rounding decisions are
defined by single fp32 roundings) and no packed-fp32 instruction selection.
"""

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libmxfp4.so"
SOURCES = ["quantize.hip", "gemm.hip", "swiglu_bwd.hip", "dgrad_swiglu_bwd.hip", "nvfp4.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Test-only probes (tests/hip/*.hip): each becomes tests/hip/lib<name>.so.
# They run device helpers of the library on inputs a test chooses; nothing in
# the package loads them.
TEST_HIP = os.path.join(os.path.dirname(HERE), "tests", "hip")


# Measurement-only kernels (bench_kernels/*.hip): one library that bench.py
# loads for its reference measurements; not part of the ABI.
BENCH_SRC = os.path.join(HERE, "bench_kernels")
BENCH_LIB = os.path.join(HERE, "libmxfp4_bench.so")


def lib_path():
    return os.path.join(HERE, LIB_NAME)


def probe_path(name):
    return os.path.join(TEST_HIP, f"lib{name}.so")


def build(verbose=False, jobs=4):
    """Compile every source and link the shared library; raises on failure."""
    objs = []
    with tempfile.TemporaryDirectory(prefix="mxfp4_build_") as tmp:
        procs = []
        for src in SOURCES:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
            if len(procs) >= jobs:
                _wait(procs.pop(0))
        for p in procs:
            _wait(p)
        tmp_lib = lib_path() + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp_lib] + objs
        out = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        if out.returncode != 0:
            raise RuntimeError("link failed:\n" + out.stdout.decode())
        os.replace(tmp_lib, lib_path())
    return lib_path()


def build_bench_kernels(verbose=False):
    """Compile bench_kernels/*.hip into libmxfp4_bench.so."""
    srcs = sorted(os.path.join(BENCH_SRC, f) for f in os.listdir(BENCH_SRC) if f.endswith(".hip"))
    cmd = [HIPCC] + FLAGS + ["-shared"] + srcs + ["-o", BENCH_LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    _wait(("bench_kernels", _Done(p)))
    os.replace(BENCH_LIB + ".tmp", BENCH_LIB)
    return BENCH_LIB


def build_test_probes(verbose=False):
    """Compile every tests/hip/*.hip into its own shared library."""
    built = []
    if not os.path.isdir(TEST_HIP):
        return built
    for src in sorted(f for f in os.listdir(TEST_HIP) if f.endswith(".hip")):
        name = os.path.splitext(src)[0]
        out = probe_path(name)
        cmd = [HIPCC] + FLAGS + ["-shared", os.path.join(TEST_HIP, src), "-o", out + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        _wait((src, _Done(p)))
        os.replace(out + ".tmp", out)
        built.append(out)
    return built


class _Done:
    """A finished subprocess.run result in the shape _wait expects."""

    def __init__(self, r):
        self.returncode, self._out = r.returncode, r.stdout

    def communicate(self):
        return self._out, None


def _wait(item):
    src, p = item
    out, _ = p.communicate()
    text = out.decode()
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{text}")
    noise = [ln for ln in text.splitlines() if ln.strip() and "packed-fp32-ops" not in ln]
    if noise:
        sys.stderr.write(f"[{src}]\n" + "\n".join(noise) + "\n")


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_bench_kernels(verbose=True))
    print(build_test_probes(verbose=True))
