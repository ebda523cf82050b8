"""Python binding of libmxfp4: MXFP4 producers and block-scaled E2M1 GEMM on gfx950.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
declared in include/mxfp4.h.  torch provides device memory and the current
stream.  There is no fallback: if the shared library is missing or no GPU is
visible, the calls raise.

Functions carry the C names.  Output buffers may be passed in (the ABI's
explicit-ownership form) or are allocated with torch.empty.  bf16 tensors may
be torch.bfloat16 or int16/uint16 bit patterns.
"""

import ctypes
import os

import torch

from .build import lib_path

FP4_RTN, FP4_SR = 0, 1
STATUS = {0: "FP4_OK", 1: "FP4_EINVAL", 2: "FP4_ESHAPE", 3: "FP4_EALIGN", 4: "FP4_EHIP"}

_lib = None

_i64, _u64, _u32, _int, _vp = ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_void_p

_SIGS = {
    "fp4_quantize_rows": [_vp, _i64, _i64, _i64, _vp, _vp, _int, _u64, _u64, _vp],
    "fp4_quantize_cols": [_vp, _i64, _i64, _i64, _vp, _vp, _int, _u32, _vp],
    "fp4_quantize_dual": [_vp, _i64, _i64, _i64, _vp, _vp, _int, _u64, _u64, _vp, _vp, _int, _u32, _vp],
    "fp4_quantize_w2d32": [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, ctypes.c_float, _vp],
    "fp4_gemm": [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _i64, _int, _vp],
    "fp4_gemm_pair": [_i64, _i64, _i64] + [_vp] * 9 + [_i64, _int, _vp],
    "fp4_gemm_grouped": [_vp, _int, _vp],
    "fp4_swiglu_producer": [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _u32, _vp],
    "fp4_swiglu_backward": [_i64, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp],
    "fp4_swiglu_backward_producer": [_i64, _i64, _vp, _i64, _vp, _vp, _u64, _u64, _u64, _u32] + [_vp] * 9,
    "fp4_gemm_swiglu_backward_producer": [_i64, _i64, _i64] + [_vp] * 6 + [_u64, _u64, _u64, _u32] + [_vp] * 9,
    "fp4_nv_quantize_rows": [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _int, _u64, _u64, _vp],
    "fp4_nv_quantize_w2d16": [_vp, _i64, _i64, _i64] + [_vp] * 7,
    "fp4_nv_gemm": [_i64, _i64, _i64, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _i64, _vp, _i64, _int, _vp],
    "fp4_sign_mask_from_seed": [_u64],
    "fp4_last_hip_error": [],
    "fp4_abi_version": [],
}
EXPORTS = tuple(_SIGS)


class Fp4Error(RuntimeError):
    pass


def load(path=None):
    """Load the shared library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or lib_path()
    if not os.path.exists(path):
        raise Fp4Error(f"{path} is missing: build it with __graft_entry__.build() "
                       "or python -m precision_mxfp4_producers_amd.build")
    lib = ctypes.CDLL(path)
    for name, args in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_uint32 if name == "fp4_sign_mask_from_seed" else ctypes.c_int
    _lib = lib
    return lib


def _check(status):
    if status != 0:
        msg = STATUS.get(status, str(status))
        if status == 4:
            msg += f" (hipError {load().fp4_last_hip_error()})"
        raise Fp4Error(msg)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise Fp4Error(f"{name} must be a CUDA (HIP) tensor")
    # the kernels run on the current device's current stream: a tensor on
    # another device would be read through that device's memory, unmapped here
    if t.device.index != torch.cuda.current_device():
        raise Fp4Error(f"{name} is on {t.device}, the current device is cuda:{torch.cuda.current_device()}")
    return t


def _bf16_2d(x, name):
    _dev(x, name)
    if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise Fp4Error(f"{name} must hold bf16 values or their 16-bit patterns")
    if x.dim() != 2 or x.stride(1) != 1:
        raise Fp4Error(f"{name} must be 2-D with unit column stride")
    return x


def _out(t, shape, dtype, device, name):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _dev(t, name)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise Fp4Error(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}")
    return t


def _p(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def fp4_quantize_rows(x, mode=FP4_RTN, seed=0, offset=0, codes=None, scales=None):
    x = _bf16_2d(x, "x")
    rows, cols = x.shape
    codes = _out(codes, (rows, cols // 2), torch.uint8, x.device, "codes")
    scales = _out(scales, (rows, cols // 32), torch.uint8, x.device, "scales")
    _check(load().fp4_quantize_rows(_p(x), rows, cols, x.stride(0), _p(codes), _p(scales), int(mode),
                                    int(seed), int(offset), _stream()))
    return codes, scales


def fp4_quantize_cols(x, hadamard=0, sign_mask16=0, codes_t=None, scales_t=None):
    x = _bf16_2d(x, "x")
    rows, cols = x.shape
    codes_t = _out(codes_t, (cols, rows // 2), torch.uint8, x.device, "codes_t")
    scales_t = _out(scales_t, (cols, rows // 32), torch.uint8, x.device, "scales_t")
    _check(load().fp4_quantize_cols(_p(x), rows, cols, x.stride(0), _p(codes_t), _p(scales_t), int(hadamard),
                                    int(sign_mask16), _stream()))
    return codes_t, scales_t


def fp4_quantize_dual(x, mode=FP4_RTN, seed=0, offset=0, hadamard=0, sign_mask16=0, codes=None, scales=None,
                      codes_t=None, scales_t=None):
    """Row-facing and column-facing MXFP4 of x from one read: returns
    (codes, scales, codes_t, scales_t), the bytes of fp4_quantize_rows and
    fp4_quantize_cols."""
    x = _bf16_2d(x, "x")
    rows, cols = x.shape
    codes = _out(codes, (rows, cols // 2), torch.uint8, x.device, "codes")
    scales = _out(scales, (rows, cols // 32), torch.uint8, x.device, "scales")
    codes_t = _out(codes_t, (cols, rows // 2), torch.uint8, x.device, "codes_t")
    scales_t = _out(scales_t, (cols, rows // 32), torch.uint8, x.device, "scales_t")
    _check(load().fp4_quantize_dual(_p(x), rows, cols, x.stride(0), _p(codes), _p(scales), int(mode), int(seed),
                                    int(offset), _p(codes_t), _p(scales_t), int(hadamard), int(sign_mask16),
                                    _stream()))
    return codes, scales, codes_t, scales_t


def fp4_quantize_w2d32(w, finer_ratio=0.87, row_codes=None, row_scales=None, col_codes=None, col_scales=None):
    w = _bf16_2d(w, "w")
    n, k = w.shape
    row_codes = _out(row_codes, (n, k // 2), torch.uint8, w.device, "row_codes")
    row_scales = _out(row_scales, (n, k // 32), torch.uint8, w.device, "row_scales")
    col_codes = _out(col_codes, (k, n // 2), torch.uint8, w.device, "col_codes")
    col_scales = _out(col_scales, (k, n // 32), torch.uint8, w.device, "col_scales")
    _check(load().fp4_quantize_w2d32(_p(w), n, k, w.stride(0), _p(row_codes), _p(row_scales), _p(col_codes),
                                     _p(col_scales), float(finer_ratio), _stream()))
    return row_codes, row_scales, col_codes, col_scales


def _gemm_shapes(pairs):
    """(m, n, k) of the products C (+)= sum of A B^T over `pairs` of
    (a_codes, a_scales, b_codes, b_scales) with names; all pairs alike."""
    for quad in pairs:
        for t, nm in quad:
            _dev(t, nm)
            if t.dtype != torch.uint8 or not t.is_contiguous() or t.dim() != 2:
                raise Fp4Error(f"{nm} must be a contiguous 2-D uint8 tensor")
    (ac, _), _, (bc, _), _ = pairs[0]
    m, k2 = ac.shape
    n = bc.shape[0]
    k = 2 * k2
    for (ac, _), (asc, _), (bc, _), (bsc, _) in pairs:
        if (tuple(ac.shape) != (m, k2) or tuple(bc.shape) != (n, k2) or tuple(asc.shape) != (m, k // 32)
                or tuple(bsc.shape) != (n, k // 32)):
            raise Fp4Error("operand shapes disagree")
    return m, n, k


def _gemm_out(c, m, n, accumulate, device):
    if c is None:
        if accumulate:
            raise Fp4Error("accumulate needs an output tensor")
        return torch.empty((m, n), dtype=torch.float32, device=device)
    _dev(c, "c")
    if c.dtype != torch.float32 or c.dim() != 2 or c.stride(1) != 1 or tuple(c.shape) != (m, n):
        raise Fp4Error("c must be fp32 [m][n] with unit column stride")
    return c


def fp4_gemm(a_codes, a_scales, b_codes, b_scales, c=None, accumulate=False):
    m, n, k = _gemm_shapes([((a_codes, "a_codes"), (a_scales, "a_scales"), (b_codes, "b_codes"),
                             (b_scales, "b_scales"))])
    c = _gemm_out(c, m, n, accumulate, a_codes.device)
    _check(load().fp4_gemm(m, n, k, _p(a_codes), _p(a_scales), _p(b_codes), _p(b_scales), _p(c), c.stride(0),
                           1 if accumulate else 0, _stream()))
    return c


def fp4_gemm_pair(a1_codes, a1_scales, b1_codes, b1_scales, a2_codes, a2_scales, b2_codes, b2_scales, c=None,
                  accumulate=False):
    """C (+)= A1 B1^T + A2 B2^T, one fp32 sum over both K ranges (same shapes)."""
    ops = ((a1_codes, "a1_codes"), (a1_scales, "a1_scales"), (b1_codes, "b1_codes"), (b1_scales, "b1_scales"),
           (a2_codes, "a2_codes"), (a2_scales, "a2_scales"), (b2_codes, "b2_codes"), (b2_scales, "b2_scales"))
    m, n, k = _gemm_shapes([ops[:4], ops[4:]])
    c = _gemm_out(c, m, n, accumulate, a1_codes.device)
    _check(load().fp4_gemm_pair(m, n, k, *(_p(t) for t, _ in ops), _p(c), c.stride(0), 1 if accumulate else 0,
                                _stream()))
    return c


class _GemmProblem(ctypes.Structure):
    _fields_ = [("m", _i64), ("n", _i64), ("k", _i64), ("a_codes", _vp), ("a_scales", _vp), ("b_codes", _vp),
                ("b_scales", _vp), ("a2_codes", _vp), ("a2_scales", _vp), ("b2_codes", _vp), ("b2_scales", _vp),
                ("c", _vp), ("ldc", _i64), ("accumulate", _int)]


GEMM_GROUP_MAX = 4
_GEMM_KEYS = ("a_codes", "a_scales", "b_codes", "b_scales")
_GEMM2_KEYS = ("a2_codes", "a2_scales", "b2_codes", "b2_scales")


def fp4_gemm_grouped(problems):
    """Independent products in one launch.  Each problem is a dict with
    a_codes, a_scales, b_codes, b_scales, optionally a2_codes, a2_scales,
    b2_codes, b2_scales (the fp4_gemm_pair form), c and accumulate; returns the
    list of C tensors (allocated where c is missing)."""
    if len(problems) > GEMM_GROUP_MAX:
        raise Fp4Error(f"at most {GEMM_GROUP_MAX} problems per call")
    arr = (_GemmProblem * max(1, len(problems)))()
    outs = []
    for q, pr in enumerate(problems):
        quads = [tuple((pr[key], f"problems[{q}].{key}") for key in _GEMM_KEYS)]
        pair = any(pr.get(key) is not None for key in _GEMM2_KEYS)
        if pair:
            quads.append(tuple((pr.get(key), f"problems[{q}].{key}") for key in _GEMM2_KEYS))
        m, n, k = _gemm_shapes(quads)
        acc = bool(pr.get("accumulate", False))
        c = _gemm_out(pr.get("c"), m, n, acc, pr["a_codes"].device)
        outs.append(c)
        ptrs = [_p(pr[key]) for key in _GEMM_KEYS] + [_p(pr[key]) if pair else None for key in _GEMM2_KEYS]
        arr[q] = _GemmProblem(m, n, k, *ptrs, _p(c), c.stride(0), 1 if acc else 0)
    _check(load().fp4_gemm_grouped(ctypes.cast(arr, _vp), len(problems), _stream()))
    return outs


def _u8_2d(t, name, shape=None):
    _dev(t, name)
    if t.dtype != torch.uint8 or t.dim() != 2 or not t.is_contiguous():
        raise Fp4Error(f"{name} must be a contiguous 2-D uint8 tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise Fp4Error(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    return t


def _bf16_tf(x, name, shape):
    _dev(x, name)
    if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or not x.is_contiguous() or tuple(x.shape) != shape:
        raise Fp4Error(f"{name} must be a contiguous bf16 tensor of shape {shape}")
    return x


def fp4_swiglu_producer(x_codes, x_scales, w13_codes, w13_scales, sign_mask16=0, emit_cols=True,
                        a=None, b=None, h_codes=None, h_scales=None, ht_codes=None, ht_scales=None):
    _u8_2d(x_codes, "x_codes")
    _u8_2d(w13_codes, "w13_codes")
    t, d2 = x_codes.shape
    d = 2 * d2
    f2, wd2 = w13_codes.shape
    if wd2 != d2:
        raise Fp4Error(f"w13_codes has {2 * wd2} values per row, x_codes {d}")
    if f2 % 2:
        raise Fp4Error("w13_codes must stack W1 and W3: an even number of rows")
    f = f2 // 2
    _u8_2d(x_scales, "x_scales", (t, d // 32))
    _u8_2d(w13_scales, "w13_scales", (f2, d // 32))
    dev = x_codes.device
    a = _out(a, (t, f), torch.int16, dev, "a") if a is not None else torch.empty((t, f), dtype=torch.int16, device=dev)
    b = _out(b, (t, f), torch.int16, dev, "b") if b is not None else torch.empty((t, f), dtype=torch.int16, device=dev)
    h_codes = _out(h_codes, (t, f // 2), torch.uint8, dev, "h_codes")
    h_scales = _out(h_scales, (t, f // 32), torch.uint8, dev, "h_scales")
    if emit_cols:
        ht_codes = _out(ht_codes, (f, t // 2), torch.uint8, dev, "ht_codes")
        ht_scales = _out(ht_scales, (f, t // 32), torch.uint8, dev, "ht_scales")
    else:
        ht_codes = ht_scales = None
    _check(load().fp4_swiglu_producer(t, f, d, _p(x_codes), _p(x_scales), _p(w13_codes), _p(w13_scales), _p(a),
                                      _p(b), _p(h_codes), _p(h_scales), _p(ht_codes), _p(ht_scales),
                                      int(sign_mask16), _stream()))
    return a, b, h_codes, h_scales, ht_codes, ht_scales


def fp4_swiglu_backward(dh, a, b, da=None, db=None):
    _dev(dh, "dh")
    _dev(a, "a")
    t, f = a.shape
    if dh.dtype != torch.float32 or dh.dim() != 2 or dh.stride(1) != 1 or tuple(dh.shape) != (t, f):
        raise Fp4Error("dh must be fp32 [t][f] with unit column stride")
    _bf16_tf(a, "a", (t, f))
    _bf16_tf(b, "b", (t, f))
    da = _out(da, (t, f), torch.int16, a.device, "da") if da is not None else torch.empty((t, f), dtype=torch.int16, device=a.device)
    db = _out(db, (t, f), torch.int16, a.device, "db") if db is not None else torch.empty((t, f), dtype=torch.int16, device=a.device)
    _check(load().fp4_swiglu_backward(t, f, _p(dh), dh.stride(0), _p(a), _p(b), _p(da), _p(db), _stream()))
    return da, db


def fp4_swiglu_backward_producer(dh, a, b, seed, offset_a, offset_b, sign_mask16, out=None):
    """dA, dB of the SwiGLU backward emitted directly as MXFP4: returns
    ((da_codes, da_scales), (db_codes, db_scales), (dat_codes, dat_scales),
    (dbt_codes, dbt_scales)) -- row-facing SR and column-facing H32."""
    _dev(dh, "dh")
    _dev(a, "a")
    t, f = a.shape
    if dh.dtype != torch.float32 or dh.dim() != 2 or dh.stride(1) != 1 or tuple(dh.shape) != (t, f):
        raise Fp4Error("dh must be fp32 [t][f] with unit column stride")
    _bf16_tf(a, "a", (t, f))
    _bf16_tf(b, "b", (t, f))
    dev = a.device
    shapes = [(t, f // 2), (t, f // 32), (t, f // 2), (t, f // 32),
              (f, t // 2), (f, t // 32), (f, t // 2), (f, t // 32)]
    names = ["da_codes", "da_scales", "db_codes", "db_scales", "dat_codes", "dat_scales", "dbt_codes", "dbt_scales"]
    out = list(out) if out is not None else [None] * 8
    bufs = [_out(o, shp, torch.uint8, dev, nm) for o, shp, nm in zip(out, shapes, names)]
    _check(load().fp4_swiglu_backward_producer(t, f, _p(dh), dh.stride(0), _p(a), _p(b), int(seed), int(offset_a),
                                               int(offset_b), int(sign_mask16), *[_p(x) for x in bufs], _stream()))
    return (bufs[0], bufs[1]), (bufs[2], bufs[3]), (bufs[4], bufs[5]), (bufs[6], bufs[7])


def fp4_gemm_swiglu_backward_producer(dy_codes, dy_scales, w2c_codes, w2c_scales, a, b, seed, offset_a, offset_b,
                                      sign_mask16, out=None):
    """W2 Dgrad dH = Q_r(dY) W2_c^T with the SwiGLU backward producer in its
    epilogue: returns ((da_codes, da_scales), (db_codes, db_scales),
    (dat_codes, dat_scales), (dbt_codes, dbt_scales)), the bytes of fp4_gemm
    followed by fp4_swiglu_backward_producer, without dH in memory."""
    _u8_2d(dy_codes, "dy_codes")
    _u8_2d(w2c_codes, "w2c_codes")
    t, d2 = dy_codes.shape
    f, wd2 = w2c_codes.shape
    d = 2 * d2
    if wd2 != d2:
        raise Fp4Error(f"w2c_codes has {2 * wd2} values per row, dy_codes {d}")
    _u8_2d(dy_scales, "dy_scales", (t, d // 32))
    _u8_2d(w2c_scales, "w2c_scales", (f, d // 32))
    _bf16_tf(a, "a", (t, f))
    _bf16_tf(b, "b", (t, f))
    dev = a.device
    shapes = [(t, f // 2), (t, f // 32), (t, f // 2), (t, f // 32),
              (f, t // 2), (f, t // 32), (f, t // 2), (f, t // 32)]
    names = ["da_codes", "da_scales", "db_codes", "db_scales", "dat_codes", "dat_scales", "dbt_codes", "dbt_scales"]
    out = list(out) if out is not None else [None] * 8
    bufs = [_out(o, shp, torch.uint8, dev, nm) for o, shp, nm in zip(out, shapes, names)]
    _check(load().fp4_gemm_swiglu_backward_producer(t, f, d, _p(dy_codes), _p(dy_scales), _p(w2c_codes),
                                                    _p(w2c_scales), _p(a), _p(b), int(seed), int(offset_a),
                                                    int(offset_b), int(sign_mask16), *[_p(x) for x in bufs],
                                                    _stream()))
    return (bufs[0], bufs[1]), (bufs[2], bufs[3]), (bufs[4], bufs[5]), (bufs[6], bufs[7])


def fp4_nv_quantize_rows(x, mode=FP4_RTN, seed=0, offset=0, out=None):
    """CTA-local NVFP4 of x along its columns: returns (codes [r][c/2],
    scales [r][c/16] E4M3 bytes, factors [ceil(r/256)] fp32, panel maxima
    [ceil(r/256)] fp32)."""
    x = _bf16_2d(x, "x")
    rows, cols = x.shape
    panels = (rows + 255) // 256
    out = list(out) if out is not None else [None] * 4
    codes = _out(out[0], (rows, cols // 2), torch.uint8, x.device, "codes")
    scales = _out(out[1], (rows, cols // 16), torch.uint8, x.device, "scales")
    factors = _out(out[2], (panels,), torch.float32, x.device, "factors")
    amax = _out(out[3], (panels,), torch.float32, x.device, "panel_amax")
    _check(load().fp4_nv_quantize_rows(_p(x), rows, cols, x.stride(0), _p(codes), _p(scales), _p(factors),
                                       _p(amax), int(mode), int(seed), int(offset), _stream()))
    return codes, scales, factors, amax


def fp4_nv_quantize_w2d16(w, out=None):
    """CTA-local 2D16 weight encoding: returns (row_codes, row_scales,
    col_codes, col_scales, factor [1], amax [1])."""
    w = _bf16_2d(w, "w")
    n, k = w.shape
    shapes = [(n, k // 2), (n, k // 16), (k, n // 2), (k, n // 16)]
    names = ["row_codes", "row_scales", "col_codes", "col_scales"]
    out = list(out) if out is not None else [None] * 6
    bufs = [_out(o, shp, torch.uint8, w.device, nm) for o, shp, nm in zip(out[:4], shapes, names)]
    factor = _out(out[4], (1,), torch.float32, w.device, "factor")
    amax = _out(out[5], (1,), torch.float32, w.device, "amax")
    _check(load().fp4_nv_quantize_w2d16(_p(w), n, k, w.stride(0), *[_p(b) for b in bufs], _p(factor), _p(amax),
                                        _stream()))
    return (*bufs, factor, amax)


def fp4_nv_gemm(a_codes, a_scales, a_factors, b_codes, b_scales, b_factors, c=None, accumulate=False):
    """C (+)= RN(S_A S_B) * sum_k dec(A) dec(B) over CTA-local NVFP4 operands.
    A factor vector of one element is shared by all rows (stride 0); otherwise
    it holds one factor per 256-row panel."""
    _u8_2d(a_codes, "a_codes")
    _u8_2d(b_codes, "b_codes")
    m, k2 = a_codes.shape
    n = b_codes.shape[0]
    k = 2 * k2
    if b_codes.shape[1] != k2:
        raise Fp4Error("operand shapes disagree")
    _u8_2d(a_scales, "a_scales", (m, k // 16))
    _u8_2d(b_scales, "b_scales", (n, k // 16))
    strides = []
    for fac, rows, nm in ((a_factors, m, "a_factors"), (b_factors, n, "b_factors")):
        _dev(fac, nm)
        panels = (rows + 255) // 256
        if fac.dtype != torch.float32 or fac.dim() != 1 or not fac.is_contiguous() or fac.numel() not in (1, panels):
            raise Fp4Error(f"{nm} must be a contiguous fp32 vector of 1 or {panels} elements")
        strides.append(0 if fac.numel() == 1 else 1)
    if c is None:
        if accumulate:
            raise Fp4Error("accumulate needs an output tensor")
        c = torch.empty((m, n), dtype=torch.float32, device=a_codes.device)
    else:
        _dev(c, "c")
        if c.dtype != torch.float32 or c.dim() != 2 or c.stride(1) != 1 or tuple(c.shape) != (m, n):
            raise Fp4Error("c must be fp32 [m][n] with unit column stride")
    _check(load().fp4_nv_gemm(m, n, k, _p(a_codes), _p(a_scales), _p(a_factors), strides[0], _p(b_codes),
                              _p(b_scales), _p(b_factors), strides[1], _p(c), c.stride(0), 1 if accumulate else 0,
                              _stream()))
    return c


def fp4_sign_mask_from_seed(seed):
    return int(load().fp4_sign_mask_from_seed(int(seed)))
