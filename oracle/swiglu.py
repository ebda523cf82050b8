"""SwiGLU producer arithmetic: the shared exp, forward h and backward dA/dB.

"Format-Aware Fusion for Fast FP4 Pretraining", §3.2 (gated FFN): the paired
W1/W3 projections run as one producer whose output, h = SiLU(a) * b, goes out
already in FP4 for W2; in the backward pass the gradient that W2's Dgrad
returns is multiplied through the gate's derivative inside the same fused
step; the saved a and b stay exact bf16, and the fusion moves data only: the
model computed is unchanged.

Reading of the precision chain (the pages print none): the serial BF16
schedule.  a, b are the fp32 GEMM outputs rounded to bf16 (RNE) and saved;
all further steps are single fp32 IEEE round-to-nearest operations in the
written order, with no fused multiply-add outside exp_spec:
  sig = 1 / (1 + exp_spec(-a));  s = a * sig;  h = bf16(s * b)
  dA  = bf16(((dH * b) * sig) * (1 + a * (1 - sig)));  dB = bf16(dH * s)
dH is the fp32 output of the W2 Dgrad contraction, used without rounding.

exp_spec is a textbook Cody-Waite exponential written from its definition, so
that both sides can evaluate it identically.  fma(u, v, w) is RN_fp32(u*v + w)
with a single rounding:
  n  = rint(x * LOG2E)                       (fp32 product, ties to even)
  r  = fma(-n, LN2_LO, fma(-n, LN2_HI, x))   (LN2_HI = 355/512: n * LN2_HI exact)
  p  = degree-7 Taylor polynomial of e^r, coefficients RN_fp32(1/k!), in Horner
       form with one fma per degree
  e^x = (p * 2^floor(n/2)) * 2^(n - floor(n/2))
  x > 89 -> +inf, x < -104 -> +0.
Accuracy against float64 exp and the exactness of fma_f32 are pinned in the tests.
"""

import math

import numpy as np

F32 = np.float32
LOG2E_F32 = F32(1.0 / math.log(2.0))
LN2_HI_F32 = F32(355.0 / 512.0)                    # 9 significant bits
LN2_LO_F32 = F32(math.log(2.0) - 355.0 / 512.0)
EXP_COEFFS_F32 = [F32(1.0 / math.factorial(k)) for k in range(8)]   # 1/k!, k = 0..7
EXP_X_HI = F32(89.0)
EXP_X_LO = F32(-104.0)


def _pow2_f32(n):
    """2**n as float32 for integer n in [-126, 127], built from the exponent field."""
    n = np.asarray(n, dtype=np.int64)
    return ((n + 127).astype(np.uint32) << np.uint32(23)).view(np.float32)


def fma_f32(a, b, c):
    """RN_fp32(a*b + c) with one rounding, for fp32 a, b, c (finite results).

    a*b is exact in float64 (two 24-bit significands).  s = fl64(a*b + c) and
    its two-sum error e satisfy a*b + c = s + e exactly.  An fp32 midpoint is
    itself a float64, so the exact sum and s lie on the same side of every
    midpoint unless s is one: rounding s to fp32 is then already correct, and
    at a midpoint the sign of e decides (e = 0: ties to even).
    """
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    c = np.asarray(c, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        p = a.astype(np.float64) * b.astype(np.float64)
        c64 = c.astype(np.float64)
        s = p + c64
        bv = s - p
        e = (p - (s - bv)) + (c64 - bv)
        r = s.astype(np.float32)
        r64 = r.astype(np.float64)
        other = np.nextafter(r, np.where(s > r64, np.float32(np.inf), np.float32(-np.inf)).astype(np.float32))
        mid = (s != r64) & (2.0 * s == r64 + other.astype(np.float64))
        hi, lo = np.maximum(r, other), np.minimum(r, other)
        r = np.where(mid & (e > 0), hi, np.where(mid & (e < 0), lo, r))
    return np.asarray(r, dtype=np.float32)


def exp_spec(x):
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore", under="ignore", invalid="ignore"):
        xc = np.clip(x, EXP_X_LO, EXP_X_HI).astype(np.float32)
        n = np.rint((xc * LOG2E_F32).astype(np.float32)).astype(np.float32)
        r = fma_f32(-n, LN2_LO_F32, fma_f32(-n, LN2_HI_F32, xc))
        p = EXP_COEFFS_F32[7]
        for k in range(6, -1, -1):
            p = fma_f32(p, r, EXP_COEFFS_F32[k])
        ni = n.astype(np.int64)
        n1 = np.floor_divide(ni, 2)
        n2 = ni - n1
        res = ((p * _pow2_f32(n1)).astype(np.float32) * _pow2_f32(n2)).astype(np.float32)
        res = np.where(x > EXP_X_HI, np.float32(np.inf), res)
        res = np.where(x < EXP_X_LO, np.float32(0.0), res)
    return res.astype(np.float32)


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(x):
    """Round float32 to bf16 bits, nearest-even; NaN -> canonical quiet NaN."""
    x = np.asarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    rounded = ((b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16))
    out = rounded.astype(np.uint16)
    return np.where(np.isnan(x), np.uint16(0x7FC0), out).astype(np.uint16)


def sigmoid_silu(a_f32):
    one = np.float32(1.0)
    with np.errstate(over="ignore", invalid="ignore"):
        sig = (one / (one + exp_spec(-a_f32)).astype(np.float32)).astype(np.float32)
        s = (a_f32 * sig).astype(np.float32)
    return sig, s


def swiglu_h(a_bits, b_bits):
    """h bits = bf16(SiLU(a) * b) from the saved bf16 a, b."""
    a = bf16_bits_to_f32(a_bits)
    b = bf16_bits_to_f32(b_bits)
    _, s = sigmoid_silu(a)
    return f32_to_bf16_rne((s * b).astype(np.float32))


def swiglu_backward(dh_f32, a_bits, b_bits):
    """(dA bits, dB bits) from fp32 dH and the saved bf16 a, b."""
    dh = np.asarray(dh_f32, dtype=np.float32)
    a = bf16_bits_to_f32(a_bits)
    b = bf16_bits_to_f32(b_bits)
    sig, s = sigmoid_silu(a)
    one = np.float32(1.0)
    with np.errstate(over="ignore", invalid="ignore"):
        g = (one + (a * (one - sig).astype(np.float32)).astype(np.float32)).astype(np.float32)
        da = ((((dh * b).astype(np.float32)) * sig).astype(np.float32) * g).astype(np.float32)
        db = (dh * s).astype(np.float32)
    return f32_to_bf16_rne(da), f32_to_bf16_rne(db)
