"""Pins of the GEMM reference and of the SwiGLU arithmetic."""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import synthetic
from oracle import formats as F
from oracle import gemm as G
from oracle import quant as Q
from oracle import swiglu as S


def exact_decode(codes, scales):
    nib = F.unpack_nibbles(codes)
    R, C = nib.shape
    out = [[None] * C for _ in range(R)]
    for r in range(R):
        for c in range(C):
            n = int(nib[r, c])
            v = Fraction(float(F.E2M1_GRID[n & 7])) * Fraction(2) ** (int(scales[r, c // 32]) - 127)
            out[r][c] = -v if n & 8 else v
    return out


def test_gemm_brute_force_rationals():
    x = synthetic.tensor((5, 64), std=1.0, seed=1, outlier_rate=0.1, outlier_scale=40.0)
    w = synthetic.tensor((7, 64), std=0.02, seed=2)
    ac, as_ = Q.quantize_rows(x)
    bc, bs = Q.quantize_rows(w)
    C, E = G.gemm_ref(ac, as_, bc, bs)
    A, B = exact_decode(ac, as_), exact_decode(bc, bs)
    for m in range(5):
        for n in range(7):
            exact = sum(A[m][k] * B[n][k] for k in range(64))
            mag = sum(abs(A[m][k] * B[n][k]) for k in range(64))
            assert abs(Fraction(C[m, n]) - exact) <= Fraction(64) * Fraction(2) ** -53 * mag
            assert E[m, n] == float(mag)


def test_gemm_closed_forms():
    K = 256
    # all-code-7 operands: every product is 36 * 2^(ea + eb)
    a_codes = np.full((2, K // 2), 0x77, dtype=np.uint8)
    b_codes = np.full((3, K // 2), 0x77, dtype=np.uint8)
    a_scales = np.full((2, K // 32), 127 + 2, dtype=np.uint8)
    b_scales = np.full((3, K // 32), 127 - 5, dtype=np.uint8)
    C, _ = G.gemm_ref(a_codes, a_scales, b_codes, b_scales)
    assert np.all(C == 36.0 * K * 2.0 ** (2 - 5))
    # one-hot codes select a single product; negative sign via bit 3
    a_codes = np.zeros((1, K // 2), dtype=np.uint8)
    b_codes = np.zeros((1, K // 2), dtype=np.uint8)
    a_codes[0, 37] = 0x50              # element 75 = code 5 (3.0)
    b_codes[0, 37] = 0xE0              # element 75 = -4.0
    a_scales = np.full((1, K // 32), 127, dtype=np.uint8)
    b_scales = np.full((1, K // 32), 127, dtype=np.uint8)
    b_scales[0, 75 // 32] = 127 + 3
    C, E = G.gemm_ref(a_codes, a_scales, b_codes, b_scales)
    assert C[0, 0] == -3.0 * 4.0 * 8 and E[0, 0] == 96.0


def test_gemm_library_special_case_and_bound():
    x = synthetic.tensor((32, 128), seed=3)
    w = synthetic.tensor((64, 128), std=0.02, seed=4)
    ac, as_ = Q.quantize_rows(x)
    bc, bs = Q.quantize_rows(w)
    C, E = G.gemm_ref(ac, as_, bc, bs)
    A = torch.tensor(F.decode(ac, as_))
    B = torch.tensor(F.decode(bc, bs))
    assert np.allclose(C, (A @ B.T).numpy(), rtol=0, atol=1e-12 * E.max())
    c32 = C.astype(np.float32)
    assert G.within_bound(c32, C, E).all()
    bad = c32.copy()
    bad[1, 2] += np.float32(2e-5 * E[1, 2])
    assert not G.within_bound(bad, C, E)[1, 2]
    prev = np.full_like(c32, 3.0)
    assert G.within_bound(c32 + prev, C, E, c_prev=prev).all()


def _rn_f32_exact(q):
    """Nearest fp32 to the rational q (ties to even), by exact comparison of candidates."""
    x = np.float32(float(q))
    cands = [np.nextafter(x, np.float32(-np.inf)), x, np.nextafter(x, np.float32(np.inf))]
    best = min(abs(Fraction(float(c)) - q) for c in cands)
    near = [c for c in cands if abs(Fraction(float(c)) - q) == best]
    if len(near) > 1:
        near = [c for c in near if int(np.float32(c).view(np.uint32)) % 2 == 0]
    return np.float32(near[0])


def _midpoint_factors(down):
    """24-bit A, B with A*B = 2^47 + j (down: 2^47 - j), 1 <= j < 2^18."""
    for A in range(1 << 23, 1 << 24):
        B = -(-(1 << 47) // A) if not down else (1 << 47) // A
        j = abs(A * B - (1 << 47))
        if 1 <= j < (1 << 18) and B < (1 << 24):
            return A, B
    raise AssertionError("no factors")


def test_fma_f32_single_rounding():
    rng = np.random.default_rng(21)
    n = 3000
    a = (rng.standard_normal(n) * np.exp2(rng.integers(-20, 20, n))).astype(np.float32)
    b = (rng.standard_normal(n) * np.exp2(rng.integers(-20, 20, n))).astype(np.float32)
    c = (rng.standard_normal(n) * np.exp2(rng.integers(-40, 40, n))).astype(np.float32)
    c[: n // 3] = -(a[: n // 3] * b[: n // 3])            # cancellation: the product's rounding error
    c[n // 3: n // 2] = 0.0
    # a*b + c lands an fp64 rounding exactly on an fp32 midpoint, the exact sum just above (up)
    # or just below (down) it: a plain fp64-then-fp32 rounding goes the wrong way in both
    A, B = _midpoint_factors(False)
    a_up, b_up = np.float32(A * 2.0 ** -24), np.float32(B * 2.0 ** -47)
    A, B = _midpoint_factors(True)
    a_dn, b_dn = np.float32(A * 2.0 ** -24), np.float32(B * 2.0 ** -47)
    c_dn = np.float32(1 + 2.0 ** -23)
    a = np.concatenate([a, [a_up, a_dn, np.float32(2.0 ** -75)]]).astype(np.float32)
    b = np.concatenate([b, [b_up, b_dn, np.float32(2.0 ** -70)]]).astype(np.float32)
    c = np.concatenate([c, [np.float32(1.0), c_dn, np.float32(2.0 ** -140)]]).astype(np.float32)
    got = S.fma_f32(a, b, c)
    for i in range(len(a)):
        want = _rn_f32_exact(Fraction(float(a[i])) * Fraction(float(b[i])) + Fraction(float(c[i])))
        assert got[i].view(np.uint32) == want.view(np.uint32), (i, a[i], b[i], c[i], got[i], want)
    assert got[-3] == np.float32(1 + 2.0 ** -23)           # naive double rounding gives 1.0
    assert got[-2] == c_dn                                 # naive double rounding gives 1 + 2^-22
    assert (np.float32(1.0) + np.float32(2.0 ** -24)) == np.float32(1.0)
    # exact product error: fl(a*b) + fma(a, b, -fl(a*b)) == a*b in float64 (no underflow here)
    x = (rng.standard_normal(5000) * 8).astype(np.float32)
    y = (rng.standard_normal(5000) * 8).astype(np.float32)
    pr = (x * y).astype(np.float32)
    err = S.fma_f32(x, y, -pr)
    assert np.array_equal(pr.astype(np.float64) + err.astype(np.float64), x.astype(np.float64) * y.astype(np.float64))


def test_exp_spec_accuracy():
    x = np.linspace(-87.0, 88.0, 400_001, dtype=np.float32)
    x = np.concatenate([x, np.float32([0.0, -0.0, 1e-8, -1e-8, 0.3465, -0.3466])])
    got = S.exp_spec(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    err = np.abs(got - ref) / ulp
    assert err.max() <= 2.0, err.max()
    assert S.exp_spec(np.float32([0.0]))[0] == 1.0
    assert S.exp_spec(np.float32([100.0]))[0] == np.inf
    assert S.exp_spec(np.float32([-110.0]))[0] == 0.0
    sub = S.exp_spec(np.float32([-100.0]))[0]
    assert 0 < sub < np.finfo(np.float32).tiny


def test_exp_spec_constants_from_definitions():
    assert float(S.LN2_HI_F32) == 355 / 512
    assert abs(float(S.LN2_HI_F32) + float(S.LN2_LO_F32) - math.log(2)) <= 2 ** -37   # half an fp32 ulp of LN2_LO
    assert [float(c) for c in S.EXP_COEFFS_F32[:3]] == [1.0, 1.0, 0.5]
    assert float(S.EXP_COEFFS_F32[7]) == float(np.float32(1 / 5040))


def test_bf16_rounding_matches_library():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(200_000) * np.exp(rng.uniform(-30, 30, 200_000))).astype(np.float32)
    x = np.concatenate([x, np.float32([0.0, -0.0, np.inf, -np.inf, 3.3895314e38])])
    ours = S.f32_to_bf16_rne(x)
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, lib)


def test_silu_special_values():
    sig, s = S.sigmoid_silu(np.float32([0.0, 200.0, -200.0]))
    assert sig[0] == 0.5 and s[0] == 0.0
    assert sig[1] == 1.0 and s[1] == 200.0
    assert sig[2] == 0.0 and s[2] == 0.0


def test_swiglu_forward_close_to_float64():
    a = synthetic.tensor((64, 64), std=1.3, seed=6)
    b = synthetic.tensor((64, 64), std=1.3, seed=7)
    h = S.swiglu_h(a, b)
    av, bv = F.bf16_bits_to_f64(a), F.bf16_bits_to_f64(b)
    ref = av / (1 + np.exp(-av)) * bv
    hv = F.bf16_bits_to_f64(h)
    assert np.all(np.abs(hv - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)


def test_swiglu_backward_matches_analytic_derivative():
    a = synthetic.tensor((32, 64), std=1.3, seed=8)
    b = synthetic.tensor((32, 64), std=1.3, seed=9)
    rng = np.random.default_rng(10)
    dh = rng.standard_normal((32, 64)).astype(np.float32)
    da, db = S.swiglu_backward(dh, a, b)
    av, bv, dhv = F.bf16_bits_to_f64(a), F.bf16_bits_to_f64(b), dh.astype(np.float64)
    sig = 1 / (1 + np.exp(-av))
    # d/da [a sig(a) b] = b (sig + a sig (1 - sig)) = b sig (1 + a (1 - sig))
    ref_da = dhv * bv * sig * (1 + av * (1 - sig))
    ref_db = dhv * av * sig
    for got, ref in ((da, ref_da), (db, ref_db)):
        gv = F.bf16_bits_to_f64(got)
        assert np.all(np.abs(gv - ref) <= 2.0 ** -8 * np.abs(ref) + 2 ** -20 * np.abs(dhv))
    # finite-difference check of the derivative formula itself
    eps = 1e-6
    f = lambda t: t / (1 + np.exp(-t)) * bv
    fd = (f(av + eps) - f(av - eps)) / (2 * eps) * dhv
    assert np.allclose(fd, ref_da, rtol=1e-5, atol=1e-7)


def test_bound_covers_fp32_accumulation_in_the_subnormal_range():
    """The subnormal floor of the GEMM bound: a running fp32 sum of K exact
    products spread from far below the fp32 range up to its subnormals (each
    product reaches the fp32 grid with one rounding, at most 2^-150, and
    sums of grid values below 2^-126 are exact) stays within
    1e-5 * sum|p| + K * 2^-150 of the exact sum rounded once, while the
    relative term alone misses many such sums (the floor is needed)."""
    rng = np.random.default_rng(11)
    K = 512
    rel_only_misses = 0
    for _ in range(200):
        p = rng.integers(-36, 37, size=K) * 2.0 ** rng.integers(-180, -140, size=K).astype(np.float64)
        acc = np.float32(0.0)
        for v in p:
            acc = np.float32(acc + np.float32(v))
        exact = float(np.sum(p))                        # fp64: its error is far below 2^-150
        e = float(np.abs(p).sum())
        assert bool(G.within_bound(np.float64(acc), np.float64(np.float32(exact)), e, k=K))
        rel_only_misses += int(not G.within_bound(np.float64(acc), np.float64(np.float32(exact)), e))
    assert rel_only_misses > 0
