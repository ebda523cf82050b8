"""Pins of the CTA-local NVFP4 oracle (oracle/nvfp4.py) against independent
derivations: the OCP E4M3 grid and torch's float8_e4m3fn conversion, closed
forms of the outer factor and of the vanishing block, the E2M1 spacing bound on
reconstruction, the 2D16 orientation invariant, exact rational contractions and
the unbiasedness of SR."""

from fractions import Fraction

import numpy as np
import pytest
import torch

import synthetic
from oracle import formats as F
from oracle import nvfp4 as N


def test_e4m3_grid_definition():
    v = N.e4m3_values()
    assert len(v) == 127 and v[0] == 0.0
    assert v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9      # subnormals m * 2^-9
    assert v[0x08] == 2.0 ** -6 and v[0x38] == 1.0 and v[0x7E] == 448.0
    assert np.all(np.diff(v) > 0)
    # consecutive codes within a binade differ by one mantissa step
    assert v[0x39] - v[0x38] == 0.125


def test_e4m3_round_matches_torch_and_brute_force():
    rng = np.random.default_rng(1)
    v = N.e4m3_values()
    mids = (v[1:] + v[:-1]) / 2                                      # every tie
    t = np.concatenate([v, mids, rng.uniform(0, 448, 20000), np.exp(rng.uniform(-12, 6, 20000))])
    t = t[t <= 448].astype(np.float32)
    byte, val = N.e4m3_round(t)
    ref = torch.from_numpy(t).to(torch.float8_e4m3fn)
    assert np.array_equal(byte, ref.view(torch.uint8).numpy())
    assert np.array_equal(val, ref.to(torch.float64).numpy())
    # brute force: nearest grid value, ties to the even byte
    d = np.abs(t.astype(np.float64)[:, None] - v[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    even = cand & (np.arange(127) % 2 == 0)
    bf = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
    assert np.array_equal(byte, bf)
    # saturation instead of overflow
    assert N.e4m3_round(np.float32([449.0, 1e30]))[1].tolist() == [448.0, 448.0]


def test_panel_factor_puts_the_largest_block_at_448():
    x = synthetic.tensor((512, 256), std=1.0, seed=3)
    codes, scales, S, amax = N.quantize_rows(x)
    xv = F.bf16_bits_to_f64(x)
    for p in range(2):
        assert amax[p] == np.float32(np.abs(xv[256 * p:256 * (p + 1)]).max())
        assert S[p] == np.float32(amax[p] / np.float32(2688.0))
        assert N.e4m3_decode(scales[256 * p:256 * (p + 1)]).max() == 448.0


def test_vanishing_block_and_zero_panel():
    x = np.zeros((256, 32), dtype=np.uint16)
    x[0, 0] = synthetic.bf16_bits(np.array([1.0e4], dtype=np.float32))[0]
    x[5, 16:32] = synthetic.bf16_bits(np.full(16, 1.0e-6, dtype=np.float32))
    codes, scales, S, _ = N.quantize_rows(x)
    # 1e-6 * 2688 / 1e4 is below half the smallest E4M3 value 2^-9: the block's scale is 0
    assert scales[5, 1] == 0 and np.all(F.unpack_nibbles(codes)[5, 16:32] == 0)
    z = np.zeros((256, 32), dtype=np.uint16)
    codes, scales, S, amax = N.quantize_rows(z)
    assert S[0] == 1.0 and amax[0] == 0 and not codes.any() and not scales.any()


def _half_spacing(y):
    return np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0))


def test_rtn_reconstruction_within_half_an_e2m1_step():
    x = synthetic.tensor((256, 512), std=1.0, seed=4, outlier_rate=0.01, outlier_scale=30.0)
    codes, scales, S, _ = N.quantize_rows(x)
    xv = F.bf16_bits_to_f64(x)
    inner = N.decode(codes, scales)
    d = N.e4m3_decode(scales).repeat(16, axis=1)
    unit = S[0] * d                                                 # S * delta per element
    y = np.abs(xv) / np.where(unit > 0, unit, 1)
    ok = unit > 0
    err = np.abs(xv - S[0] * inner)
    bound = unit * (_half_spacing(np.minimum(y, 6.0)) + np.maximum(y - 6.0, 0.0)) * (1 + 2.0 ** -20)
    assert np.all(err[ok] <= bound[ok])
    assert np.array_equal(np.signbit(inner[xv != 0]), np.signbit(xv[xv != 0]))


def test_w2d16_orientation_invariant_and_common_factor():
    w = synthetic.tensor((96, 160), std=0.02, seed=5)
    rc, rs, cc, cs, S, amax = N.quantize_w2d16(w)
    assert S == np.float32(amax / np.float32(2688.0))
    assert amax == np.float32(np.abs(F.bf16_bits_to_f64(w)).max())
    assert np.array_equal(N.decode(rc, rs), N.decode(cc, cs).T)
    t = rs.reshape(96 // 16, 16, 160 // 16)
    assert np.all(t == t[:, :1, :])                                 # one byte per 16x16 tile
    assert np.array_equal(rs[::16], cs[::16].T)
    # a 1D along-K encoding with its own block maxima differs (2D16 shares scales)
    r1 = N.quantize_rows(w)
    assert not np.array_equal(r1[1], rs)


def test_gemm_ref_exact_rationals_and_plain_special_case():
    rng = np.random.default_rng(6)
    m, n, k = 5, 7, 32
    ac = rng.integers(0, 256, size=(m, k // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    asc = rng.integers(0, 0x7F, size=(m, k // 16), dtype=np.uint8)
    bsc = rng.integers(0, 0x7F, size=(n, k // 16), dtype=np.uint8)
    fa, fb = np.float32([0.0078125 * 3]), np.float32([5.0e-4])
    ref, e = N.gemm_ref(ac, asc, fa, bc, bsc, fb)
    grid = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
            Fraction(6)]

    def e4(bt):
        ex, mm = int(bt) >> 3, int(bt) & 7
        return Fraction(mm, 512) if ex == 0 else (1 + Fraction(mm, 8)) * Fraction(2) ** (ex - 7)

    def val(codes, scales, i, kk):
        byte = int(codes[i, kk // 2])
        nib = byte & 0xF if kk % 2 == 0 else byte >> 4
        q = grid[nib & 7] * (-1 if nib & 8 else 1)
        return q * e4(scales[i, kk // 16])

    ref1, _ = N.gemm_ref(ac, asc, np.float32([1]), bc, bsc, np.float32([1]))
    f = Fraction(float(fa[0])) * Fraction(float(fb[0]))
    for i in range(m):
        for j in range(n):
            s = sum(val(ac, asc, i, kk) * val(bc, bsc, j, kk) for kk in range(k))
            assert Fraction(ref1[i, j]) == s                        # the inner sum is exact in fp64
            assert abs(Fraction(ref[i, j]) - s * f) <= abs(s * f) * Fraction(1, 2 ** 52)   # one fp64 rounding
    # unit factors reduce to the plain decoded product
    assert np.array_equal(ref1, N.decode(ac, asc) @ N.decode(bc, bsc).T)


def test_sr_unbiased_and_bracketed():
    # one block of fixed values, many offsets: each element lands on an adjacent
    # grid point and the mean of S * delta * q approaches x
    x = synthetic.tensor((256, 16), std=1.0, seed=7)[:1]
    x = np.repeat(x, 256, axis=0)                                   # one panel: same factor everywhere
    xv = F.bf16_bits_to_f64(x[0])
    recon = []
    for off in range(40):
        codes, scales, S, _ = N.quantize_rows(x, N.SR, seed=9, offset=off)
        recon.append(S[0] * N.decode(codes, scales))
    r = np.concatenate(recon)                                       # 10240 draws per element
    codes_rtn, scales_rtn, S_rtn, _ = N.quantize_rows(x)
    unit = S_rtn[0] * N.e4m3_decode(scales_rtn[0, 0])
    sigma = unit                                                    # a draw's spread: half a spacing <= 1
    y = np.minimum(np.abs(xv) / unit, 6.0)
    assert np.all(np.abs(r.mean(axis=0) - np.sign(xv) * y * unit) <= 5 * sigma / np.sqrt(len(r)) + 1e-12)
    # every draw is one of the two grid neighbours of y (up to the rounding of 1/den)
    g = F.E2M1_GRID
    lo = g[np.clip(np.searchsorted(g, y * (1 - 2.0 ** -20), side="right") - 1, 0, 7)]
    hi = g[np.clip(np.searchsorted(g, y * (1 + 2.0 ** -20), side="left"), 0, 7)]
    q = np.abs(r / unit)
    assert np.all((q >= lo[None, :] - 1e-12) & (q <= hi[None, :] + 1e-12))


def test_sampling_hooks_equal_the_whole_computation():
    """row0, factor and rows/cols only select: slices of whole panels, strips
    of whole tiles with the tensor's factor and sampled rows/columns give the
    whole computation's values."""
    x = synthetic.tensor((768, 64), std=1.0, seed=8)
    whole = N.quantize_rows(x, N.SR, 3, 5)
    part = N.quantize_rows(x[256:512], N.SR, 3, 5, row0=256)
    assert np.array_equal(part[0], whole[0][256:512]) and np.array_equal(part[1], whole[1][256:512])
    assert part[2][0] == whole[2][1] and part[3][0] == whole[3][1]
    w = synthetic.tensor((96, 64), std=0.1, seed=9)
    rc, rs, cc, cs, S, _ = N.quantize_w2d16(w)
    src, srs, scc, scs, sS, _ = N.quantize_w2d16(w[32:64], factor=S)
    assert sS == S and np.array_equal(src, rc[32:64]) and np.array_equal(srs, rs[32:64])
    assert np.array_equal(scc, cc[:, 16:32]) and np.array_equal(scs, cs[:, 2:4])
    b = N.quantize_rows(synthetic.tensor((320, 64), std=1.0, seed=10))
    ref, e = N.gemm_ref(whole[0], whole[1], whole[2], b[0], b[1], b[2])
    rows, cols = np.array([0, 300, 767]), np.array([5, 256, 319])
    sref, se = N.gemm_ref(whole[0], whole[1], whole[2], b[0], b[1], b[2], rows=rows, cols=cols)
    assert np.array_equal(sref, ref[np.ix_(rows, cols)]) and np.array_equal(se, e[np.ix_(rows, cols)])
