"""Pins of the fixed-sign H32 transform and of the Philox generator."""

from fractions import Fraction

import numpy as np
import scipy.linalg

from oracle import hadamard as H
from oracle import philox as P


def test_norm_constant_is_nearest_fp32_to_inv_sqrt32():
    c = H.H32_NORM_F32
    assert int(np.float32(c).view(np.uint32)) == 0x3E3504F3
    # nearest: (c - ulp/2)^2 < 1/32 < (c + ulp/2)^2, exactly
    cf = Fraction(float(c))
    half_ulp = Fraction(2) ** (-3 - 24)          # c in [2^-3, 2^-2): ulp = 2^-26
    assert (cf - half_ulp) ** 2 < Fraction(1, 32) < (cf + half_ulp) ** 2


def test_h32_unsigned_is_sylvester_hadamard():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((200, 32)).astype(np.float32)
    t = H.h32_fixed_sign(x, 0).astype(np.float64)
    ref = (x.astype(np.float64) @ scipy.linalg.hadamard(32).T) * 2.0 ** -2.5
    # fp32 error bound: 5 butterfly stages + 1 multiply
    bound = 6 * 2.0 ** -24 * 2.0 ** -2.5 * np.abs(x).sum(axis=1, keepdims=True)
    assert np.all(np.abs(t - ref) <= bound)


def test_h32_signed_closed_form_and_orthogonality():
    mask = 0x3C96
    d = H.sign_vector32(mask).astype(np.float64)
    assert np.array_equal(d[:16], d[16:])
    assert all((d[j] < 0) == bool((mask >> j) & 1) for j in range(16))
    Hn = scipy.linalg.hadamard(32) * 2.0 ** -2.5
    R = Hn @ np.diag(d)
    assert np.allclose(R.T @ R, np.eye(32), atol=1e-15)
    H32 = scipy.linalg.hadamard(32).astype(np.float64)
    assert np.array_equal(H32 @ H32, 32 * np.eye(32))
    rng = np.random.default_rng(1)
    x = rng.standard_normal((100, 32)).astype(np.float32) * np.float32(100)
    t = H.h32_fixed_sign(x, mask).astype(np.float64)
    ref = x.astype(np.float64) @ R.T
    bound = 6 * 2.0 ** -24 * 2.0 ** -2.5 * np.abs(x).sum(axis=1, keepdims=True)
    assert np.all(np.abs(t - ref) <= bound)


def test_h32_pair_preserves_dot_product():
    # Eq. 10: (R dy)^T (R x) = dy^T x before quantization.
    rng = np.random.default_rng(2)
    mask = P.sign_mask_from_seed(0)
    dy = (rng.standard_normal((64, 32)) * 1e-3).astype(np.float32)
    x = rng.standard_normal((64, 32)).astype(np.float32)
    x[3, 4] = 50.0
    tdy = H.h32_fixed_sign(dy, mask).astype(np.float64)
    tx = H.h32_fixed_sign(x, mask).astype(np.float64)
    got = (tdy * tx).sum(axis=1)
    want = (dy.astype(np.float64) * x.astype(np.float64)).sum(axis=1)
    mag = np.sqrt((dy.astype(np.float64) ** 2).sum(1) * (x.astype(np.float64) ** 2).sum(1))
    assert np.all(np.abs(got - want) <= 64 * 2.0 ** -24 * 6 * mag)
    # transforming only one side changes the product
    only = (tdy * x.astype(np.float64)).sum(axis=1)
    assert np.max(np.abs(only - want) / mag) > 1e-2


def test_philox_round_is_a_bijection_on_small_domain():
    # Philox is a permutation of the counter space for a fixed key: distinct
    # counters give distinct outputs.
    n = 1 << 16
    c = np.arange(n, dtype=np.uint64)
    o = P.philox4x32_10(c, 0, 0, 0, 123, 456)
    key = (o[0] << np.uint64(32)) | o[1]
    assert len(np.unique(key)) == n


def test_philox_statistics():
    n = 1 << 18
    u = P.draws(seed=42, offset=0, index=np.arange(n, dtype=np.uint64)).astype(np.uint32)
    # bit balance per bit position
    bits = ((u[:, None] >> np.arange(32, dtype=np.uint32)) & 1).mean(axis=0)
    assert np.all(np.abs(bits - 0.5) < 5 * 0.5 / np.sqrt(n))
    # byte chi-square (255 dof): mean 255, sd ~22.6
    bytes_ = u.view(np.uint8)
    hist = np.bincount(bytes_, minlength=256)
    expct = bytes_.size / 256
    chi2 = ((hist - expct) ** 2 / expct).sum()
    assert 255 - 6 * 22.6 < chi2 < 255 + 6 * 22.6
    # successive draws uncorrelated
    uf = u.astype(np.float64)
    r = np.corrcoef(uf[:-1], uf[1:])[0, 1]
    assert abs(r) < 5 / np.sqrt(n)


def test_philox_offsets_and_seeds_give_disjoint_streams():
    idx = np.arange(1 << 14, dtype=np.uint64)
    a = P.draws(7, 0, idx)
    b = P.draws(7, 1, idx)
    c = P.draws(8, 0, idx)
    assert len(np.intersect1d(a, b)) < 5 and len(np.intersect1d(a, c)) < 5
    # four consecutive elements share one counter and use words 0..3
    o = P.philox4x32_10(1, 0, 0, 0, 7, 0)
    assert [int(v) for v in P.draws(7, 0, np.arange(4, 8, dtype=np.uint64))] == [int(w) for w in o]


def test_philox_key_schedule_depends_on_both_key_words():
    o1 = P.philox4x32_10(5, 6, 7, 8, 1, 2)
    o2 = P.philox4x32_10(5, 6, 7, 8, 1, 3)
    o3 = P.philox4x32_10(5, 6, 7, 8, 2, 2)
    assert tuple(map(int, o1)) != tuple(map(int, o2)) != tuple(map(int, o3))


def test_sign_mask_is_deterministic_16_bit():
    m = P.sign_mask_from_seed(0)
    assert m == P.sign_mask_from_seed(0) and 0 <= m < 1 << 16
    assert P.sign_mask_from_seed(1) != m
