"""Pins of the oracle's E2M1/E8M0 arithmetic against independent derivations.

Each test derives the expected result a different way than the oracle does:
IEEE minifloat rounding for RTN, exhaustive search for the upward exponent, an
fp32 bit-field closed form, exact rational thresholds for SR.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import philox as P


def all_finite_positive_bf16():
    bits = np.arange(0x0001, 0x7F80, dtype=np.uint16)         # +subnormals .. +max finite
    return bits, F.bf16_bits_to_f64(bits)


def ieee_e2m1_rne(y):
    """Round y >= 0 to E2M1 as an IEEE-style minifloat (1 fraction bit, emin 0,
    subnormal quantum 0.5), ties to even significand, saturating at 6.  Returns
    the rounded value (float64)."""
    y = np.asarray(y, dtype=np.float64)
    _, E = np.frexp(np.where(y > 0, y, 1.0))                  # y in [2^(E-1), 2^E)
    e = np.maximum(E - 1, 0)                                   # unbiased exponent, >= emin
    q = np.ldexp(1.0, e - 1)                                   # quantum with 1 fraction bit
    n = np.round(y / q)                                        # numpy rounds half to even
    return np.minimum(np.where(y > 0, n * q, 0.0), 6.0)


def test_grid_and_decode_table():
    nib = np.arange(16, dtype=np.uint8)
    dec = F.decode_nibble(nib)
    assert list(dec[:8]) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(-dec[8:]) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert np.signbit(dec[8])                                   # 0x8 is -0
    assert F.Q_MAX == dec.max()


def test_rtn_exhaustive_vs_ieee_minifloat():
    _, vals = all_finite_positive_bf16()
    ys = np.concatenate([np.zeros(1)] + [vals * 2.0 ** k for k in range(-3, 4)])
    ys = ys[ys <= 64.0]
    codes = F.rtn_code(ys)
    expect = ieee_e2m1_rne(ys)
    assert np.array_equal(F.E2M1_GRID[codes], expect)


@pytest.mark.parametrize("y,code", [
    (0.25, 0), (0.2500001, 1), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4),
    (3.5, 6), (5.0, 6), (5.0000001, 7), (6.0, 7), (1e30, 7), (0.0, 0)])
def test_rtn_ties_and_saturation(y, code):
    assert int(F.rtn_code(np.array([y]))[0]) == code


def test_upward_exponent_exhaustive_bf16():
    bits, a = all_finite_positive_bf16()
    e = F.upward_exponent(a)
    # exhaustive: the smallest e in [-127, 127] with a <= 6 * 2^e
    es = np.arange(-127, 128)
    ok = a[:, None] <= 6.0 * np.ldexp(1.0, es)[None, :]
    smallest = es[np.argmax(ok, axis=1)]
    assert np.array_equal(e, smallest)
    # invariant 6*2^(e-1) < a <= 6*2^e wherever the clamp is inactive
    free = e > -127
    assert np.all(a[free] > 6.0 * np.ldexp(1.0, e[free] - 1))
    assert np.all(a <= 6.0 * np.ldexp(1.0, e))


def test_upward_exponent_fp32_bitfield_closed_form():
    # For a normal fp32 a = 1.f * 2^E: e = E - 2 + (fraction bits > 0x400000).
    _, a = all_finite_positive_bf16()
    a32 = a.astype(np.float32)
    b = a32.view(np.uint32).astype(np.int64)
    E = (b >> 23) - 127
    f = b & 0x7FFFFF
    closed = np.maximum(E - 2 + (f > 0x400000), -127)
    assert np.array_equal(F.upward_exponent(a), closed)
    assert int(F.upward_exponent(np.array([0.0]))[0]) == -127
    assert F.scale_byte(np.array([-127, 0, 126])).tolist() == [0, 127, 253]


def test_upward_scale_never_saturates():
    _, a = all_finite_positive_bf16()
    e = F.upward_exponent(a)
    y = F.scaled_magnitude(a, e)
    assert y.max() <= 6.0


def test_sr_threshold_exact():
    # For off-grid y the up-probability is frac = (y - q-)/(q+ - q-); with 32-bit
    # draws the decision is u < ceil(frac * 2^32).  Check the words on both sides
    # of the threshold, computed with rationals.
    rng = np.random.default_rng(1)
    _, vals = all_finite_positive_bf16()
    ys = vals[(vals > 0) & (vals < 6)]
    ys = rng.choice(ys, 2000, replace=False)
    grid = [Fraction(g) for g in F.E2M1_GRID]
    for y in ys:
        yf = Fraction(float(y))
        lo = max(g for g in grid if g <= yf)
        if lo == yf:
            assert F.sr_code(np.array([y]), np.array([0]))[0] == F.rtn_code(np.array([y]))[0]
            continue
        hi = min(g for g in grid if g > yf)
        frac = (yf - lo) / (hi - lo)
        t = -((-frac * 2**32) // 1)                          # ceil, exact
        lo_code = grid.index(lo)
        below = F.sr_code(np.array([y, y]), np.array([t - 1, t]))
        assert below[0] == lo_code + 1 and below[1] == lo_code
        assert F.sr_code(np.array([y]), np.array([0]))[0] == lo_code + 1
        assert F.sr_code(np.array([y]), np.array([2**32 - 1]))[0] == lo_code


def test_sr_tiny_value_rounds_up_only_for_zero_word():
    y = np.array([2.0 ** -200, 2.0 ** -200])
    assert F.sr_code(y, np.array([0, 1])).tolist() == [1, 0]


def test_sr_unbiased_in_range():
    # Eq. 9: the expectation of the rounded value equals y for y in [0, 6].
    n = 100_000
    ys = [0.1, 0.3, 0.7, 1.1, 1.9, 2.6, 3.3, 4.4, 5.9]
    idx = np.arange(n, dtype=np.uint64)
    for j, y in enumerate(ys):
        u = P.draws(seed=1234, offset=j, index=idx)
        codes = F.sr_code(np.full(n, y), u)
        vals = F.E2M1_GRID[codes]
        lo = F.E2M1_GRID[F.E2M1_GRID <= y].max()
        hi = F.E2M1_GRID[F.E2M1_GRID > y].min()
        assert set(np.unique(vals)) <= {lo, hi}
        sigma = (hi - lo) / (2 * np.sqrt(n))
        assert abs(vals.mean() - y) < 5 * sigma, (y, vals.mean())


def test_packing_order_and_roundtrip():
    nib = np.array([[1, 2, 3, 4, 15, 0]], dtype=np.uint8)
    packed = F.pack_nibbles(nib)
    assert packed.tolist() == [[0x21, 0x43, 0x0F]]
    assert np.array_equal(F.unpack_nibbles(packed), nib)


def test_sign_of_zero():
    x = np.array([-0.0, -0.1, 0.0, 0.1])
    nib = F.sign_nibble(x, F.rtn_code(np.abs(x)))
    assert nib.tolist() == [8, 8, 0, 0]


def test_decode_matches_formula():
    codes = np.array([[0x7F, 0x21] * 16], dtype=np.uint8)          # 64 elements
    scales = np.array([[127, 130]], dtype=np.uint8)
    d = F.decode(codes, scales)
    assert d[0, 0] == -6.0 and d[0, 1] == 6.0 and d[0, 2] == 0.5 and d[0, 3] == 1.0
    assert d[0, 32] == -6.0 * 8 and d[0, 35] == 8.0
