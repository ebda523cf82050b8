"""E2M1 values, E8M0 scales, rounding decisions, packing and decode.

Follows "Format-Aware Fusion for Fast FP4 Pretraining":
  * §2.2, Eq. 1 -- one value is x_hat = S * delta * Q_E2M1(x / (S * delta));
    for MXFP4 the outer scale S is 1 and delta is a power of two (E8M0).
    Q_E2M1 rounds to the E2M1 grid and saturates at its largest magnitude.
  * §2.2.1 (and the §1 summary of the per-operand contract) -- activation and
    gradient block scales are rounded upward.
  * §2.5, Eq. 9 -- adjacent-bin stochastic rounding: between neighbouring grid
    points q- < y < q+, round up with probability (y - q-)/(q+ - q-).
E2M1 itself (1 sign, 2 exponent, 1 fraction bit; largest magnitude 6) is stated
in the paper's notation paragraph; its eight magnitudes are
{0, 0.5, 1, 1.5, 2, 3, 4, 6}.

Readings where the pages leave a step open:
  * ties in round-to-nearest go to the even code (IEEE RNE on one fraction bit);
  * the sign bit is the sign of the input, so -0 and small negatives that round
    to zero encode as 0x8;
  * two codes per byte, element 2j in bits 0-3 and element 2j+1 in bits 4-7;
  * an all-zero block takes exponent -127 (scale byte 0); exponents are clamped
    to [-127, 127], so byte 0xFF is never produced;
  * SR rounds up iff the element's 32-bit random word u satisfies
    u < frac * 2^32, compared exactly (u < ceil(frac * 2^32)).
"""

import numpy as np

# Magnitudes of the eight E2M1 codes 0..7 (sign is bit 3).
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
Q_MAX = 6.0
E_MIN, E_MAX = -127, 127


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16) -> exact float64 values."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_to_f64(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def upward_exponent(amax):
    """Smallest integer e with amax <= Q_MAX * 2**e, clamped to [-127, 127].

    This is the encode-centric, upward-rounded E8M0 scale of §2.2.1: the block
    maximum divided by the scale never exceeds the largest E2M1 magnitude, so no
    element saturates.  amax == 0 gives -127.
    """
    amax = np.asarray(amax, dtype=np.float64)
    if not np.all(np.isfinite(amax)):
        # an infinite or NaN block maximum has no admissible exponent: such
        # blocks (non-finite inputs, or an H32 sum beyond the fp32 range) lie
        # outside the quantizer contract
        raise ValueError("block maximum is not finite: outside the quantizer contract")
    _, E = np.frexp(amax)            # amax in [2**(E-1), 2**E)
    e = E.astype(np.int64) - 4       # 6 * 2**(E-4) < 2**(E-1) <= amax: too small
    for _ in range(4):               # walk up to the smallest admissible e
        e = np.where(amax > Q_MAX * np.ldexp(1.0, e), e + 1, e)
    e = np.where(amax == 0.0, E_MIN, e)
    return np.clip(e, E_MIN, E_MAX)


def scale_byte(e):
    """E8M0 byte for exponent e (bias 127)."""
    return (np.asarray(e, dtype=np.int64) + 127).astype(np.uint8)


def scaled_magnitude(x64, e):
    """y = |x| * 2**-e, exact in float64 for every bf16/fp32 x and e in range."""
    return np.abs(x64) * np.ldexp(1.0, -np.asarray(e, dtype=np.int64))


def rtn_code(y):
    """Round-to-nearest E2M1 magnitude code for y >= 0, ties to the even code.

    Saturation is part of the definition: every y > 6 is nearest to 6 (code 7),
    so y is first limited to 6 (this also keeps every distance below exact in
    float64: y carries at most 24 significant bits).
    """
    y = np.minimum(np.asarray(y, dtype=np.float64), Q_MAX)
    dist = np.abs(y[..., None] - E2M1_GRID)
    best = dist.min(axis=-1, keepdims=True)
    tied = dist == best
    even = tied & (np.arange(8) % 2 == 0)
    has_even = even.any(axis=-1)
    return np.where(has_even, np.argmax(even, axis=-1), np.argmax(tied, axis=-1)).astype(np.uint8)


def sr_code(y, u):
    """Adjacent-bin stochastic-rounding code for 0 <= y <= 6 with draws u (uint32).

    If y is a grid value it is kept.  Otherwise q- < y < q+ are its neighbours,
    frac = (y - q-)/(q+ - q-) (exact: every quantity is dyadic), and the code of
    q+ is chosen iff u < frac * 2**32 in exact arithmetic.
    """
    y = np.asarray(y, dtype=np.float64)
    u = np.asarray(u, dtype=np.uint64)
    if np.any(y > Q_MAX):
        raise ValueError("SR is defined inside the grid range only (upward scales keep y <= 6)")
    lo = np.searchsorted(E2M1_GRID, y, side="right") - 1          # largest grid value <= y
    lo = np.clip(lo, 0, 7)
    on_grid = E2M1_GRID[lo] == y
    hi = np.clip(lo + 1, 0, 7)
    q_lo, q_hi = E2M1_GRID[lo], E2M1_GRID[hi]
    frac = np.where(on_grid, 0.0, (y - q_lo) / np.where(on_grid, 1.0, q_hi - q_lo))
    thresh = np.ceil(frac * 2.0**32).astype(np.uint64)            # exact: frac is dyadic
    up = (~on_grid) & (u < thresh)
    return np.where(up, hi, lo).astype(np.uint8)


def sign_nibble(x64, code):
    """Attach the input's sign bit (bit 3) to the magnitude code."""
    neg = np.signbit(np.asarray(x64, dtype=np.float64))
    return (code.astype(np.uint8) | (neg.astype(np.uint8) << 3)).astype(np.uint8)


def pack_nibbles(nib):
    """[..., 2n] nibbles -> [..., n] bytes: element 2j low, 2j+1 high."""
    nib = np.asarray(nib, dtype=np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def decode_nibble(nib):
    nib = np.asarray(nib, dtype=np.uint8)
    mag = E2M1_GRID[nib & 7]
    return np.where(nib & 8, -mag, mag)


def decode(codes, scales):
    """Exact float64 values of row-major MXFP4 data: codes [R][C/2], scales [R][C/32].

    value = (-1)^s * E2M1_GRID[code] * 2**(byte - 127).
    """
    vals = decode_nibble(unpack_nibbles(codes))
    R, C = vals.shape
    s = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    return (vals.reshape(R, C // 32, 32) * s[:, :, None]).reshape(R, C)
