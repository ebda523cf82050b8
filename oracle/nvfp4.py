"""CTA-local NVFP4 producers and contraction (oracle).

"Format-Aware Fusion for Fast FP4 Pretraining":
  * §2.2, Eq. 1 -- one value is x_hat = S * delta_b * Q_E2M1(x / (S * delta_b)):
    E2M1 codes, a block dequantization multiplier delta_b (for NVFP4 an E4M3
    number shared by 16 values) and an optional fp32 outer scale S.
  * §2.2.2 and the §1/§2.2 summaries -- CTA-local NVFP4 derives its outer
    factors inside the tile that owns them (a row factor for the first operand's
    rows, a column factor for the second's) instead of from a tensor-wide
    maximum; the contraction's inner sum runs on the factor-free values and
    the two factors multiply the finished sum once, after the K loop.
  * §2.4 -- the CTA-local weight producer keeps the 2D16 invariant: one E4M3
    scale per 16x16 tile, one common fp32 outer factor for both orientations,
    decoded values equal in both layouts.
  * §2.5 -- SR stays on the row-facing dY of Dgrad; the operand-wise hybrid uses
    CTA-local NVFP4 for Dgrad only (§3.3).
  * The attention page notes that an E4M3 block scale that rounds to zero drops
    its whole block and that a saturating scale encoder avoids overflow past
    E4M3's largest finite value, 448.

Readings where the pages leave a step open:
  * E4M3 is the OCP E4M3FN format: bias 7, subnormals m * 2^-9, largest
    finite value 448, no infinity; rounding to nearest, ties to even, saturating
    at 448; 0x7F (NaN) is never produced.
  * The tile that owns an outer factor is a panel of 256 consecutive rows of
    the operand (the contraction's output tile is 256 x 256), over the full K.
    The factor is S = RN32(amax / 2688), 2688 = 6 * 448, so that the panel's
    largest block scale lands at (or one E4M3 step below) 448; an all-zero
    panel takes S = 1.
  * Block scale, in single fp32 roundings: inv6 = RN32(1 / RN32(6 S)),
    delta_b = E4M3(RN32(amax_b * inv6)).
  * Element: den = RN32(delta_b * S), r = RN32(1 / den), y = RN32(|x| * r),
    code = RTN_E2M1(y) (saturating at 6), or for SR the adjacent-bin rule of
    Eq. 9 on min(y, 6) with the MX producers' Philox draws.  delta_b = 0 makes
    every code of the block a signed zero (the block vanishes).
  * Weights: one outer factor S_W = RN32(amax_W / 2688) for the whole tensor,
    computed from all 16x16 tile maxima; each tile's E4M3 scale and codes as
    above; the scale byte is replicated into both layouts' 1x16 scale rows.
  * Contraction: C[m][n] = RN32(RN32(S_A(m) S_B(n)) * acc), acc the fp32 sum of
    the exact products (delta_a q_a)(delta_b q_b); checked against the fp64
    value S_A S_B sum(...) within the GEMM bound of formats/gemm.

Parity unpinned: the readings above as readings (the owning panel, the outer
factor's formula and the order of roundings) -- the pages print no NVFP4
worked example.  The tests pin the arithmetic as read: the E4M3 grid and its
rounding against the OCP definition and torch's float8_e4m3fn conversion, the
factor's closed form, vanishing blocks, the reconstruction bound, the 2D16
orientation invariant, exact rational contractions and SR's unbiasedness.
"""

import numpy as np

from . import formats as F
from . import philox as P

E4M3_MAX = 448.0
PANEL = 256                      # rows owning one outer factor
BLOCK = 16                       # values sharing one E4M3 scale
RTN, SR = 0, 1


def _f32(x):
    return np.asarray(x, dtype=np.float32)


def e4m3_values():
    """All 127 non-negative finite OCP E4M3FN values (bytes 0x00 .. 0x7E) in byte order."""
    b = np.arange(0x7F)
    e, m = b >> 3, b & 7
    return np.where(e == 0, m * 2.0 ** -9, (1 + m / 8.0) * 2.0 ** (e - 7))


def e4m3_round(t):
    """Round non-negative fp32 t to the nearest E4M3 value, ties to the even
    mantissa, saturating at 448.  Returns (byte, value as float64)."""
    t = np.asarray(t, dtype=np.float64)
    vals = e4m3_values()
    tc = np.minimum(t, E4M3_MAX)
    idx = np.clip(np.searchsorted(vals, tc, side="right") - 1, 0, 126)   # largest value <= t
    lo = vals[idx]
    hi = vals[np.minimum(idx + 1, 126)]
    up = (tc - lo) > (hi - tc)
    tie = (tc - lo) == (hi - tc)
    up = up | (tie & (idx % 2 == 1) & (idx < 126))                        # even mantissa: even byte
    byte = np.where(up, idx + 1, idx).astype(np.uint8)
    return byte, vals[byte]


def e4m3_decode(byte):
    return e4m3_values()[np.asarray(byte, dtype=np.int64)]


def outer_factor(amax):
    """S = RN32(amax / 2688); 1 for an all-zero panel."""
    amax = _f32(amax)
    s = (amax / np.float32(6.0 * E4M3_MAX)).astype(np.float32)
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def block_scales(amax_b, S):
    """E4M3 bytes and values of blocks with maxima amax_b under outer factor S
    (broadcast): inv6 = RN32(1/RN32(6 S)), delta = E4M3(RN32(amax_b * inv6))."""
    S = _f32(S)
    inv6 = (np.float32(1.0) / (np.float32(6.0) * S).astype(np.float32)).astype(np.float32)
    t = (_f32(amax_b) * inv6).astype(np.float32)
    return e4m3_round(t)


def _encode(x64, delta, S, mode, u=None):
    """Nibbles of values x64 [..., 16] with block scale values delta [...] and
    outer factors S [...] (broadcast against the block axis)."""
    den = (_f32(delta) * _f32(S)).astype(np.float32)
    with np.errstate(divide="ignore"):
        r = np.where(den > 0, np.float32(1.0) / np.where(den > 0, den, np.float32(1.0)), np.float32(0.0))
    r = _f32(r)
    y = (np.abs(x64).astype(np.float32) * r[..., None]).astype(np.float32).astype(np.float64)
    if mode == RTN:
        code = F.rtn_code(y)
    else:
        code = F.sr_code(np.minimum(y, F.Q_MAX), u)
    return F.sign_nibble(x64, code)


def quantize_rows(x_bits, mode=RTN, seed=0, offset=0, row0=0):
    """CTA-local NVFP4 of a bf16 tensor [R][C] along C (the consumer's K):
    returns (codes [R][C/2], scales [R][C/16] E4M3 bytes, factors [ceil(R/256)]
    fp32, panel maxima [ceil(R/256)] fp32).  SR draws as MX rows: Philox at
    (seed, offset), element index (row0 + r)*C + c.  A slice of whole panels
    of a larger tensor (row0 a multiple of 256) gives that tensor's rows."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, C = x_bits.shape
    assert row0 % PANEL == 0
    assert C % BLOCK == 0
    x = F.bf16_bits_to_f64(x_bits)
    npan = (R + PANEL - 1) // PANEL
    amax_p = np.array([np.abs(x[p * PANEL:(p + 1) * PANEL]).max(initial=0.0) for p in range(npan)], dtype=np.float32)
    S = outer_factor(amax_p)
    S_row = np.repeat(S, PANEL)[:R]
    xb = x.reshape(R, C // BLOCK, BLOCK)
    amax_b = np.abs(xb).max(axis=-1)
    byte, delta = block_scales(amax_b, S_row[:, None])
    u = None
    if mode == SR:
        idx = (np.arange(R, dtype=np.uint64)[:, None] + np.uint64(row0)) * np.uint64(C) + \
            np.arange(C, dtype=np.uint64)[None, :]
        u = P.draws(seed, offset, idx).reshape(R, C // BLOCK, BLOCK)
    nib = _encode(xb, delta, S_row[:, None], mode, u).reshape(R, C)
    return F.pack_nibbles(nib), byte.astype(np.uint8), S, amax_p


def quantize_w2d16(w_bits, factor=None):
    """2D16 CTA-local weight producer for W [N][K]: one E4M3 scale per 16x16
    tile, one common outer factor.  Returns (row_codes [N][K/2], row_scales
    [N][K/16], col_codes [K][N/2], col_scales [K][N/16], factor S_W, amax_W).
    `factor` supplies S_W for a strip of whole 16-row tiles of a larger
    weight (its amax_W comes from the whole tensor); amax_W is then the
    strip's own maximum."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    N, K = w_bits.shape
    assert N % BLOCK == 0 and K % BLOCK == 0
    w = F.bf16_bits_to_f64(w_bits)
    tiles = w.reshape(N // BLOCK, BLOCK, K // BLOCK, BLOCK)
    amax_t = np.abs(tiles).max(axis=(1, 3))                              # [N/16][K/16]
    amax_w = np.float32(amax_t.max(initial=0.0))
    S = outer_factor(amax_w) if factor is None else np.float32(factor)
    byte_t, delta_t = block_scales(amax_t, S)
    d_elem = np.repeat(delta_t, BLOCK, axis=0)                           # [N][K/16]
    nib = _encode(w.reshape(N, K // BLOCK, BLOCK), d_elem, S, RTN).reshape(N, K)
    row_codes = F.pack_nibbles(nib)
    col_codes = F.pack_nibbles(np.ascontiguousarray(nib.T))
    row_scales = np.repeat(byte_t, BLOCK, axis=0).astype(np.uint8)       # [N][K/16]
    col_scales = np.repeat(byte_t.T, BLOCK, axis=0).astype(np.uint8)     # [K][N/16]
    return row_codes, row_scales, col_codes, col_scales, np.float32(S), amax_w


def decode(codes, scales):
    """Inner values delta_b * q (float64, exact) of [R][C/2] codes with [R][C/16] E4M3 scales."""
    vals = F.decode_nibble(F.unpack_nibbles(codes))
    R, C = vals.shape
    d = e4m3_decode(scales)
    return (vals.reshape(R, C // BLOCK, BLOCK) * d[:, :, None]).reshape(R, C)


def decode_full(codes, scales, factors):
    """S * delta_b * q with the per-256-row-panel factors."""
    inner = decode(codes, scales)
    S = np.repeat(np.asarray(factors, dtype=np.float64), PANEL)[:inner.shape[0]]
    return inner * S[:, None]


def gemm_ref(a_codes, a_scales, a_factors, b_codes, b_scales, b_factors, rows=None, cols=None):
    """C_ref[m][n] = S_A(m) S_B(n) sum_k dec(A)[m,k] dec(B)[n,k] in float64 and
    its magnitude sum E (same factors), as (C_ref, E).  `rows` / `cols` select
    rows of A / B by their global indices (which pick the panel factors)."""
    ia = np.arange(np.asarray(a_codes).shape[0]) if rows is None else np.asarray(rows)
    ib = np.arange(np.asarray(b_codes).shape[0]) if cols is None else np.asarray(cols)
    A = decode(np.asarray(a_codes)[ia], np.asarray(a_scales)[ia])
    B = decode(np.asarray(b_codes)[ib], np.asarray(b_scales)[ib])
    sa = np.asarray(a_factors, dtype=np.float64)[ia // PANEL]
    sb = np.asarray(b_factors, dtype=np.float64)[ib // PANEL]
    f = sa[:, None] * sb[None, :]
    return f * (A @ B.T), f * (np.abs(A) @ np.abs(B).T)
