"""Row-facing, column-facing and 2D32 MXFP4 producers (oracle).

"Format-Aware Fusion for Fast FP4 Pretraining":
  * §2.3 (Eq. 4-6, Fig. 4): for Y = X W^T the three contractions consume a
    row-facing Q_r or a column-facing Q_c view of each tensor.  Both keep the
    logical shape; the consumer reduces along the packed (contiguous) axis.
  * §2.2.1: activation and gradient scales are rounded upward over 32-value
    blocks; 2D32 weight tiles may take the finer scale when a_T/s_T < 0.87.
  * §2.4 (Eq. 7-8, Fig. 5): one scale per 32x32 weight tile, one encoding,
    reused in both orientations; decoded values agree between the layouts.
  * §2.5: SR only on the row-facing dY consumed by Dgrad; fixed-sign H32 only on
    the column-facing Wgrad operands.

Layouts (readings):
  row-facing  x [R][C]   -> codes [R][C/2],  scales [R][C/32]   (blocks along C)
  col-facing  x [R][C]   -> codes [C][R/2],  scales [C][R/32]   (row-facing of x^T)
  2D32        w [N][K]   -> row codes [N][K/2] + row scales [N][K/32],
                            col codes [K][N/2] + col scales [K][N/32],
                            every scale byte is its tile's byte.
Finer-scale reading: with e_up the upward exponent of the tile maximum a_T,
r = (a_T / 6) / 2^e_up lies in (0.5, 1]; the tile takes e_up - 1 iff
r < finer_ratio (exact comparison) and e_up > -127.  finer_ratio = 0 disables.

Parity unpinned: the normalisation in which the pages' 0.87 is compared (the
reading above) -- the pages give the constant but no worked example, so the
tests pin the rule's arithmetic as read (boundary cases, ratio 0 reducing to
the upward scale), not its meaning.  Everything else here is pinned.
"""

import numpy as np

from . import formats as F
from . import philox as P
from .hadamard import h32_fixed_sign

RTN, SR = 0, 1


def _encode_blocks(vals64, e, mode, u=None):
    """vals64 [..., nb, 32] exact values, e [..., nb] exponents -> nibbles [..., nb, 32]."""
    y = F.scaled_magnitude(vals64, e[..., None])
    if mode == RTN:
        code = F.rtn_code(y)
    else:
        code = F.sr_code(y, u)
    return F.sign_nibble(vals64, code)


def quantize_rows(x_bits, mode=RTN, seed=0, offset=0, row_ids=None):
    """Row-facing MXFP4 of a bf16 tensor x_bits [R][C] (uint16 bit patterns).

    RTN for activations and weights; SR (Eq. 9) for the Dgrad-facing gradient,
    with draws from Philox at (seed, offset) indexed by the element's row-major
    index r*C + c in the full tensor.  `row_ids` gives the full-tensor row
    numbers when x_bits holds only some of the rows (sampled checks).
    Returns (codes [R][C/2] uint8, scales [R][C/32] uint8).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, C = x_bits.shape
    assert C % 32 == 0
    x = F.bf16_bits_to_f64(x_bits).reshape(R, C // 32, 32)
    amax = np.abs(x).max(axis=-1)
    e = F.upward_exponent(amax)
    u = None
    if mode == SR:
        rows = np.arange(R) if row_ids is None else np.asarray(row_ids)
        idx = (rows.astype(np.uint64)[:, None] * np.uint64(C)
               + np.arange(C, dtype=np.uint64)[None, :])
        u = P.draws(seed, offset, idx).reshape(R, C // 32, 32)
    nib = _encode_blocks(x, e, mode, u).reshape(R, C)
    return F.pack_nibbles(nib), F.scale_byte(e)


def quantize_cols(x_bits, hadamard=0, sign_mask16=0):
    """Column-facing MXFP4 of x_bits [R][C]: blocks of 32 consecutive rows of one
    column, stored transposed (codes [C][R/2], scales [C][R/32]).

    With hadamard == 32 each block is first transformed by the fixed-sign H32
    in fp32; the upward scale and RTN then apply to the transformed values.
    The transformed values must be finite (every block's fp32 butterfly sums
    stay below 2^128, e.g. |x| < 2^123); otherwise the block has no upward
    scale and the call is outside the contract (ValueError).
    Rounding is always deterministic here (the Wgrad view).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, C = x_bits.shape
    assert R % 32 == 0
    xt_bits = np.ascontiguousarray(x_bits.T)                  # [C][R]
    if hadamard == 0:
        vals = F.bf16_bits_to_f64(xt_bits).reshape(C, R // 32, 32)
    elif hadamard == 32:
        xf = (xt_bits.astype(np.uint32) << 16).view(np.float32).reshape(C, R // 32, 32)
        vals = h32_fixed_sign(xf, sign_mask16).astype(np.float64)
    else:
        raise ValueError("hadamard must be 0 or 32")
    amax = np.abs(vals).max(axis=-1)
    e = F.upward_exponent(amax)
    nib = _encode_blocks(vals, e, RTN).reshape(C, R)
    return F.pack_nibbles(nib), F.scale_byte(e)


def tile_exponent_2d32(amax_tile, finer_ratio):
    """Scale exponent of a 32x32 weight tile (adaptive 2D32 rule, §2.2.1)."""
    e_up = F.upward_exponent(amax_tile)
    # r = (a_T / 6) / 2^e_up < ratio  <=>  a_T * 2^-e_up < 6 * ratio; both sides
    # of the right-hand form are exact in float64 (ratio is an fp32 value).
    lhs = np.asarray(amax_tile, dtype=np.float64) * np.ldexp(1.0, -e_up)
    rhs = F.Q_MAX * np.float64(np.float32(finer_ratio))
    finer = (lhs < rhs) & (e_up > F.E_MIN)
    return np.where(finer, e_up - 1, e_up)


def quantize_w2d32(w_bits, finer_ratio=0.87):
    """2D32 weight producer: one exponent per 32x32 tile, one encoding, two layouts.

    Returns (row_codes [N][K/2], row_scales [N][K/32],
             col_codes [K][N/2], col_scales [K][N/32]).
    Values above 6 * 2^e (possible only with the finer scale) saturate to code 7.
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    N, K = w_bits.shape
    assert N % 32 == 0 and K % 32 == 0
    w = F.bf16_bits_to_f64(w_bits)
    tiles = w.reshape(N // 32, 32, K // 32, 32)
    amax = np.abs(tiles).max(axis=(1, 3))                       # [N/32][K/32]
    e_tile = tile_exponent_2d32(amax, finer_ratio)
    e_elem = np.repeat(np.repeat(e_tile, 32, axis=0), 32, axis=1)  # [N][K]
    y = F.scaled_magnitude(w, e_elem)
    nib = F.sign_nibble(w, F.rtn_code(y))                       # [N][K], one encoding
    row_codes = F.pack_nibbles(nib)
    col_codes = F.pack_nibbles(np.ascontiguousarray(nib.T))
    row_scales = F.scale_byte(np.repeat(e_tile, 32, axis=0))    # [N][K/32]
    col_scales = F.scale_byte(np.repeat(e_tile.T, 32, axis=0))  # [K][N/32]
    return row_codes, row_scales, col_codes, col_scales
