"""Fixed-sign H32 preconditioning of the Wgrad operands.

"Format-Aware Fusion for Fast FP4 Pretraining", §2.5 (Eq. 10) and App. A.1:
R = H D with H the normalised block Hadamard matrix and D a diagonal of signs;
applied to both Wgrad operands it cancels, (R dY)^T (R X) = dY^T X.  H32 repeats
a fixed 16-entry sign vector over the two 16-value halves of a 32-value block and
then applies the cross-half butterfly.  It runs inside column quantization.

Reading of the arithmetic (the pages print no formula for the stage order):
  v_j = d_{j mod 16} * x_j                       (exact sign flips)
  for stride s in 1, 2, 4, 8, 16:                fp32, in this order
      (v_lo, v_hi) <- (v_lo + v_hi, v_lo - v_hi) for lo with bit s clear, hi = lo + s
  t_j = v_j * C,  C = RN_fp32(2^-2.5) = 0x3E3504F3
The result is the natural-order (Sylvester) transform
t_j ~= C * sum_i (-1)^popcount(i & j) d_i x_i.
"""

import numpy as np

H32_NORM_F32 = np.float32(2.0 ** -2.5)  # nearest fp32 to 1/sqrt(32); pinned in tests


def sign_vector32(sign_mask16):
    """d_j for j = 0..31: the 16-entry vector repeated over both halves."""
    j = np.arange(32)
    bit = (int(sign_mask16) >> (j % 16)) & 1
    return np.where(bit == 1, -1.0, 1.0).astype(np.float32)


def h32_fixed_sign(blocks, sign_mask16):
    """Transform float32 blocks [..., 32] along the last axis; returns float32."""
    v = np.asarray(blocks, dtype=np.float32) * sign_vector32(sign_mask16)
    v = v.astype(np.float32)
    for s in (1, 2, 4, 8, 16):
        lo_idx = np.array([j for j in range(32) if not (j & s)])
        hi_idx = lo_idx + s
        lo = v[..., lo_idx]
        hi = v[..., hi_idx]
        v[..., lo_idx] = lo + hi
        v[..., hi_idx] = lo - hi
    return (v * H32_NORM_F32).astype(np.float32)
