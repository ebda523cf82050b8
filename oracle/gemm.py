"""Decode-then-contract reference for the block-scaled E2M1 GEMM.

"Format-Aware Fusion for Fast FP4 Pretraining", §2.3 (Eq. 4-6): Fprop
Y = Q_r(X) Q_r(W)^T, Dgrad dX = Q_r(dY) Q_c(W), Wgrad dW = Q_c(dY)^T Q_c(X).
With both operands stored K-major (row-facing along the reduced axis) every one
of them is C[m][n] = sum_k dec(A)[m,k] * dec(B)[n,k].

Each product of two decoded values is exact in float64 (E2M1 x E2M1 needs 4
significant bits, E8M0 factors are powers of two), so the reference sums in
float64; its own error (<= K * 2^-53 * E) is negligible against the bound.

Acceptance (per element): |C_gpu - C_ref| <= 1e-5 * E with
E[m][n] = sum_k |dec(A)[m,k] * dec(B)[n,k]|; where E == 0, C_gpu must be 0.
Below 2^-126 fp32 has a fixed spacing of 2^-149, so a sum accumulated in
fp32 there can be off by up to half that spacing per accumulated term, an
absolute amount the relative bound cannot cover; given the reduction length
K, the bound therefore gains K * 2^-150 (negligible for results in the
normal range).
"""

import numpy as np

from . import formats as F

GEMM_REL_TOL = 1e-5


def gemm_ref(a_codes, a_scales, b_codes, b_scales, rows=None):
    """Return (C_ref, E) in float64.  `rows` optionally selects rows of A."""
    A = F.decode(a_codes, a_scales)
    if rows is not None:
        A = A[np.asarray(rows)]
    B = F.decode(b_codes, b_scales)
    C = A @ B.T
    E = np.abs(A) @ np.abs(B).T
    return C, E


F32_SUBNORMAL_HALF_SPACING = 2.0 ** -150


def within_bound(c_gpu, c_ref, e_bound, c_prev=None, tol=GEMM_REL_TOL, k=None):
    """Boolean mask of elements meeting the bound.

    With accumulation the previous value is one more term of the sum, so it
    joins both the reference and the magnitude sum: |c_prev| is added to E.
    Given the reduction length k, the fp32 subnormal term k * 2^-150 is added.
    """
    c_gpu = np.asarray(c_gpu, dtype=np.float64)
    if c_prev is None:
        ref, bound = c_ref, e_bound
    else:
        prev = np.asarray(c_prev, dtype=np.float64)
        ref, bound = c_ref + prev, e_bound + np.abs(prev)
    floor = 0.0 if k is None else float(k) * F32_SUBNORMAL_HALF_SPACING
    ok = np.abs(c_gpu - ref) <= tol * bound + floor
    if c_prev is None:
        ok &= ~((e_bound == 0) & (c_gpu != 0))
    return ok
