/*
 * mxfp4.h -- C ABI of the MXFP4 operand producers and the block-scaled E2M1
 * GEMM for one linear layer's Fprop, Dgrad and Wgrad on gfx950 (MI355X).
 *
 * Method: "Format-Aware Fusion for Fast FP4 Pretraining" (arXiv 2610.00053).
 *   - §2.2 (Eq. 1): x_hat = delta * Q_E2M1(x / delta); delta is an E8M0 power
 *     of two shared by 32 values; Q_E2M1 rounds to {0,.5,1,1.5,2,3,4,6} and
 *     saturates at 6.
 *   - §2.2.1: activation/gradient scales rounded upward; 2D32 weight tiles may
 *     take the finer scale when a_T/s_T < 0.87.
 *   - §2.3 (Eq. 4-6): row-facing and column-facing views feed Fprop, Dgrad and
 *     Wgrad.
 *   - §2.4 (Eq. 7-8): one 2D32 weight encoding, both layouts, equal decode.
 *   - §2.5 (Eq. 9-10): SR only on the row-facing dY for Dgrad; paired
 *     fixed-sign H32 only on the Wgrad operands.
 *   - §3.1-§3.2: producers emit every layout, scale and saved value the next
 *     contraction needs; the gated-FFN producer emits the W2 input directly.
 *   - App. A.1: SR state is a seed plus a counter offset; explicit buffer
 *     ownership keeps asynchronous lifetimes safe.
 *
 * Data conventions (all calls):
 *   - Tensors are DEVICE pointers allocated and owned by the caller.  The
 *     library allocates and frees nothing and keeps no state except a
 *     thread-local last HIP error.
 *   - bf16 tensors are passed as their 16-bit patterns (uint16_t).
 *   - "codes" hold two E2M1 nibbles per byte: element 2j in bits 0-3, element
 *     2j+1 in bits 4-7; bit 3 of a nibble is the sign (the input's sign bit,
 *     so -0 and negatives rounding to zero encode as 0x8).
 *   - "scales" hold one E8M0 byte per 32 values: value 2^(byte-127).  Bytes
 *     lie in [0, 253]; 0xFF is never written.
 *   - Row-major everywhere; ld* are leading dimensions in ELEMENTS.
 *   - Every blocked dimension must be a multiple of 32 (the rows of
 *     fp4_quantize_rows may be any count).  Pointers must be 16-byte aligned
 *     and ld* multiples of 8 (bf16) / 4 (fp32).
 *   - Empty calls are valid: a call whose output has no elements returns
 *     FP4_OK without touching the GPU, and its pointers may be NULL.  An empty
 *     reduction writes its definition: fp4_gemm with k = 0 sets C to 0 (leaves
 *     it unchanged when accumulating); fp4_swiglu_producer with d = 0 writes
 *     a = b = h = +0 and quantizes that h as usual (the H32 view of a zero
 *     block holds the signed zeros the fixed signs produce).
 *   - Outputs must not alias inputs or each other.
 *   - Inputs must be finite; Inf/NaN inputs give unspecified codes.  With
 *     the fixed-sign H32 (hadamard = 32, and the H32 views of the fused
 *     producers) the transformed values must be finite too: every 32-token
 *     block's fp32 butterfly sums must stay below 2^128, which |x| < 2^122
 *     guarantees; a block beyond that has no upward scale and unspecified
 *     codes.
 *   - Each call validates its arguments on the host, enqueues its kernels on
 *     `stream` (NULL = the default stream) and returns without
 *     synchronising.  Results are valid once the stream has reached them.
 *   - Errors: FP4_EINVAL (null pointer or bad enum), FP4_ESHAPE (negative
 *     dimension, dimension not a multiple of 32, or ld smaller than the row
 *     length),
 *     FP4_EALIGN (alignment), FP4_EHIP (launch failed; fp4_last_hip_error()
 *     returns the hipError_t value).  Kernels report no data-dependent errors.
 *     On any error nothing has been enqueued (except after FP4_EHIP, where
 *     earlier kernels of the same call may have been).
 */
#ifndef MXFP4_H_
#define MXFP4_H_

#include <stdint.h>

#include <hip/hip_runtime_api.h>   /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP4_OK = 0,
  FP4_EINVAL = 1,
  FP4_ESHAPE = 2,
  FP4_EALIGN = 3,
  FP4_EHIP = 4
} fp4_status;

/* Rounding of row-facing producers.  An int-sized enumeration; any other
 * value is rejected with FP4_EINVAL (C++ gives it int as its fixed underlying
 * type so that such a value is representable). */
#ifdef __cplusplus
enum fp4_round : int { FP4_RTN = 0, FP4_SR = 1 };
#else
typedef enum { FP4_RTN = 0, FP4_SR = 1 } fp4_round;
#endif

/*
 * Row-facing MXFP4 (Q_r): blocks of 32 consecutive values along `cols`, the
 * reduced (K) axis of the consuming GEMM.  §2.2.1 upward E8M0 scale
 *   e = smallest integer with amax <= 6 * 2^e, clamped to [-127, 127],
 * then round-to-nearest-even E2M1 (mode FP4_RTN; activations, weights) or
 * adjacent-bin stochastic rounding (mode FP4_SR; §2.5 Eq. 9, only for the dY
 * consumed by Dgrad).  The scale never depends on the rounding mode.
 * SR draws: Philox4x32-10 keyed by (lo32(seed), hi32(seed)) at counter
 * (lo32(i>>2), hi32(i>>2), lo32(offset), hi32(offset)), word i&3, with
 * i = r*cols + c the element's logical row-major index; an element rounds up
 * iff its word u < frac * 2^32 (exact).  Callers advance `offset` per call and
 * checkpoint (seed, offset) so resumed runs never reuse draws (App. A.1).
 *   x       [rows][ldx] bf16, reads rows x cols
 *   codes   [rows][cols/2] u8,   scales [rows][cols/32] u8
 * Errors: FP4_EINVAL bad mode or null pointer; FP4_ESHAPE rows < 0, cols not
 * a non-negative multiple of 32, or ldx < cols; FP4_EALIGN x or codes not
 * 16-byte aligned, or ldx not a multiple of 8.
 */
fp4_status fp4_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                             uint8_t* codes, uint8_t* scales,
                             fp4_round mode, uint64_t seed, uint64_t offset, hipStream_t stream);

/*
 * Column-facing MXFP4 (Q_c) for the Wgrad operands: blocks of 32 consecutive
 * ROWS (tokens) of one column, stored transposed so that the token axis is
 * contiguous (the K axis of Wgrad).  Always deterministic (RTN, upward scale).
 * hadamard = 32 applies the fixed-sign H32 of §2.5 (Eq. 10) in fp32 before the
 * scale: v_j = d_(j mod 16) x_j (d_j = -1 iff bit j of sign_mask16 is set),
 * butterflies (lo,hi) <- (lo+hi, lo-hi) at strides 1,2,4,8,16 in that order,
 * then t_j = v_j * RN_fp32(2^-2.5).  Both operands of one Wgrad must use the
 * same sign_mask16.  hadamard = 0 quantizes the values directly.
 *   x        [rows][ldx] bf16
 *   codes_t  [cols][rows/2] u8,   scales_t [cols][rows/32] u8
 * Errors: FP4_EINVAL hadamard not 0 or 32, or null pointer; FP4_ESHAPE rows
 * or cols not a non-negative multiple of 32, ldx < cols, or rows > 8388480
 * (more than 65535 tiles of 128 tokens); FP4_EALIGN x or codes_t not 16-byte
 * aligned, or ldx not a multiple of 8.
 */
fp4_status fp4_quantize_cols(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                             uint8_t* codes_t, uint8_t* scales_t,
                             int hadamard, uint32_t sign_mask16, hipStream_t stream);

/*
 * Both activation-gradient views from one read (§2.3 Eq. 5-6 with §2.5: the
 * Dgrad reads dY row-facing with SR, the Wgrad reads it column-facing with
 * the fixed-sign H32).  Byte-identical to
 *   fp4_quantize_rows(x, mode, seed, offset)      -> row_codes, row_scales
 *   fp4_quantize_cols(x, hadamard, sign_mask16)   -> codes_t, scales_t
 * on the same tensor; x is read once.  rows and cols must be multiples of 32.
 *   x         [rows][ldx] bf16
 *   row_codes [rows][cols/2], row_scales [rows][cols/32]
 *   codes_t   [cols][rows/2], scales_t   [cols][rows/32]
 * Errors as the two calls (FP4_EINVAL for a bad mode or hadamard; FP4_ESHAPE
 * also for rows > 8388480, more than 65535 tiles of 128 tokens; FP4_EALIGN
 * also for row_codes).
 */
fp4_status fp4_quantize_dual(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                             uint8_t* row_codes, uint8_t* row_scales,
                             fp4_round mode, uint64_t seed, uint64_t offset,
                             uint8_t* codes_t, uint8_t* scales_t,
                             int hadamard, uint32_t sign_mask16, hipStream_t stream);

/*
 * 2D32 weight producer (§2.4, Eq. 7-8; adaptive rule of §2.2.1).  One
 * exponent per 32x32 tile: e_up from the tile maximum a_T; the finer exponent
 * e_up - 1 is taken iff (a_T/6)/2^e_up < finer_ratio (exact comparison) and
 * e_up > -127 (finer_ratio = 0.87 on the pages; 0 disables).  Values beyond
 * 6 * 2^e saturate to +-6 * 2^e.  One encoding is emitted in both layouts;
 * col codes at (k, n) hold the same nibble as row codes at (n, k) and every
 * scale byte is its tile's byte.
 *   w           [n][ldw] bf16 (W of Y = X W^T: n outputs, k inputs)
 *   row_codes   [n][k/2],  row_scales [n][k/32]   (Fprop view, K-major)
 *   col_codes   [k][n/2],  col_scales [k][n/32]   (Dgrad view, N-major)
 * Errors: FP4_EINVAL finer_ratio outside [0, 1] or null pointer; FP4_ESHAPE n
 * or k not a non-negative multiple of 32, ldw < k, n > 8388480 (more than
 * 65535 strips of 128 rows), or ldw >= 2^22 (a 128-row strip is addressed
 * with 32-bit byte offsets); FP4_EALIGN w, row_codes or col_codes not 16-byte
 * aligned, or ldw not a multiple of 8.
 */
fp4_status fp4_quantize_w2d32(const uint16_t* w, int64_t n, int64_t k, int64_t ldw,
                              uint8_t* row_codes, uint8_t* row_scales,
                              uint8_t* col_codes, uint8_t* col_scales,
                              float finer_ratio, hipStream_t stream);

/*
 * Block-scaled E2M1 GEMM, NT form (§2.3 Eq. 4-6): with both operands stored
 * K-major with 1x32 E8M0 scales along K,
 *   C[m][n] = sum_k dec(A)[m][k] * dec(B)[n][k]          (accumulate = 0)
 *   C[m][n] = C[m][n] + sum_k ...                        (accumulate = 1)
 * in fp32.  Fprop: A = Q_r(X), B = Q_r(W).  Dgrad: A = Q_r(dY), B = W col
 * layout.  Wgrad: A = Q_c(dY), B = Q_c(X).  Deterministic (no split-K).
 *   a_codes [m][k/2], a_scales [m][k/32]; b_codes [n][k/2], b_scales [n][k/32]
 *   c       [m][ldc] fp32
 * Errors: FP4_EINVAL accumulate not 0 or 1, or null pointer; FP4_ESHAPE m, n
 * or k not a non-negative multiple of 32, ldc < n, or more than 2^31 - 1
 * output tiles of 256 x 256; FP4_EALIGN an operand or c not 16-byte aligned,
 * or ldc not a multiple of 4.
 */
fp4_status fp4_gemm(int64_t m, int64_t n, int64_t k,
                    const uint8_t* a_codes, const uint8_t* a_scales,
                    const uint8_t* b_codes, const uint8_t* b_scales,
                    float* c, int64_t ldc, int accumulate, hipStream_t stream);

/*
 * Two block-scaled products summed in one fp32 accumulation:
 *   C[m][n] (+)= sum_k dec(A1)[m][k] dec(B1)[n][k] + sum_k dec(A2)[m][k] dec(B2)[n][k]
 * For the gated FFN's input gradient (§3.2 with §2.3 Eq. 5): dX = dA W1 + dB W3
 * reads the row-facing SR codes of dA and dB and the column layouts of W1 and
 * W3, i.e. one Dgrad over the concatenated K = 2f.  All eight operands have the
 * shapes of fp4_gemm's (same m, n, k).  When k is a multiple of 256 the sum
 * runs over the K steps of pair 1, then pair 2, into the same accumulators;
 * otherwise it is fp4_gemm(pair 1) followed by fp4_gemm(pair 2, accumulate).
 * Deterministic.  Errors as fp4_gemm.
 */
fp4_status fp4_gemm_pair(int64_t m, int64_t n, int64_t k,
                         const uint8_t* a1_codes, const uint8_t* a1_scales,
                         const uint8_t* b1_codes, const uint8_t* b1_scales,
                         const uint8_t* a2_codes, const uint8_t* a2_scales,
                         const uint8_t* b2_codes, const uint8_t* b2_scales,
                         float* c, int64_t ldc, int accumulate, hipStream_t stream);

/*
 * Independent block-scaled products in one launch (§2.3 Eq. 4-6: the FFN
 * backward's contractions that read the same producers' outputs, e.g. the
 * W2 Dgrad and the W2 Wgrad of one step).  Problem q computes what
 *   fp4_gemm(m, n, k, a, b, c, ldc, accumulate)            (a2_codes NULL)
 *   fp4_gemm_pair(m, n, k, a, b, a2, b2, c, ldc, accumulate) (otherwise)
 * computes, with the same bytes.  When every k is a multiple of 256 the
 * problems share one launch of the GEMM kernel, longest K per tile first, so
 * the tiles of one problem fill the CUs that another problem's last round of
 * tiles leaves idle; a problem with k = 0 or k % 256 != 0 runs as its own
 * call, after the shared launch.  No order holds between the problems: no
 * problem's c may overlap another problem's c or any operand.
 *   problems  host array of `count` descriptors, read during the call only
 *   count     0 .. FP4_GEMM_GROUP_MAX
 * Errors: FP4_EINVAL count outside 0 .. FP4_GEMM_GROUP_MAX, problems NULL
 * with count > 0, or a problem that fp4_gemm / fp4_gemm_pair would reject
 * with FP4_EINVAL (for the pair form all four of a2_codes, a2_scales,
 * b2_codes, b2_scales must be non-NULL, otherwise all four NULL); FP4_ESHAPE,
 * FP4_EALIGN as those calls, and FP4_ESHAPE when the problems together have
 * more than 2^31 - 1 tiles.  Every problem is checked before anything is
 * enqueued.
 */
#define FP4_GEMM_GROUP_MAX 4

typedef struct fp4_gemm_problem {
  int64_t m, n, k;
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  const uint8_t* a2_codes;
  const uint8_t* a2_scales;
  const uint8_t* b2_codes;
  const uint8_t* b2_scales;
  float* c;
  int64_t ldc;
  int accumulate;
} fp4_gemm_problem;

fp4_status fp4_gemm_grouped(const fp4_gemm_problem* problems, int count, hipStream_t stream);

/*
 * Fused gated-FFN producer (§3.2): a = X W1^T and b = X W3^T computed together
 * on the block-scaled MFMA, rounded to bf16 (RNE) and saved for backward; then
 *   sig = 1/(1 + exp(-a)), s = a*sig, h = bf16(s*b)
 * in fp32 with single roundings and no fused multiply-add outside the exp
 * (exp: Cody-Waite reduction with LN2 split 355/512 + remainder, degree-7
 * Taylor polynomial in Horner form, the reduction and Horner steps as fused
 * multiply-adds with one rounding each, two-step power-of-two scaling;
 * x > 89 -> inf, x < -104 -> 0; a NaN result of any step is stored as 0x7FC0).
 * h is emitted directly as MXFP4: row-facing RTN (input of W2 Fprop) and,
 * if ht_codes is non-NULL, column-facing with H32 (input of W2 Wgrad).
 *   x_codes [t][d/2], x_scales [t][d/32]       (Q_r(X))
 *   w13_codes [2f][d/2], w13_scales [2f][d/32] (rows 0..f-1: W1, f..2f-1: W3,
 *                                               2D32 row layout)
 *   a_bf16, b_bf16 [t][f]
 *   h_codes [t][f/2], h_scales [t][f/32]
 *   ht_codes [f][t/2], ht_scales [f][t/32]     (optional; both or neither)
 * Errors: FP4_EINVAL exactly one of ht_codes, ht_scales NULL, or another null
 * pointer (the operands may be NULL when d = 0); FP4_ESHAPE t, f or d not a
 * non-negative multiple of 32, or more than 2^31 - 1 tiles of 256 tokens x
 * 128 columns; FP4_EALIGN an operand, a_bf16, b_bf16, h_codes or ht_codes not
 * 16-byte aligned.
 */
fp4_status fp4_swiglu_producer(int64_t t, int64_t f, int64_t d,
                               const uint8_t* x_codes, const uint8_t* x_scales,
                               const uint8_t* w13_codes, const uint8_t* w13_scales,
                               uint16_t* a_bf16, uint16_t* b_bf16,
                               uint8_t* h_codes, uint8_t* h_scales,
                               uint8_t* ht_codes, uint8_t* ht_scales,
                               uint32_t sign_mask16, hipStream_t stream);

/*
 * SwiGLU backward, elementwise (§3.2), from the fp32 W2 Dgrad output dH and
 * the saved bf16 a, b, in fp32 with single roundings and no FMA outside the
 * exp (the same exp as fp4_swiglu_producer); NaN results are stored as 0x7FC0:
 *   dA = bf16(((dH*b)*sig) * (1 + a*(1 - sig))),   dB = bf16(dH*(a*sig))
 *   dh [t][lddh] fp32; a_bf16, b_bf16, da_bf16, db_bf16 [t][f]
 * Errors: FP4_EINVAL null pointer; FP4_ESHAPE t or f not a non-negative
 * multiple of 32, or lddh < f; FP4_EALIGN a pointer not 16-byte aligned, or
 * lddh not a multiple of 4.
 */
fp4_status fp4_swiglu_backward(int64_t t, int64_t f, const float* dh, int64_t lddh,
                               const uint16_t* a_bf16, const uint16_t* b_bf16,
                               uint16_t* da_bf16, uint16_t* db_bf16, hipStream_t stream);

/*
 * Fused SwiGLU backward producer (§3.1-§3.2: the producer completes every
 * representation its consumers read; §2.3 Eq. 5-6 and §2.5: the W1/W3 Dgrad
 * reads dA, dB row-facing with SR, the W1/W3 Wgrad reads them column-facing
 * with the fixed-sign H32).  Bit-identical to
 *   fp4_swiglu_backward(dh, a, b) -> dA, dB, then
 *   fp4_quantize_rows(dA, FP4_SR, seed, offset_a) -> da_codes, da_scales
 *   fp4_quantize_rows(dB, FP4_SR, seed, offset_b) -> db_codes, db_scales
 *   fp4_quantize_cols(dA, 32, sign_mask16)        -> dat_codes, dat_scales
 *   fp4_quantize_cols(dB, 32, sign_mask16)        -> dbt_codes, dbt_scales
 * without writing the bf16 dA, dB.  SR draws are indexed by the element's
 * row-major index in the [t][f] tensor, as in fp4_quantize_rows.
 *   dh [t][lddh] fp32; a_bf16, b_bf16 [t][f]
 *   da_codes, db_codes [t][f/2]; da_scales, db_scales [t][f/32]
 *   dat_codes, dbt_codes [f][t/2]; dat_scales, dbt_scales [f][t/32]
 * Errors: FP4_EINVAL null pointer; FP4_ESHAPE t or f negative or not a
 * multiple of 32, lddh < f, or lddh >= 2^23 (the kernel addresses a 64-row
 * chunk of dh with 32-bit offsets); FP4_EALIGN dh, a, b or a code buffer not
 * 16-byte aligned, or lddh not a multiple of 4.
 */
fp4_status fp4_swiglu_backward_producer(int64_t t, int64_t f, const float* dh, int64_t lddh,
                                        const uint16_t* a_bf16, const uint16_t* b_bf16,
                                        uint64_t seed, uint64_t offset_a, uint64_t offset_b,
                                        uint32_t sign_mask16,
                                        uint8_t* da_codes, uint8_t* da_scales,
                                        uint8_t* db_codes, uint8_t* db_scales,
                                        uint8_t* dat_codes, uint8_t* dat_scales,
                                        uint8_t* dbt_codes, uint8_t* dbt_scales, hipStream_t stream);

/*
 * W2 data gradient with the fused SwiGLU backward producer in its epilogue
 * (§3.2: the gate's derivative is applied to the W2 Dgrad output within the
 * fused backward step, which emits the operands of the W1/W3 Dgrad and Wgrad
 * contractions; §3.1).  Bit-identical to
 *   fp4_gemm(t, f, d, dy_codes, dy_scales, w2c_codes, w2c_scales) -> dH (fp32)
 *   fp4_swiglu_backward_producer(t, f, dH, f, a, b, seed, offset_a, offset_b,
 *                                sign_mask16, ...)
 * without writing or reading dH: each 256 x 256 tile of dH stays on chip.
 *   dy_codes [t][d/2], dy_scales [t][d/32]      (Q_r(dY), SR)
 *   w2c_codes [f][d/2], w2c_scales [f][d/32]    (2D32 column layout of W2 [d][f])
 *   a_bf16, b_bf16 [t][f]                       (saved gate / up outputs)
 *   da_codes, db_codes [t][f/2]; da_scales, db_scales [t][f/32]
 *   dat_codes, dbt_codes [f][t/2]; dat_scales, dbt_scales [f][t/32]
 * Errors: FP4_EINVAL null pointer; FP4_ESHAPE t, f or d not a non-negative
 * multiple of 32, d not a positive multiple of 256 (the fused main loop's K
 * step), f >= 2^22 or d >= 2^24 (32-bit offsets within a 256-row panel), or
 * more than 2^31 - 1 tiles; FP4_EALIGN an operand, a_bf16, b_bf16 or a code
 * buffer not 16-byte aligned.
 */
fp4_status fp4_gemm_swiglu_backward_producer(int64_t t, int64_t f, int64_t d,
                                             const uint8_t* dy_codes, const uint8_t* dy_scales,
                                             const uint8_t* w2c_codes, const uint8_t* w2c_scales,
                                             const uint16_t* a_bf16, const uint16_t* b_bf16,
                                             uint64_t seed, uint64_t offset_a, uint64_t offset_b,
                                             uint32_t sign_mask16,
                                             uint8_t* da_codes, uint8_t* da_scales,
                                             uint8_t* db_codes, uint8_t* db_scales,
                                             uint8_t* dat_codes, uint8_t* dat_scales,
                                             uint8_t* dbt_codes, uint8_t* dbt_scales, hipStream_t stream);

/*
 * CTA-local NVFP4 (§2.2 Eq. 1 with §2.2.2 and §2.4): a value is
 * S * delta * q with q an E2M1 code, delta an OCP E4M3FN scale byte shared by
 * 16 values along K, and S an fp32 outer factor owned by one 256-row panel
 * (the rows one 256 x 256 output tile of fp4_nv_gemm reads), or one factor
 * for a whole weight.  The pages fix the roles, not the arithmetic; this
 * library takes, in single fp32 roundings:
 *   S = amax_panel / 2688 (2688 = 6 * 448; S = 1 for an all-zero panel),
 *   inv6 = 1 / (6 S), delta = E4M3(amax_block * inv6) (nearest, ties to the
 *   even mantissa, saturating at 448; 0x7F is never written),
 *   r = 1 / (delta * S) (r = 0 when delta = 0: the block vanishes),
 *   y = |x| * r, then RTN E2M1 (saturating at 6) or, for FP4_SR, the
 *   adjacent-bin rule of §2.5 Eq. 9 on min(y, 6) with the draws of
 *   fp4_quantize_rows (same Philox counters for the same (seed, offset)).
 * "nv scales" hold one E4M3 byte per 16 values.  Every panel maximum must be 0
 * or at least 2^-100 (below that the reciprocals overflow and codes are
 * unspecified).
 */

/*
 * Row-facing CTA-local NVFP4 of an activation or gradient X [rows][cols]
 * along cols (the consuming GEMM's K).  Writes the panel maxima (fp32, one per
 * 256 rows, the last panel may be short), the factors S and the codes.
 *   x          [rows][ldx] bf16
 *   codes      [rows][cols/2] u8, scales [rows][cols/16] u8 (E4M3)
 *   factors    [ceil(rows/256)] fp32,  panel_amax [ceil(rows/256)] fp32
 * Three kernels: zero the maxima, reduce them (atomic max), quantize.
 * Errors: FP4_EINVAL bad mode or null pointer; FP4_ESHAPE rows < 0, cols not a
 * non-negative multiple of 32, ldx < cols, or rows > 2097120 (65535 groups of
 * 32 rows); FP4_EALIGN x or codes not 16-byte aligned, or ldx not a multiple
 * of 8.
 */
fp4_status fp4_nv_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                uint8_t* codes, uint8_t* scales, float* factors,
                                float* panel_amax, fp4_round mode, uint64_t seed, uint64_t offset,
                                hipStream_t stream);

/*
 * CTA-local 2D16 weight producer (§2.4 with §2.2.2): one E4M3 scale per 16x16
 * tile of W [n][k], one fp32 outer factor S_W = amax_W / 2688 for the whole
 * tensor, RTN codes, one encoding in both layouts (col codes at (j, i) hold the
 * nibble of row codes at (i, j); each 1x16 scale byte is its tile's byte).
 *   w          [n][ldw] bf16
 *   row_codes  [n][k/2],  row_scales [n][k/16]   (Fprop view)
 *   col_codes  [k][n/2],  col_scales [k][n/16]   (Dgrad view)
 *   factor     [1] fp32 (S_W),  amax_out [1] fp32 (amax_W)
 * Errors: FP4_EINVAL null pointer; FP4_ESHAPE n or k not a non-negative
 * multiple of 32, ldw < k, n > 2097120, or ldw >= 2^22 (a 128-row strip is
 * addressed with 32-bit byte offsets); FP4_EALIGN w, row_codes or col_codes
 * not 16-byte aligned, or ldw not a multiple of 8.
 */
fp4_status fp4_nv_quantize_w2d16(const uint16_t* w, int64_t n, int64_t k, int64_t ldw,
                                 uint8_t* row_codes, uint8_t* row_scales,
                                 uint8_t* col_codes, uint8_t* col_scales,
                                 float* factor, float* amax_out, hipStream_t stream);

/*
 * Contraction of two CTA-local NVFP4 operands, NT form:
 *   C[m][n] (+)= RN(S_A(m) * S_B(n)) * sum_k (delta_a q_a)(delta_b q_b)
 * with S_A(m) = a_factors[(m / 256) * a_factor_stride] and likewise for B
 * (stride 1: one factor per 256-row panel, as fp4_nv_quantize_rows writes;
 * stride 0: one factor, as fp4_nv_quantize_w2d16 writes).  Each inner value
 * delta * q is exact in f16; the sum runs on the f16 matrix cores in fp32;
 * the factor product is applied once per output in the epilogue.
 *   a_codes [m][k/2], a_scales [m][k/16]; b_codes [n][k/2], b_scales [n][k/16]
 *   c       [m][ldc] fp32
 * Errors: FP4_EINVAL accumulate not 0 or 1, negative stride or null pointer;
 * FP4_ESHAPE m or n not a non-negative multiple of 32, k not a non-negative
 * multiple of 64, ldc < n, k >= 2^24, or more than 2^31 - 1 output tiles;
 * FP4_EALIGN a code buffer or c not 16-byte aligned, or ldc not a multiple
 * of 4.  k = 0 writes C = 0 (unchanged when accumulating).
 */
fp4_status fp4_nv_gemm(int64_t m, int64_t n, int64_t k,
                       const uint8_t* a_codes, const uint8_t* a_scales,
                       const float* a_factors, int64_t a_factor_stride,
                       const uint8_t* b_codes, const uint8_t* b_scales,
                       const float* b_factors, int64_t b_factor_stride,
                       float* c, int64_t ldc, int accumulate, hipStream_t stream);

/*
 * Fixed 16-entry sign vector for H32 as a bit mask (bit j set => d_j = -1).
 * App. A.1 fixes one 16-entry sign vector, shared by both Wgrad operands and
 * repeated over the two halves of each 32-value block, but its literal
 * entries are not given; this library derives it from a seed: the low 16
 * bits of word 0 of Philox4x32-10 at counter (0,0,0,0) under key
 * (lo32(seed), hi32(seed)).  Host-only, no device work.
 */
uint32_t fp4_sign_mask_from_seed(uint64_t seed);

/* hipError_t of the last FP4_EHIP on this thread (0 if none). */
int fp4_last_hip_error(void);

/* ABI version: (major << 16) | minor. */
int fp4_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_H_ */
