// Device helpers for the MXFP4 producers on gfx950: E8M0 upward exponent,
// E2M1 round-to-nearest and stochastic rounding, Philox4x32-10, the SwiGLU
// exponential, bf16 rounding and wave-level reductions.
//
// Method: "Format-Aware Fusion for Fast FP4 Pretraining", §2.2 (Eq. 1),
// §2.2.1 (upward scales), §2.5 (Eq. 9 adjacent-bin SR), App. A.1 (seed plus
// counter offset).  Philox4x32-10 follows Salmon et al., SC'11.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

// ---------------------------------------------------------------- bf16 / fp32
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// maxNum against the canonical fp32 quiet NaN 0x7FC00000 (first operand):
// gfx950's v_max_f32 returns x for every non-NaN x and 0x7FC00000 for every
// quiet NaN x (checked over all 2^32 patterns in the kernels' IEEE mode with
// fp32 denormals kept); a signalling NaN keeps its payload, but the callers
// only pass results of arithmetic, which are never signalling.  The asm keeps
// the compiler from folding maxNum(NaN, x) to x.
__device__ __forceinline__ float canon_qnan(float x) {
  float r;
  asm("v_max_f32 %0, 0x7fc00000, %1" : "=v"(r) : "v"(x));
  return r;
}

// Two fp32 arithmetic results -> packed bf16 (x low), round to nearest even,
// NaN -> 0x7FC0.  gfx950's v_cvt_pk_bf16_f32 rounds to nearest even on every
// non-NaN fp32 pattern (checked against the integer rounding on all 2^32
// inputs); a NaN keeps its sign and upper payload bits there, so NaNs are
// first made the canonical quiet NaN, which converts to 0x7FC0 (one v_max per
// value; a compare and a select before).
__device__ __forceinline__ uint32_t bf16_pack2_rne(float x, float y) {
  const bf16x2_t v = {(__bf16)canon_qnan(x), (__bf16)canon_qnan(y)};
  return __builtin_bit_cast(uint32_t, v);
}

// fp32 -> bf16 bits, round to nearest even; NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t b = __float_as_uint(x);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------- E8M0 scale
// Upward exponent of a block maximum given as fp32 bits (finite, >= 0):
// smallest e with amax <= 6 * 2^e, clamped below at -127.  For a normal
// amax = 1.f * 2^E this is E - 2 + (f > 1.5); zero and subnormal maxima give
// -127 through the clamp.  Finite bf16/fp32 maxima never exceed e = 126.
__device__ __forceinline__ int upward_exp(uint32_t amax_bits) {
  int E = (int)(amax_bits >> 23) - 127;
  int e = E - 2 + ((amax_bits & 0x7FFFFFu) > 0x400000u ? 1 : 0);
  return e < -127 ? -127 : e;
}

// 2^-e as fp32 for e in [-127, 126] (exact, normal).
__device__ __forceinline__ float inv_pow2(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

// ---------------------------------------------------------------- E2M1 codes
// Round-to-nearest-even E2M1 uses the gfx950 converter
// v_cvt_scalef32_pk_fp4_{bf16,f32}: two values divided by a power-of-two
// scale, rounded to nearest even, saturated at 6, sign kept (so -0 and small
// negatives give 0x8), packed low element first into the selected byte.  Its
// results were checked against the rounding contract on every bf16 pattern at
// every exponent in [-127, 126] and on 4M random fp32 inputs; the GPU parity
// tests compare every producer with the CPU reference.

// 2^e as fp32 for e in [-127, 126] (2^-127 is the subnormal 0x00400000).
__device__ __forceinline__ float pow2_scale(int e) {
  return __uint_as_float(e > -127 ? (uint32_t)(e + 127) << 23 : 0x00400000u);
}

// Eight bf16 values (four packed words, element 2j in the low half of word j)
// -> eight RTN nibbles in one word (element k in bits 4k..4k+3).
__device__ __forceinline__ uint32_t rtn8_bf16(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, float scale) {
  uint32_t o = 0;
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(o, __builtin_bit_cast(bf16x2_t, w0), scale, 0);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(o, __builtin_bit_cast(bf16x2_t, w1), scale, 1);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(o, __builtin_bit_cast(bf16x2_t, w2), scale, 2);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(o, __builtin_bit_cast(bf16x2_t, w3), scale, 3);
  return o;
}

// Eight fp32 values -> eight RTN nibbles in one word.
__device__ __forceinline__ uint32_t rtn8_f32(const float* f, float scale) {
  uint32_t o = 0;
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, f[0], f[1], scale, 0);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, f[2], f[3], scale, 1);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, f[4], f[5], scale, 2);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, f[6], f[7], scale, 3);
  return o;
}

// Adjacent-bin SR code of y in [0, 6] with 32-bit draw u (software: the
// hardware SR converter uses its random bits differently from the contract).
// With q- the largest grid value <= y and q+ the next one, y rounds up iff
// u < ceil(frac * 2^32), frac = (y - q-)/(q+ - q-).  Read off the fp32 bits
// of y (biased exponent eb, fraction f):
//   y >= 1       q- has code 2 + 2(eb-127) + f[22]; the step is 2^(eb-128),
//                so frac * 2^32 = f[21:0] * 2^10 (an integer: yb << 10);
//   0.5 <= y < 1 q- = 0.5 (code 1), step 0.5: frac * 2^32 = f * 2^9 (yb << 9);
//   y < 0.5      q- = 0, step 0.5: frac * 2^32 = y * 2^33, rounded up; an
//                input so small that y is zero or subnormal still has
//                0 < frac * 2^32 < 1, threshold 1 (`nonzero`: 1 for a
//                non-zero input, else 0).
// y <= 6 always (upward scale), so q+ exists.  Branch-free after if-conversion.
__device__ __forceinline__ uint32_t e2m1_sr(float y, uint32_t u, uint32_t nonzero) {   // nonzero: 0 or 1
  const uint32_t yb = __float_as_uint(y);
  const bool big = yb >= 0x3F800000u;                    // y >= 1
  const bool small = yb < 0x3F000000u;                   // y < 0.5
  const uint32_t t_small = max((uint32_t)ceilf(y * 0x1p33f), nonzero);
  const uint32_t thr = small ? t_small : (yb << (big ? 10u : 9u));
  const uint32_t lo = small ? 0u : (big ? (yb >> 22) - 252u : 1u);
  return lo + (u < thr ? 1u : 0u);
}

// Exact SR nibbles (sign | code, element k at bits 4k) of eight bf16 values
// (four packed words) under block exponent e: e2m1_sr per element.
__device__ __forceinline__ uint32_t sr8_exact(const uint32_t* w, int e, const uint32_t* u) {
  const float inv = inv_pow2(e);
  uint32_t packed = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t bits = (w[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
    const uint32_t mag = bits & 0x7FFFu;
    const float y = bf16_bits_to_f32(mag) * inv;         // exact (power-of-two scale)
    packed |= (e2m1_sr(y, u[k], min(mag, 1u)) | ((bits >> 12) & 8u)) << (4 * k);
  }
  return packed;
}

// Fast SR form, exact for every element whose scaled magnitude y = |x| 2^-e
// is 0 or at least 2^-16.  E2M1's magnitude code is the bit pattern of a
// float with one fraction bit, exponent bias 1 and subnormals, which is the
// pattern of fp32 with its low 22 fraction bits dropped once the value is
// moved by 2^-126: z = y 2^-126 is an fp32 subnormal for y < 1 and normal
// above, and bits(z) >> 22 is the code of y rounded toward zero.  For such y
// (8 significant bits, the lowest at 2^-23 or above) z is exact, and the
// contract's threshold ceil(frac 2^32) is the low 22 bits of bits(z) times
// 2^10, so "u < threshold" is the carry out of those 22 bits when
// floor(~u / 2^10) = (u >> 10) ^ (2^22 - 1) is added.  z comes from
// v_ldexp_f32, exact for these values (normal inputs, subnormal results
// included).  The signs come from
// the hardware RTN converter applied to the signed zeros of the sign bits (it
// keeps the sign of a zero: nibble 0 or 8).
// (x ^ y) + z in one v_xad_u32; the compiler rewrites the xor with a low-bit
// mask into a not and a shift and loses the fused form.
__device__ __forceinline__ uint32_t xad_u32(uint32_t x, uint32_t y, uint32_t z) {
  uint32_t r;
  asm("v_xad_u32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(y), "v"(z));
  return r;
}

__device__ __forceinline__ uint32_t sr8_fast(const uint32_t* w, int e, const uint32_t* u) {
  const int sh = -126 - e;
  uint32_t packed = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    // the value with its sign: ldexp keeps the sign in bit 31, and bits 25-30
    // of bits(z) stay clear for |y| <= 6, so the code field is unaffected
    const uint32_t xb = (k & 1) ? (w[k >> 1] & 0xFFFF0000u) : (w[k >> 1] << 16);
    const uint32_t zb = __float_as_uint(__builtin_amdgcn_ldexpf(__uint_as_float(xb), sh));
    const uint32_t s = xad_u32(u[k] >> 10, 0x3FFFFFu, zb);   // code in bits 22-24
    packed |= __builtin_amdgcn_ubfe(s, 22, 3) << (4 * k);
  }
  return packed | rtn8_bf16(w[0] & 0x80008000u, w[1] & 0x80008000u, w[2] & 0x80008000u, w[3] & 0x80008000u, 1.0f);
}

// True when some of the NW/2 x 2 values of a block with exponent e needs the
// exact form: a non-zero magnitude below 2^(e-16), i.e. bf16 pattern
// 1 <= mag < bits(2^(e-16)), taken as max(e + 111, 1) << 7 (exact for
// e >= -110; below that every subnormal input goes to the exact form); or a
// block exponent of 126 or more, which a finite block reaches only with a
// maximum of at least 1.5 * 2^127 and every non-finite one reaches (so that
// non-finite blocks, outside the contract, give the same bytes whichever
// kernel encodes them).  One packed 16-bit subtract and min per two values.
template <int NW>
__device__ __forceinline__ bool sr_needs_exact(const uint32_t* w, int e) {
  u16x2_t m = {0xFFFFu, 0xFFFFu};
  const u16x2_t one = {1u, 1u};
#pragma unroll
  for (int j = 0; j < NW; ++j)
    m = __builtin_elementwise_min(m, __builtin_bit_cast(u16x2_t, w[j] & 0x7FFF7FFFu) - one);   // 0 wraps to 0xFFFF
  const uint32_t lim = (uint32_t)max(e + 111, 1) << 7;
  return (min((uint32_t)m[0], (uint32_t)m[1]) < lim - 1u) || e >= 126;
}

// SR nibbles of NW/4 groups of eight bf16 values (NW packed words) sharing one
// block exponent: the fast form unless some lane of the wave holds a value
// that needs the exact one (one wave-uniform branch).  draws(q, u) fills the
// eight SR words of group q; it is called inside the branch, so that the
// words of one group at a time are live.
template <int NW, typename Draws>
__device__ __forceinline__ void sr_encode(const uint32_t* w, int e, Draws&& draws, uint32_t* packed) {
  static_assert(NW % 4 == 0, "groups of eight values");
  if (__builtin_amdgcn_ballot_w64(sr_needs_exact<NW>(w, e)) == 0) {
#pragma unroll
    for (int q = 0; q < NW / 4; ++q) {
      uint32_t u[8];
      draws(q, u);
      packed[q] = sr8_fast(w + 4 * q, e, u);
    }
  } else {
#pragma unroll
    for (int q = 0; q < NW / 4; ++q) {
      uint32_t u[8];
      draws(q, u);
      packed[q] = sr8_exact(w + 4 * q, e, u);
    }
  }
}

// ---------------------------------------------------------------- H32
// Fixed-sign 32-point Hadamard of one block (signs already applied): fp32
// butterflies (lo, hi) <- (lo + hi, lo - hi) with strides 1, 2, 4, 8, 16, then
// times RN_fp32(2^-2.5); output in natural (Sylvester) order.
__device__ __forceinline__ void h32_fp32(float (&f)[32]) {
#pragma unroll
  for (int s = 1; s < 32; s <<= 1) {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if ((j & s) == 0) {
        const float lo = f[j], hi = f[j + s];
        f[j] = __fadd_rn(lo, hi);
        f[j + s] = __fsub_rn(lo, hi);
      }
    }
  }
  const float c = 0x1.6a09e6p-3f;                        // RN_fp32(2^-2.5)
#pragma unroll
  for (int j = 0; j < 32; ++j) f[j] = __fmul_rn(f[j], c);
}

// Fixed-sign H32 inputs of one column of a pair: word k holds token k of two
// columns (low and high bf16).  Value k of column c as fp32 with the sign
// d_(k mod 16) applied, one instruction per value: the low half by a shift
// and an add of the sign bit (adding bit 31 flips it), the high half by one
// and-xor.  sign_mask16 = 0 unpacks without signs.
__device__ __forceinline__ void h32_column(const uint32_t (&v)[32], int c, uint32_t sign_mask16, float (&f)[32]) {
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const uint32_t s = ((sign_mask16 >> (k & 15)) & 1u) << 31;
    f[k] = __uint_as_float(c ? ((v[k] & 0xFFFF0000u) ^ s) : ((v[k] << 16) + s));
  }
}

// RTN MXFP4 of one 32-value fp32 block: upward scale of its maximum, codes.
__device__ __forceinline__ uint4 encode32_rtn(const float (&f)[32], int& e_out) {
  float am = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) am = fmaxf(am, fabsf(f[j]));
  const int e = upward_exp(__float_as_uint(am));
  const float sc = pow2_scale(e);
  e_out = e;
  return make_uint4(rtn8_f32(f, sc), rtn8_f32(f + 8, sc), rtn8_f32(f + 16, sc), rtn8_f32(f + 24, sc));
}

// Largest 15-bit magnitude pattern among eight bf16 values (four words).
__device__ __forceinline__ uint32_t bf16_absmax8(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  const u16x2_t a = __builtin_bit_cast(u16x2_t, w0 & 0x7FFF7FFFu), b = __builtin_bit_cast(u16x2_t, w1 & 0x7FFF7FFFu);
  const u16x2_t c = __builtin_bit_cast(u16x2_t, w2 & 0x7FFF7FFFu), d = __builtin_bit_cast(u16x2_t, w3 & 0x7FFF7FFFu);
  const u16x2_t m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  return max((uint32_t)m[0], (uint32_t)m[1]);
}

// ---------------------------------------------------------------- Philox
struct u32x4 { uint32_t x, y, z, w; };

__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)M0 * c.x, p1 = (uint64_t)M1 * c.z;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    // three-input XOR in one gfx950 v_bitop3_b32 (truth table 0x96: odd parity)
    u32x4 n;
    n.x = __builtin_amdgcn_bitop3_b32(hi1, c.y, k0, 0x96);
    n.y = lo1;
    n.z = __builtin_amdgcn_bitop3_b32(hi0, c.w, k1, 0x96);
    n.w = lo0;
    c = n;
    k0 += W0;
    k1 += W1;
  }
  return c;
}

// Four SR words for elements 4*blk .. 4*blk+3 of a tensor.
__device__ __forceinline__ u32x4 sr_words(uint64_t blk, uint64_t seed, uint64_t offset) {
  u32x4 c{(uint32_t)blk, (uint32_t)(blk >> 32), (uint32_t)offset, (uint32_t)(offset >> 32)};
  return philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
}

// The same for blk < 2^32 (tensors of at most 2^34 elements), with the
// counter's second word the constant 0: with a wave-uniform offset the first
// round's high product and the second round's first product then come out
// wave-uniform (scalar), one 32x32->64 multiply and one XOR less per call.
__device__ __forceinline__ u32x4 sr_words32(uint32_t blk, uint64_t seed, uint64_t offset) {
  u32x4 c{blk, 0u, (uint32_t)offset, (uint32_t)(offset >> 32)};
  return philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
}

// ---------------------------------------------------------------- exp
// Cody-Waite exponential used by the SwiGLU producer and its backward; every
// operation is one fp32 IEEE rounding, matching the oracle: the two reduction
// steps and the seven Horner steps are fused multiply-adds (v_fma_f32, one
// rounding each), everything else is plain.

__device__ __forceinline__ float exp_spec(float x) {
  const float LOG2E = 0x1.715476p+0f;                      // RN(1/ln 2)
  const float LN2_HI = 0.693359375f;                       // 355/512
  const float LN2_LO = -0x1.bd0106p-13f;                   // RN(ln 2 - 355/512)
  // inputs beyond [-104, 89] clamp to its ends, where this same arithmetic
  // already gives +inf (x = 89) and +0 (x = -104): one v_med3, no branch (a
  // branch per element splits the unrolled element loops into exec-masked
  // regions the scheduler cannot interleave).  A NaN x may come out finite;
  // every caller multiplies by the NaN argument itself, so results stay NaN.
  const float xs = __builtin_amdgcn_fmed3f(x, -104.0f, 89.0f);
  const float n = rintf(__fmul_rn(xs, LOG2E));
  // |n| <= 150, so n * LN2_HI (8 x 9 significant bits) is exact in the first step
  const float r = __builtin_fmaf(-n, LN2_LO, __builtin_fmaf(-n, LN2_HI, xs));
  float p = 0x1.a01a02p-13f;                               // RN(1/7!)
  p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);                // RN(1/6!)
  p = __builtin_fmaf(p, r, 0x1.111112p-7f);                 // RN(1/5!)
  p = __builtin_fmaf(p, r, 0x1.555556p-5f);                 // RN(1/4!)
  p = __builtin_fmaf(p, r, 0x1.555556p-3f);                 // RN(1/3!)
  p = __builtin_fmaf(p, r, 0.5f);                          // 1/2!
  p = __builtin_fmaf(p, r, 1.0f);                          // 1/1!
  p = __builtin_fmaf(p, r, 1.0f);                          // 1/0!
  // p * 2^n with one rounding: the two-step product (p * 2^floor(n/2)) *
  // 2^(n - floor(n/2)), whose first step is exact here, equals gfx950's
  // v_ldexp_f32 for every fp32 p in [0.5, 2) and n in [-160, 130] (checked on
  // the GPU; here p in [0.7, 1.42], n in [-150, 128])
  return __builtin_amdgcn_ldexpf(p, (int)n);
}

// sig = 1/(1+exp(-a)), s = a*sig
__device__ __forceinline__ void sigmoid_silu(float a, float& sig, float& s) {
  sig = __fdiv_rn(1.0f, __fadd_rn(1.0f, exp_spec(-a)));
  s = __fmul_rn(a, sig);
}

// 1/y for y in [1, 2^126]: the hardware reciprocal and one Newton step with
// FMAs give the IEEE quotient there (checked on gfx950 for every fp32 y in
// that range).  Above 2^126 the hardware reciprocal flushes the subnormal
// results, and +inf gives NaN: callers must take the division there.
constexpr float kRecipNewtonMax = 0x1p126f;
__device__ __forceinline__ float recip_newton(float y) {
  const float r = __builtin_amdgcn_rcpf(y);
  return __builtin_fmaf(__builtin_fmaf(-y, r, 1.0f), r, r);
}

// sigmoid_silu for N values at once, same results: the quotient comes from
// recip_newton unless 1 + exp(-a) exceeds 2^126 (a < -87.3) for some value of
// some lane of the wave, in which case the whole batch divides (one wave-wide
// vote per batch, no per-element branch).
template <int N>
__device__ __forceinline__ void sigmoid_silu_n(const float (&a)[N], float (&sig)[N], float (&s)[N]) {
  float y[N];
  float ymax = 1.0f;                                     // y >= 1; a NaN y drops out (either path suits it)
#pragma unroll
  for (int k = 0; k < N; ++k) {
    y[k] = __fadd_rn(1.0f, exp_spec(-a[k]));
    ymax = fmaxf(ymax, y[k]);
  }
  if (__builtin_amdgcn_ballot_w64(ymax > kRecipNewtonMax) == 0) {
#pragma unroll
    for (int k = 0; k < N; ++k) sig[k] = recip_newton(y[k]);
  } else {
#pragma unroll
    for (int k = 0; k < N; ++k) sig[k] = __fdiv_rn(1.0f, y[k]);
  }
#pragma unroll
  for (int k = 0; k < N; ++k) s[k] = __fmul_rn(a[k], sig[k]);
}

// ---------------------------------------------------------------- one-shot loads
// Inputs a kernel reads exactly once (the producers' bf16 tensors, the
// backward producer's dH, a, b) are loaded with the non-temporal hint, so that
// streaming them does not evict the freshly written codes and operands that
// the next launches read from the caches.
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_once_u4(const void* p) {
  const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
constexpr int kLoadOnce = 2;                             // buffer-load cache policy: non-temporal

// ---------------------------------------------------------------- buffer loads
// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes
// return zero, so out-of-range lanes need no branch (a branch around a load
// keeps the compiler from counting outstanding loads, and it then waits for
// all of them).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}
constexpr uint32_t kOffNone = 0x80000000u;               // beyond any resource: reads zero

// ---------------------------------------------------------------- XCD-aware block order
// The hardware deals a grid's workgroups round-robin to the 8 XCDs in linear
// order (x fastest), and each XCD has its own L2.  Two workgroups that write
// the two halves of one 128-byte line should share an L2, or the line is
// assembled from partial writes of two XCDs.  xcd_block returns the block
// (bx, by) of a logical order in which `fast` (0: x, 1: y) varies fastest and
// each XCD owns one contiguous range of it; grids whose size is not a
// multiple of 8 keep the hardware order.
__device__ __forceinline__ void xcd_block(int fast, uint32_t& bx, uint32_t& by) {
  const uint64_t gx = gridDim.x, gy = gridDim.y, num = gx * gy;
  uint64_t l = blockIdx.x + gx * blockIdx.y;
  if ((num & 7u) == 0) l = (l & 7u) * (num >> 3) + (l >> 3);
  if (fast == 0) { bx = (uint32_t)(l % gx); by = (uint32_t)(l / gx); }
  else { by = (uint32_t)(l % gy); bx = (uint32_t)(l / gy); }
}

// ---------------------------------------------------------------- reductions
// max over each group of 4 consecutive lanes (DPP quad permutes; all lanes active)
__device__ __forceinline__ uint32_t max_quad(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  return v;
}

}  // namespace mx
