// CTA-local NVFP4 producers and their contraction on gfx950
// ("Format-Aware Fusion for Fast FP4 Pretraining": §2.2 Eq. 1, §2.2.2, §2.4).
//
// A value is S * delta_b * q: q an E2M1 code, delta_b an OCP E4M3 scale shared
// by 16 values along the reduced axis, S an fp32 outer factor owned by the
// 256-row panel the contraction's output tile covers (activations and
// gradients), or one factor for a whole 2D16 weight (one E4M3 scale per 16x16
// tile, both layouts).  Every step is a single fp32 rounding, in this order:
//   S = RN(amax_panel / 2688) (1 for an all-zero panel),
//   inv6 = RN(1 / RN(6 S)), delta_b = E4M3_RNE_sat(RN(amax_b * inv6)),
//   den = RN(delta_b * S), r = RN(1 / den) (0 when den = 0),
//   y = RN(|x| * r), code = RTN_E2M1(y) or, for SR, Eq. 9 on min(y, 6).
//
// The contraction: CDNA4's block-scaled MFMA takes only E8M0 (power-of-two)
// scales over 32 values, while an NVFP4 value carries a 16-value E4M3 scale
// with three fraction bits; delta_b * q has at most six significant bits and
// lies in [2^-10, 2688], so it is exact (and normal) in f16.  The GEMM decodes
// each K step of codes and scales into f16 in LDS and runs the f16 MFMA
// (v_mfma_f32_32x32x16_f16, the dense 16-bit rate) with fp32 accumulation; the
// epilogue multiplies by RN(S_A * S_B), one product per 256 x 256 output tile
// (the tile is one panel of each operand).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "abi_common.h"
#include "gemm_core.h"
#include "mx_device.h"

namespace mx {

constexpr int kNvPanel = 256;                 // rows owning one outer factor
constexpr float kNvDiv = 2688.0f;             // 6 * 448

inline int64_t ceil_div(int64_t v, int64_t d) { return v / d + (v % d != 0); }   // v >= 0, no overflow

// ------------------------------------------------------------------ E4M3
// Nearest OCP E4M3FN value of a non-negative finite fp32 t, ties to the even
// mantissa, saturating at 448 (byte 0x7E); returns the byte.
__device__ __forceinline__ uint32_t e4m3_rne(float t) {
  t = fminf(t, 448.0f);
  const uint32_t b = __float_as_uint(t);
  const int E = (int)(b >> 23) - 127;
  if (E < -6) {                                          // subnormal range: multiples of 2^-9
    const float q = __builtin_rintf(t * 512.0f);         // exact scaling; rint ties to even
    return (uint32_t)q;                                  // 0..8 (8 = the smallest normal, byte 0x08)
  }
  // normal: keep 3 fraction bits, round to nearest even on the dropped 20
  const uint32_t f = b & 0x7FFFFFu;
  uint32_t m = f >> 20;
  const uint32_t rest = f & 0xFFFFFu;
  uint32_t e = (uint32_t)(E + 7);
  if (rest > 0x80000u || (rest == 0x80000u && (m & 1u))) {
    if (++m == 8u) { m = 0; ++e; }
  }
  return (e << 3) | m;                                   // t <= 448: never past 0x7E
}

// Value of an E4M3 byte (bit 7 ignored): (8 + m) 2^(e - 10) for e >= 1 and
// m 2^-9 for e = 0, as one exact ldexp of the integer significand (no branch).
__device__ __forceinline__ float e4m3_value(uint32_t byte) {
  const uint32_t e = (byte >> 3) & 15u;
  const uint32_t sig = (byte & 7u) | (min(e, 1u) << 3);
  return __builtin_amdgcn_ldexpf((float)sig, (int)max(e, 1u) - 10);
}

__device__ __forceinline__ float nv_factor(float amax) {
  return amax == 0.0f ? 1.0f : __fdiv_rn(amax, kNvDiv);
}

// Block scale byte and encode multiplier r of a block with maximum amax_b.
__device__ __forceinline__ void nv_block(float amax_b, float S, float inv6, uint32_t& byte, float& r) {
  byte = e4m3_rne(__fmul_rn(amax_b, inv6));
  const float den = __fmul_rn(e4m3_value(byte), S);
  r = den > 0.0f ? __fdiv_rn(1.0f, den) : 0.0f;
}

// Eight values (four bf16 words) -> eight nibbles with multiplier r.
__device__ __forceinline__ uint32_t nv_rtn8(const uint32_t (&w)[4], float r) {
  float f[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) f[k] = __fmul_rn(bf16_bits_to_f32((w[k >> 1] >> (16 * (k & 1))) & 0xFFFFu), r);
  return rtn8_f32(f, 1.0f);
}

__device__ __forceinline__ uint32_t nv_sr8(const uint32_t (&w)[4], float r, const uint32_t (&u)[8]) {
  uint32_t packed = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t bits = (w[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
    const float y = fminf(__fmul_rn(bf16_bits_to_f32(bits & 0x7FFFu), r), 6.0f);
    packed |= (e2m1_sr(y, u[k], 0u) | ((bits >> 12) & 8u)) << (4 * k);
  }
  return packed;
}

// ------------------------------------------------------------------ panel maxima
// amax[p] (as fp32 bits, non-negative: ordered like unsigned integers) is the
// maximum |x| over rows [256p, 256p + 256) (or all rows when per_panel is 0).
// A workgroup covers 2048 columns x 32*nb rows (nb in {1, 2, 4, 8}, so its rows
// lie in one panel): per 32-row batch every lane issues its 32 16-byte loads
// before reducing them; wave maxima meet in LDS and one vector atomic max per
// workgroup goes out.
__global__ __launch_bounds__(256) void nv_fill_kernel(uint32_t* __restrict__ v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) v[i] = 0u;
}

__global__ __launch_bounds__(256) void nv_amax_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                      int64_t ldx, uint32_t* __restrict__ amax, int per_panel,
                                                      int nb) {
  __shared__ uint32_t wmax[4];
  const int64_t r0 = (int64_t)blockIdx.y * 32 * nb;
  // out-of-range lanes and rows re-read the last valid chunk or row (a
  // duplicate cannot change a maximum), so every load is unconditional
  const int64_t c8 = min((int64_t)blockIdx.x * 256 + threadIdx.x, (cols >> 3) - 1);
  uint32_t m = 0;
  for (int b = 0; b < nb; ++b) {
    const int64_t rb = r0 + 32 * b;
    uint4 v[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = load_once_u4(x + min(rb + j, rows - 1) * ldx + c8 * 8);
#pragma unroll
    for (int j = 0; j < 32; ++j) m = max(m, bf16_absmax8(v[j].x, v[j].y, v[j].z, v[j].w));
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, s));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    if (m != 0) atomicMax(amax + (per_panel ? r0 / kNvPanel : 0), m << 16);
  }
}

// ------------------------------------------------------------------ rows
// Lane: 8 consecutive values of one row (one 16-byte load); two lanes share a
// 16-value block (DPP pair max).  As the MXFP4 row producer, a workgroup takes
// rows blockIdx.y + j * gridDim.y and issues the loads of two rows before
// encoding either.
constexpr int kNvRowsPerPass = 2;

// kIdx32 (SR only): at most 2^34 elements, every Philox counter's second word 0.
template <bool kSR, bool kIdx32 = false>
__device__ __forceinline__ void nv_row_chunk(uint4 v, int64_t r, int64_t cols, int64_t c8, bool col_ok,
                                             uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                             float* __restrict__ factors, const uint32_t* __restrict__ amax,
                                             uint64_t seed, uint64_t offset) {
  const int64_t p = r / kNvPanel;
  const float S = nv_factor(__uint_as_float(amax[p]));
  const float inv6 = __fdiv_rn(1.0f, __fmul_rn(6.0f, S));
  uint32_t m = bf16_absmax8(v.x, v.y, v.z, v.w);
  m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false));   // pair: lanes 2j, 2j+1
  uint32_t byte;
  float rr;
  nv_block(bf16_bits_to_f32(m), S, inv6, byte, rr);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t packed;
  if constexpr (kSR) {
    const uint64_t blk = ((uint64_t)r * (uint64_t)cols + (uint64_t)c8 * 8u) >> 2;
    u32x4 a, b;
    if constexpr (kIdx32) {
      a = sr_words32((uint32_t)blk, seed, offset);
      b = sr_words32((uint32_t)blk + 1u, seed, offset);
    } else {
      a = sr_words(blk, seed, offset);
      b = sr_words(blk + 1u, seed, offset);
    }
    const uint32_t u[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    packed = nv_sr8(w, rr, u);
  } else {
    packed = nv_rtn8(w, rr);
  }
  if (col_ok) {
    *reinterpret_cast<uint32_t*>(codes + r * (cols >> 1) + c8 * 4) = packed;
    if ((c8 & 1) == 0) scales[r * (cols >> 4) + (c8 >> 1)] = (uint8_t)byte;
    if (c8 == 0 && (r % kNvPanel) == 0) factors[p] = S;
  }
}

template <bool kSR, bool kIdx32 = false>
__global__ __launch_bounds__(256) void nv_rows_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                      int64_t ldx, uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales, float* __restrict__ factors,
                                                      const uint32_t* __restrict__ amax, uint64_t seed,
                                                      uint64_t offset) {
  const int64_t c8 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool col_ok = c8 < (cols >> 3);
  const int64_t rstep = gridDim.y;
  for (int64_t r0 = blockIdx.y; r0 < rows; r0 += kNvRowsPerPass * rstep) {
    uint4 v[kNvRowsPerPass];
#pragma unroll
    for (int j = 0; j < kNvRowsPerPass; ++j) {
      const int64_t r = r0 + j * rstep;
      v[j] = make_uint4(0u, 0u, 0u, 0u);
      if (col_ok && r < rows) v[j] = load_once_u4(x + r * ldx + c8 * 8);
    }
#pragma unroll
    for (int j = 0; j < kNvRowsPerPass; ++j) {
      const int64_t r = r0 + j * rstep;
      if (r < rows)                                      // uniform over the workgroup
        nv_row_chunk<kSR, kIdx32>(v[j], r, cols, c8, col_ok, codes, scales, factors, amax, seed, offset);
    }
  }
}

// ------------------------------------------------------------------ 2D16 weights
// The walk of the MXFP4 2D32 producer with 16x16 tiles: a 256-lane workgroup
// walks consecutive 128x128 macro tiles along K with the next one's loads in
// flight.  Wave w holds rows 32w..32w+31; lane l loads rows 32w + 4q + l/16
// (q = 0..7), 8 values at column chunk l%16.  The lane's values lie in two
// 16x16 tiles (q < 4 and q >= 4) of tile column (l%16)/2; a tile maximum is a
// reduction over four of the lane's rows, its chunk pair (lane bit 0) and lane
// bits 4-5.  Row codes go out from registers, 64 bytes per row per wave store;
// the bf16 tile is staged in LDS and re-read by column pairs with the same
// tile multipliers, and the column codes are staged again so that four lanes
// write each column's 64 bytes.
constexpr int kNvWPitch = 68;                            // dwords per staged bf16 row (64 + 4 pad)
constexpr int kNvWCodePitch = 80;                        // bytes per staged column of codes (64 + 16 pad)

__device__ __forceinline__ void nv_w_load(__amdgpu_buffer_rsrc_t rs, int64_t N, int64_t K, int64_t ldw, int64_t n0,
                                          int64_t k0, uint32_t (&v)[32]) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int64_t col = k0 + (l & 15) * 8;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int row = 32 * w + 4 * q + (l >> 4);
    const bool ok = n0 + row < N && col < K;
    const v4i d = __builtin_bit_cast(
        v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, ok ? (uint32_t)(row * ldw + col) * 2u : kOffNone, 0, kLoadOnce));
    v[4 * q] = d[0]; v[4 * q + 1] = d[1]; v[4 * q + 2] = d[2]; v[4 * q + 3] = d[3];
  }
}

__device__ __forceinline__ void nv_w_tile(const uint32_t (&v)[32], int64_t N, int64_t K, int64_t n0, int64_t k0,
                                          float S, float inv6, uint8_t* __restrict__ row_codes,
                                          uint8_t* __restrict__ row_scales, uint8_t* __restrict__ col_codes,
                                          uint8_t* __restrict__ col_scales, uint32_t* tile, uint8_t* ccodes,
                                          uint32_t (*tbyte)[2][8], float (*tr)[2][8]) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int tc = (l & 15) >> 1;                          // this lane's tile column
  const int64_t col = k0 + (l & 15) * 8;
  uint32_t byte[2];
  float r[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t m = 0;
#pragma unroll
    for (int q = 4 * h; q < 4 * h + 4; ++q) m = max(m, bf16_absmax8(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]));
    m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false));   // chunk pair
    m = max(m, (uint32_t)__shfl_xor((int)m, 16));
    m = max(m, (uint32_t)__shfl_xor((int)m, 32));
    nv_block(bf16_bits_to_f32(m), S, inv6, byte[h], r[h]);
    if (l < 16 && (l & 1) == 0) {
      tbyte[w][h][tc] = byte[h];
      tr[w][h][tc] = r[h];
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q)
    *reinterpret_cast<uint4*>(&tile[(32 * w + 4 * q + (l >> 4)) * kNvWPitch + (l & 15) * 4]) =
        make_uint4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  if (n0 + 32 * w < N && col < K) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int64_t row = n0 + 32 * w + 4 * q + (l >> 4);
      const uint32_t ww[4] = {v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
      *reinterpret_cast<uint32_t*>(row_codes + row * (K >> 1) + (col >> 1)) = nv_rtn8(ww, r[q >> 2]);
      if ((l & 1) == 0) row_scales[row * (K >> 4) + (col >> 4)] = (uint8_t)byte[q >> 2];
    }
  }
  __syncthreads();

  // column pass: wave w = 32-row tile-row, lane = column pair (2l, 2l+1)
  {
    const int qr = w, pcol = l, tcc = pcol >> 3;
    const float r0 = tr[qr][0][tcc], r1 = tr[qr][1][tcc];
    uint32_t d[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) d[i] = tile[(32 * qr + i) * kNvWPitch + pcol];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint32_t sel = c ? 0x07060302u : 0x05040100u;
      uint32_t pr[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) pr[j] = __builtin_amdgcn_perm(d[2 * j + 1], d[2 * j], sel);
      const uint32_t a0[4] = {pr[0], pr[1], pr[2], pr[3]}, a1[4] = {pr[4], pr[5], pr[6], pr[7]};
      const uint32_t b0[4] = {pr[8], pr[9], pr[10], pr[11]}, b1[4] = {pr[12], pr[13], pr[14], pr[15]};
      *reinterpret_cast<uint4*>(ccodes + (2 * pcol + c) * kNvWCodePitch + qr * 16) =
          make_uint4(nv_rtn8(a0, r0), nv_rtn8(a1, r0), nv_rtn8(b0, r1), nv_rtn8(b1, r1));
    }
  }
  __syncthreads();
  // column codes out: piece p = (column p/4, tile-row p%4), four lanes per column
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int p = tid + 256 * k, kc = p >> 2, qr = p & 3;
    if (k0 + kc < K && n0 + 32 * qr < N) {
      *reinterpret_cast<uint4*>(col_codes + (k0 + kc) * (N >> 1) + (n0 >> 1) + qr * 16) =
          *reinterpret_cast<const uint4*>(ccodes + kc * kNvWCodePitch + qr * 16);
      uint8_t* cs = col_scales + (k0 + kc) * (N >> 4) + (n0 >> 4) + 2 * qr;
      cs[0] = (uint8_t)tbyte[qr][0][kc >> 4];
      cs[1] = (uint8_t)tbyte[qr][1][kc >> 4];
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void nv_w2d16_kernel(const uint16_t* __restrict__ w, int64_t N, int64_t K,
                                                       int64_t ldw, uint8_t* __restrict__ row_codes,
                                                       uint8_t* __restrict__ row_scales,
                                                       uint8_t* __restrict__ col_codes,
                                                       uint8_t* __restrict__ col_scales, float* __restrict__ factor,
                                                       const uint32_t* __restrict__ amax, int per) {
  __shared__ __attribute__((aligned(16))) uint32_t tile[128 * kNvWPitch];
  __shared__ __attribute__((aligned(16))) uint8_t ccodes[128 * kNvWCodePitch];
  __shared__ uint32_t tbyte[4][2][8];
  __shared__ float tr[4][2][8];
  uint32_t bx, by;
  xcd_block(1, bx, by);
  const int64_t n0 = (int64_t)by * 128;
  const int64_t gk = (K + 127) / 128;
  int64_t kt = (int64_t)bx * per;
  const int64_t kt_end = min(gk, kt + per);
  const float S = nv_factor(__uint_as_float(amax[0]));
  if (bx == 0 && by == 0 && threadIdx.x == 0) factor[0] = S;
  if (kt >= kt_end) return;                              // uniform over the workgroup
  const float inv6 = __fdiv_rn(1.0f, __fmul_rn(6.0f, S));
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(w + n0 * ldw, (std::min<int64_t>(128, N - n0) - 1) * ldw * 2 + K * 2);
  uint32_t v0[32], v1[32];
  nv_w_load(rs, N, K, ldw, n0, kt * 128, v0);
  for (;;) {
    int64_t kn = kt + 1 < kt_end ? kt + 1 : kt;
    nv_w_load(rs, N, K, ldw, n0, kn * 128, v1);
    nv_w_tile(v0, N, K, n0, kt * 128, S, inv6, row_codes, row_scales, col_codes, col_scales, tile, ccodes, tbyte, tr);
    if (++kt >= kt_end) break;
    kn = kt + 1 < kt_end ? kt + 1 : kt;
    nv_w_load(rs, N, K, ldw, n0, kn * 128, v0);
    nv_w_tile(v1, N, K, n0, kt * 128, S, inv6, row_codes, row_scales, col_codes, col_scales, tile, ccodes, tbyte, tr);
    if (++kt >= kt_end) break;
  }
}

// ------------------------------------------------------------------ GEMM
// 256 x 256 output tile, 8 waves of 128 x 64 (as the MXFP4 fast kernel), K in
// steps of 64 values.  Per step, lane t decodes 32 values of row t/2 of each
// operand (16 code bytes + 2 E4M3 scale bytes) into f16 and writes them to
// the LDS stage (128 bytes per row, 16-byte chunks XOR-swizzled per row).
// Sub-step s of a step reads chunk 2s + lane/32 (8 f16 = k 16s + 8(lane/32) ..).
constexpr int kNvStage = 2 * 256 * 128;                // A and B rows of one step, bytes
static_assert(2 * kNvStage <= kSmemBytes, "two stages fit");

struct NvLoad {
  uint4 ca, cb;                                        // 32 E2M1 codes of A's and B's row
  uint32_t sa, sb;                                     // their two E4M3 scale bytes
};

__device__ __forceinline__ void nv_load(NvLoad& x, __amdgpu_buffer_rsrc_t rca, __amdgpu_buffer_rsrc_t rsa,
                                        __amdgpu_buffer_rsrc_t rcb, __amdgpu_buffer_rsrc_t rsb, int64_t K, int step,
                                        int row, int half) {
  const uint32_t co = (uint32_t)(row * (K >> 1) + step * 32 + 16 * half);
  const uint32_t so = (uint32_t)(row * (K >> 4) + step * 4 + 2 * half);
  x.ca = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rca, co, 0, 0));
  x.cb = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rcb, co, 0, 0));
  x.sa = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rsa, so, 0, 0);
  x.sb = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rsb, so, 0, 0);
}

// One code word (8 values) times block scale dd -> four packed f16 words.
// gfx950's fp4 converters scale by the exponent of their fp32 scale operand
// only (an E8M0 reading: checked on every code byte and every E4M3 value), so
// the codes are converted at scale 1 and the E4M3 scale (exact in f16) is
// applied with one packed f16 multiply per two values.  q * delta has at most
// six significant bits and lies in [2^-10, 2688]: exact and normal in f16.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ uint32_t nv_dec2(f16x2_t q, f16x2_t dd) { return __builtin_bit_cast(uint32_t, q * dd); }
__device__ __forceinline__ void nv_decode8(uint32_t w, f16x2_t dd, uint32_t* o) {
  o[0] = nv_dec2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0), dd);
  o[1] = nv_dec2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1), dd);
  o[2] = nv_dec2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2), dd);
  o[3] = nv_dec2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3), dd);
}

// Chunk q (values 8q..8q+7 of this lane's 32) of the A and B rows in x,
// decoded with block scales da, db and written to the stage.
template <int Q>
__device__ __forceinline__ void nv_stage_chunk(uint8_t* stage, const NvLoad& x, f16x2_t da, f16x2_t db, int row,
                                               int half) {
  const uint32_t wa = Q == 0 ? x.ca.x : Q == 1 ? x.ca.y : Q == 2 ? x.ca.z : x.ca.w;
  const uint32_t wb = Q == 0 ? x.cb.x : Q == 1 ? x.cb.y : Q == 2 ? x.cb.z : x.cb.w;
  uint32_t a[4], b[4];
  nv_decode8(wa, da, a);
  nv_decode8(wb, db, b);
  const int ch = swz(row, 4 * half + Q);
  *reinterpret_cast<uint4*>(stage + row * 128 + ch * 16) = make_uint4(a[0], a[1], a[2], a[3]);
  *reinterpret_cast<uint4*>(stage + 256 * 128 + row * 128 + ch * 16) = make_uint4(b[0], b[1], b[2], b[3]);
}

struct NvScales {
  f16x2_t a0, a1, b0, b1;                              // E4M3 values of the lane's two A and two B blocks
};

__device__ __forceinline__ f16x2_t nv_splat(float d) {
  const _Float16 h = (_Float16)d;                      // exact: every E4M3 value is an f16 value
  return f16x2_t{h, h};
}

__device__ __forceinline__ NvScales nv_scales(const NvLoad& x) {
  return {nv_splat(e4m3_value(x.sa & 0xFFu)), nv_splat(e4m3_value(x.sa >> 8)), nv_splat(e4m3_value(x.sb & 0xFFu)),
          nv_splat(e4m3_value(x.sb >> 8))};
}

template <int Q>
__device__ __forceinline__ void nv_stage_q(uint8_t* stage, const NvLoad& x, const NvScales& d, int row, int half) {
  nv_stage_chunk<Q>(stage, x, Q < 2 ? d.a0 : d.a1, Q < 2 ? d.b0 : d.b1, row, half);
}

struct NvFrag {
  f16x8_t a[4], b[2];
};

// Fragments of sub-step ss (k 16ss .. 16ss+15) of the stage for this lane.
__device__ __forceinline__ void nv_frag(NvFrag& f, const uint8_t* stage, int ss, int wm, int wn, int r, int hl) {
  const int ch = 2 * ss + hl;
  const uint8_t* la = stage;
  const uint8_t* lb = stage + 256 * 128;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ar = wm * 128 + 32 * i + r;
    f.a[i] = *reinterpret_cast<const f16x8_t*>(la + ar * 128 + swz(ar, ch) * 16);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int br = wn * 64 + 32 * j + r;
    f.b[j] = *reinterpret_cast<const f16x8_t*>(lb + br * 128 + swz(br, ch) * 16);
  }
}

__device__ __forceinline__ void nv_mfma(v16f (&acc)[4][2], const NvFrag& f) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
}

// One K step: the MFMAs of the step held in `cur`, with the decode of the
// next step's codes (x) into `nxt` spread over the four sub-steps, so that
// each wave's conversions issue while its matrix products execute.  The
// fragments of sub-step ss+1 are read before the products of ss.
__device__ __forceinline__ void nv_step(const uint8_t* cur, uint8_t* nxt, const NvLoad& x, v16f (&acc)[4][2], int wm,
                                        int wn, int r, int hl, int row, int half) {
  NvFrag f0, f1;
  nv_frag(f0, cur, 0, wm, wn, r, hl);
  const NvScales d = nv_scales(x);
  nv_frag(f1, cur, 1, wm, wn, r, hl);
  nv_mfma(acc, f0);
  nv_stage_q<0>(nxt, x, d, row, half);
  nv_frag(f0, cur, 2, wm, wn, r, hl);
  nv_mfma(acc, f1);
  nv_stage_q<1>(nxt, x, d, row, half);
  nv_frag(f1, cur, 3, wm, wn, r, hl);
  nv_mfma(acc, f0);
  nv_stage_q<2>(nxt, x, d, row, half);
  nv_mfma(acc, f1);
  nv_stage_q<3>(nxt, x, d, row, half);
}

__global__ __launch_bounds__(512) void nv_gemm_kernel(int64_t M, int64_t N, int64_t K,
                                                      const uint8_t* __restrict__ a_codes,
                                                      const uint8_t* __restrict__ a_scales,
                                                      const float* __restrict__ a_factors, int64_t a_fstride,
                                                      const uint8_t* __restrict__ b_codes,
                                                      const uint8_t* __restrict__ b_scales,
                                                      const float* __restrict__ b_factors, int64_t b_fstride,
                                                      float* __restrict__ c, int64_t ldc, int accumulate) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kNvStage];
  uint8_t* const st0 = smem;
  uint8_t* const st1 = smem + kNvStage;
  int64_t tm, tn;
  tile_coords((M + 255) / 256, (N + 255) / 256, tm, tn);
  const int64_t m0 = tm * 256, n0 = tn * 256;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3, r = lane & 31, hl = lane >> 5;
  const int row = tid >> 1, half = tid & 1;
  const int64_t rows_a = std::min<int64_t>(256, M - m0), rows_b = std::min<int64_t>(256, N - n0);
  const __amdgpu_buffer_rsrc_t rca = buffer_rsrc(a_codes + m0 * (K >> 1), rows_a * (K >> 1));
  const __amdgpu_buffer_rsrc_t rsa = buffer_rsrc(a_scales + m0 * (K >> 4), rows_a * (K >> 4));
  const __amdgpu_buffer_rsrc_t rcb = buffer_rsrc(b_codes + n0 * (K >> 1), rows_b * (K >> 1));
  const __amdgpu_buffer_rsrc_t rsb = buffer_rsrc(b_scales + n0 * (K >> 4), rows_b * (K >> 4));
  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
  const int nk = (int)(K / 64);
  // la and lb alternate as the register copy of the next step's codes; a
  // step past the end re-reads the last one (decoded into the idle stage and
  // never read), which keeps the loop free of branches around loads
  NvLoad la, lb;
  nv_load(la, rca, rsa, rcb, rsb, K, 0, row, half);
  {
    const NvScales d = nv_scales(la);
    nv_stage_q<0>(st0, la, d, row, half);
    nv_stage_q<1>(st0, la, d, row, half);
    nv_stage_q<2>(st0, la, d, row, half);
    nv_stage_q<3>(st0, la, d, row, half);
  }
  nv_load(la, rca, rsa, rcb, rsb, K, min(1, nk - 1), row, half);
  __syncthreads();
  for (int s = 0;; s += 2) {
    nv_load(lb, rca, rsa, rcb, rsb, K, min(s + 2, nk - 1), row, half);
    nv_step(st0, st1, la, acc, wm, wn, r, hl, row, half);
    __syncthreads();
    if (s + 1 >= nk) break;
    nv_load(la, rca, rsa, rcb, rsb, K, min(s + 3, nk - 1), row, half);
    nv_step(st1, st0, lb, acc, wm, wn, r, hl, row, half);
    __syncthreads();
    if (s + 2 >= nk) break;
  }
  // epilogue: C (+)= RN(S_A S_B) * acc; lane holds row r of A sub-tile i and
  // columns 8g + 4 hl + 0..3 of B sub-tile j
  const float f = __fmul_rn(a_factors[tm * a_fstride], b_factors[tn * b_fstride]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t grow = m0 + wm * 128 + 32 * i + r;
    if (grow >= M) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t gcol = n0 + wn * 64 + 32 * j;
      if (gcol >= N) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float* p = c + grow * ldc + gcol + 8 * g + 4 * hl;
        float4 v = make_float4(__fmul_rn(f, acc[i][j][4 * g]), __fmul_rn(f, acc[i][j][4 * g + 1]),
                               __fmul_rn(f, acc[i][j][4 * g + 2]), __fmul_rn(f, acc[i][j][4 * g + 3]));
        if (accumulate) {
          const float4 pv = *reinterpret_cast<const float4*>(p);
          v.x = __fadd_rn(pv.x, v.x); v.y = __fadd_rn(pv.y, v.y); v.z = __fadd_rn(pv.z, v.z); v.w = __fadd_rn(pv.w, v.w);
        }
        *reinterpret_cast<float4*>(p) = v;
      }
    }
  }
}

}  // namespace mx

using namespace mx;

extern "C" {

// Batches of 32 rows per amax workgroup: enough workgroups to cover the chip
// (about 1024), at most one panel (8 batches) each.
static int nv_amax_batches(int64_t gx, int64_t rows) {
  int nb = 1;
  while (nb < 8 && gx * ceil_div(rows, 32 * (2 * nb)) >= 1024) nb *= 2;
  return nb;
}

fp4_status fp4_nv_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* codes,
                                uint8_t* scales, float* factors, float* panel_amax, fp4_round mode, uint64_t seed,
                                uint64_t offset, hipStream_t stream) {
  if (mode != FP4_RTN && mode != FP4_SR) return FP4_EINVAL;
  if (rows < 0 || !mult32z(cols) || ldx < cols) return FP4_ESHAPE;
  if (rows == 0 || cols == 0) return FP4_OK;
  if (!x || !codes || !scales || !factors || !panel_amax) return FP4_EINVAL;
  const int64_t gx = ceil_div(cols / 8, 256);
  if (gx > 0x7FFFFFFF || ceil_div(rows, 32) > 65535) return FP4_ESHAPE;
  if (!aligned16(x) || !aligned16(codes) || (ldx % 8) != 0) return FP4_EALIGN;
  const int64_t panels = ceil_div(rows, kNvPanel);
  const int nb = nv_amax_batches(gx, rows);
  const int64_t gya = ceil_div(rows, 32 * nb);
  const int64_t gy = std::min<int64_t>(std::min<int64_t>(std::max<int64_t>(1, 8192 / gx), ceil_div(rows, kNvRowsPerPass)),
                                       65535);
  hipStream_t s = as_stream(stream);
  uint32_t* amax = reinterpret_cast<uint32_t*>(panel_amax);
  hipLaunchKernelGGL(nv_fill_kernel, dim3((unsigned)ceil_div(panels, 256)), dim3(256), 0, s, amax, panels);
  hipLaunchKernelGGL(nv_amax_kernel, dim3((unsigned)gx, (unsigned)gya), dim3(256), 0, s, x, rows, cols, ldx, amax, 1,
                     nb);
  if (mode == FP4_SR && rows <= (int64_t(1) << 34) / cols)   // counters below 2^32
    hipLaunchKernelGGL((nv_rows_kernel<true, true>), dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s, x, rows, cols,
                       ldx, codes, scales, factors, amax, seed, offset);
  else if (mode == FP4_SR)
    hipLaunchKernelGGL(nv_rows_kernel<true>, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s, x, rows, cols, ldx,
                       codes, scales, factors, amax, seed, offset);
  else
    hipLaunchKernelGGL(nv_rows_kernel<false>, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s, x, rows, cols, ldx,
                       codes, scales, factors, amax, seed, offset);
  return launch_status();
}

fp4_status fp4_nv_quantize_w2d16(const uint16_t* w, int64_t n, int64_t k, int64_t ldw, uint8_t* row_codes,
                                 uint8_t* row_scales, uint8_t* col_codes, uint8_t* col_scales, float* factor,
                                 float* amax_out, hipStream_t stream) {
  if (!mult32z(n) || !mult32z(k) || ldw < k) return FP4_ESHAPE;
  if (n == 0 || k == 0) return FP4_OK;
  if (!w || !row_codes || !row_scales || !col_codes || !col_scales || !factor || !amax_out) return FP4_EINVAL;
  const int64_t gxa = ceil_div(k / 8, 256);
  const int64_t gk = ceil_div(k, 128), gy = ceil_div(n, 128);
  if (gxa > 0x7FFFFFFF || n / 32 > 65535 || ldw >= ((int64_t)1 << 22)) return FP4_ESHAPE;
  if (!aligned16(w) || !aligned16(row_codes) || !aligned16(col_codes) || (ldw % 8) != 0) return FP4_EALIGN;
  const int nb = nv_amax_batches(gxa, n);
  // about 512 long-running workgroups, each walking a run of macro tiles along K
  const int64_t want_x = std::max<int64_t>(1, 512 / gy);
  const int per = (int)ceil_div(gk, want_x);
  const int64_t gx = ceil_div(gk, per);
  hipStream_t s = as_stream(stream);
  uint32_t* amax = reinterpret_cast<uint32_t*>(amax_out);
  hipLaunchKernelGGL(nv_fill_kernel, dim3(1), dim3(256), 0, s, amax, (int64_t)1);
  hipLaunchKernelGGL(nv_amax_kernel, dim3((unsigned)gxa, (unsigned)ceil_div(n, 32 * nb)), dim3(256), 0, s, w, n, k,
                     ldw, amax, 0, nb);
  hipLaunchKernelGGL(nv_w2d16_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s, w, n, k, ldw, row_codes,
                     row_scales, col_codes, col_scales, factor, amax, per);
  return launch_status();
}

fp4_status fp4_nv_gemm(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes, const uint8_t* a_scales,
                       const float* a_factors, int64_t a_factor_stride, const uint8_t* b_codes,
                       const uint8_t* b_scales, const float* b_factors, int64_t b_factor_stride, float* c,
                       int64_t ldc, int accumulate, hipStream_t stream) {
  if (accumulate != 0 && accumulate != 1) return FP4_EINVAL;
  if (a_factor_stride < 0 || b_factor_stride < 0) return FP4_EINVAL;
  if (!mult32z(m) || !mult32z(n) || k < 0 || (k % 64) != 0 || ldc < n || k >= ((int64_t)1 << 24)) return FP4_ESHAPE;
  if (m == 0 || n == 0) return FP4_OK;
  if (!c) return FP4_EINVAL;
  const int64_t tm = ceil_div(m, 256), tn = ceil_div(n, 256);
  if (tm > 0x7FFFFFFF / tn) return FP4_ESHAPE;
  if (k == 0) return fp4_gemm(m, n, 0, nullptr, nullptr, nullptr, nullptr, c, ldc, accumulate, stream);
  if (!a_codes || !a_scales || !a_factors || !b_codes || !b_scales || !b_factors) return FP4_EINVAL;
  if (!aligned16(a_codes) || !aligned16(b_codes) || !aligned16(c) || (ldc % 4) != 0) return FP4_EALIGN;
  hipLaunchKernelGGL(nv_gemm_kernel, dim3((unsigned)(tm * tn)), dim3(512), 0, as_stream(stream), m, n, k, a_codes,
                     a_scales, a_factors, a_factor_stride, b_codes, b_scales, b_factors, b_factor_stride, c, ldc,
                     accumulate);
  return launch_status();
}

}  // extern "C"
