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
// lies in [2^-10, 2688], so it is exact in bf16.  The GEMM decodes each K step
// of codes and scales into bf16 in LDS and runs the bf16 MFMA
// (v_mfma_f32_32x32x16_bf16) with fp32 accumulation; the epilogue multiplies by
// RN(S_A * S_B), one product per 256 x 256 output tile (the tile is one panel
// of each operand).
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

__device__ __forceinline__ float e4m3_value(uint32_t byte) {
  const uint32_t e = (byte >> 3) & 15u, m = byte & 7u;
  return e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
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
// Each workgroup reduces 32 rows x 2048 columns and issues one atomic max.
__global__ __launch_bounds__(256) void nv_fill_kernel(uint32_t* __restrict__ v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) v[i] = 0u;
}

__global__ __launch_bounds__(256) void nv_amax_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                      int64_t ldx, uint32_t* __restrict__ amax, int per_panel) {
  const int64_t r0 = (int64_t)blockIdx.y * 32;
  const int64_t c8 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t m = 0;
  if (c8 * 8 < cols) {
    for (int r = 0; r < 32 && r0 + r < rows; ++r) {
      const uint4 v = load_once_u4(x + (r0 + r) * ldx + c8 * 8);
      m = max(m, bf16_absmax8(v.x, v.y, v.z, v.w));
    }
  }
  // wave maximum, then one atomic per wave
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, s));
  if ((threadIdx.x & 63) == 0 && m != 0) atomicMax(amax + (per_panel ? r0 / kNvPanel : 0), m << 16);
}

// ------------------------------------------------------------------ rows
// Lane: 8 consecutive values of one row (one 16-byte load); two lanes share
// a 16-value block (DPP max).
template <bool kSR>
__global__ __launch_bounds__(256) void nv_rows_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                      int64_t ldx, uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales, float* __restrict__ factors,
                                                      const uint32_t* __restrict__ amax, uint64_t seed,
                                                      uint64_t offset) {
  const int64_t cpr = cols >> 3;
  const int64_t c8 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool col_ok = c8 < cpr;
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    const int64_t p = r / kNvPanel;
    const float S = nv_factor(__uint_as_float(amax[p]));
    const float inv6 = __fdiv_rn(1.0f, __fmul_rn(6.0f, S));
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (col_ok) v = load_once_u4(x + r * ldx + c8 * 8);
    uint32_t m = bf16_absmax8(v.x, v.y, v.z, v.w);
    m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false));   // pair: lanes 2j, 2j+1
    uint32_t byte;
    float rr;
    nv_block(bf16_bits_to_f32(m), S, inv6, byte, rr);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t packed;
    if constexpr (kSR) {
      const uint64_t blk = ((uint64_t)r * (uint64_t)cols + (uint64_t)c8 * 8u) >> 2;
      const u32x4 a = sr_words(blk, seed, offset), b = sr_words(blk + 1u, seed, offset);
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
}

// ------------------------------------------------------------------ 2D16 weights
// A 256-lane workgroup owns 64 rows x 64 columns (4 x 4 tiles of 16 x 16).
// Lane (row t/4, 16-column group t%4) loads its 16 values; a tile's maximum is
// the maximum over the 16 lanes that share its column group in a wave (lane
// bits 2-5).  Row codes go out from registers; the column view re-reads the
// bf16 tile from LDS by columns with the same tile scale.
__global__ __launch_bounds__(256) void nv_w2d16_kernel(const uint16_t* __restrict__ w, int64_t N, int64_t K,
                                                       int64_t ldw, uint8_t* __restrict__ row_codes,
                                                       uint8_t* __restrict__ row_scales,
                                                       uint8_t* __restrict__ col_codes,
                                                       uint8_t* __restrict__ col_scales, float* __restrict__ factor,
                                                       const uint32_t* __restrict__ amax) {
  __shared__ __attribute__((aligned(16))) uint32_t tile[64][33];          // 64 rows x 64 bf16 (+1 dword pad)
  __shared__ uint32_t tbyte[4][4];
  __shared__ float tr[4][4];
  const int t = threadIdx.x, row = t >> 2, grp = t & 3;
  const int64_t n0 = (int64_t)blockIdx.y * 64, k0 = (int64_t)blockIdx.x * 64;
  const float S = nv_factor(__uint_as_float(amax[0]));
  const float inv6 = __fdiv_rn(1.0f, __fmul_rn(6.0f, S));
  uint32_t v[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  const bool ok = n0 + row < N && k0 + 16 * grp < K;                     // whole 16-value groups (K % 16 == 0)
  if (ok) {
    const uint4 a = load_once_u4(w + (n0 + row) * ldw + k0 + 16 * grp);
    const uint4 b = load_once_u4(w + (n0 + row) * ldw + k0 + 16 * grp + 8);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  uint32_t m = max(bf16_absmax8(v[0], v[1], v[2], v[3]), bf16_absmax8(v[4], v[5], v[6], v[7]));
#pragma unroll
  for (int s = 4; s <= 32; s <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, s));
  uint32_t byte;
  float r;
  nv_block(bf16_bits_to_f32(m), S, inv6, byte, r);
  const int tr_row = row >> 4;                                           // tile row within the macro tile
  if ((t & 63) < 4) {
    tbyte[tr_row][grp] = byte;
    tr[tr_row][grp] = r;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) tile[row][8 * grp + j] = v[j];
  if (ok) {
    const uint32_t w0[4] = {v[0], v[1], v[2], v[3]}, w1[4] = {v[4], v[5], v[6], v[7]};
    *reinterpret_cast<uint2*>(row_codes + (n0 + row) * (K >> 1) + ((k0 + 16 * grp) >> 1)) =
        make_uint2(nv_rtn8(w0, r), nv_rtn8(w1, r));
    row_scales[(n0 + row) * (K >> 4) + ((k0 >> 4) + grp)] = (uint8_t)byte;
  }
  if (blockIdx.x == 0 && blockIdx.y == 0 && t == 0) factor[0] = S;
  __syncthreads();
  // column view: lane (column t%64, 16-row group t/64)
  {
    const int c = t & 63, rg = t >> 6;
    const int64_t col = k0 + c;
    if (col < K && n0 + 16 * rg < N) {
      const uint32_t b = tbyte[rg][c >> 4];
      const float rc = tr[rg][c >> 4];
      uint32_t cw[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t lo = (tile[16 * rg + 2 * i][c >> 1] >> (16 * (c & 1))) & 0xFFFFu;
        const uint32_t hi = (tile[16 * rg + 2 * i + 1][c >> 1] >> (16 * (c & 1))) & 0xFFFFu;
        cw[i] = lo | (hi << 16);
      }
      const uint32_t w0[4] = {cw[0], cw[1], cw[2], cw[3]}, w1[4] = {cw[4], cw[5], cw[6], cw[7]};
      *reinterpret_cast<uint2*>(col_codes + col * (N >> 1) + ((n0 + 16 * rg) >> 1)) =
          make_uint2(nv_rtn8(w0, rc), nv_rtn8(w1, rc));
      col_scales[col * (N >> 4) + ((n0 >> 4) + rg)] = (uint8_t)b;
    }
  }
}

// ------------------------------------------------------------------ GEMM
// 256 x 256 output tile, 8 waves of 128 x 64 (as the MXFP4 fast kernel), K in
// steps of 64 values.  Per step, lane t decodes 32 values of row t/2 of each
// operand (16 code bytes + 2 E4M3 scale bytes) into bf16 and writes them to
// the LDS stage (128 bytes per row, 16-byte chunks XOR-swizzled per row).
// Sub-step s of a step reads chunk 2s + lane/32 (8 bf16 = k 8(lane/32) ..).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
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

// One code word (8 values) times block scale d -> four bf16 words (exact).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t nv_dec2(f32x2_t q, float d) {
  return bf16_pack2_rne(__fmul_rn(q.x, d), __fmul_rn(q.y, d));
}
__device__ __forceinline__ void nv_decode8(uint32_t w, float d, uint32_t* o) {
  o[0] = nv_dec2(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0), d);
  o[1] = nv_dec2(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1), d);
  o[2] = nv_dec2(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2), d);
  o[3] = nv_dec2(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3), d);
}

// 32 codes (16 bytes) with scales d0 (first 16) and d1 -> 32 bf16 (16 words)
__device__ __forceinline__ void nv_decode32(uint4 c, float d0, float d1, uint32_t (&o)[16]) {
  nv_decode8(c.x, d0, o);
  nv_decode8(c.y, d0, o + 4);
  nv_decode8(c.z, d1, o + 8);
  nv_decode8(c.w, d1, o + 12);
}

__device__ __forceinline__ void nv_store_stage(uint8_t* stage, const NvLoad& x, int row, int half) {
  uint32_t a[16], b[16];
  nv_decode32(x.ca, e4m3_value(x.sa & 0xFFu), e4m3_value(x.sa >> 8), a);
  nv_decode32(x.cb, e4m3_value(x.sb & 0xFFu), e4m3_value(x.sb >> 8), b);
  uint8_t* la = stage + row * 128;
  uint8_t* lb = stage + 256 * 128 + row * 128;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ch = swz(row, 4 * half + q);
    *reinterpret_cast<uint4*>(la + ch * 16) = make_uint4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
    *reinterpret_cast<uint4*>(lb + ch * 16) = make_uint4(b[4 * q], b[4 * q + 1], b[4 * q + 2], b[4 * q + 3]);
  }
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
  NvLoad ld;
  nv_load(ld, rca, rsa, rcb, rsb, K, 0, row, half);
  nv_store_stage(smem, ld, row, half);
  __syncthreads();
  for (int s = 0; s < nk; ++s) {
    const bool more = s + 1 < nk;
    if (more) nv_load(ld, rca, rsa, rcb, rsb, K, s + 1, row, half);
    const uint8_t* la = smem + (s & 1) * kNvStage;
    const uint8_t* lb = la + 256 * 128;
#pragma unroll
    for (int ss = 0; ss < 4; ++ss) {
      const int ch = 2 * ss + hl;
      bf16x8_t af[4], bfr[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ar = wm * 128 + 32 * i + r;
        af[i] = *reinterpret_cast<const bf16x8_t*>(la + ar * 128 + swz(ar, ch) * 16);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int br = wn * 64 + 32 * j + r;
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(lb + br * 128 + swz(br, ch) * 16);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
    if (more) nv_store_stage(smem + ((s + 1) & 1) * kNvStage, ld, row, half);
    __syncthreads();
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

fp4_status fp4_nv_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* codes,
                                uint8_t* scales, float* factors, float* panel_amax, int mode, uint64_t seed,
                                uint64_t offset, void* stream) {
  if (mode != FP4_RTN && mode != FP4_SR) return FP4_EINVAL;
  if (rows < 0 || !mult32z(cols) || ldx < cols) return FP4_ESHAPE;
  if (rows == 0 || cols == 0) return FP4_OK;
  if (!x || !codes || !scales || !factors || !panel_amax) return FP4_EINVAL;
  const int64_t gx = ceil_div(cols / 8, 256), gya = ceil_div(rows, 32);
  if (gx > 0x7FFFFFFF || gya > 65535) return FP4_ESHAPE;
  if (!aligned16(x) || !aligned16(codes) || (ldx % 8) != 0) return FP4_EALIGN;
  const int64_t panels = ceil_div(rows, kNvPanel);
  const int64_t gy = std::min<int64_t>(std::min<int64_t>(std::max<int64_t>(1, 8192 / gx), rows), 65535);
  hipStream_t s = as_stream(stream);
  uint32_t* amax = reinterpret_cast<uint32_t*>(panel_amax);
  hipLaunchKernelGGL(nv_fill_kernel, dim3((unsigned)ceil_div(panels, 256)), dim3(256), 0, s, amax, panels);
  hipLaunchKernelGGL(nv_amax_kernel, dim3((unsigned)gx, (unsigned)gya), dim3(256), 0, s, x, rows, cols, ldx, amax, 1);
  if (mode == FP4_SR)
    hipLaunchKernelGGL(nv_rows_kernel<true>, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s, x, rows, cols, ldx,
                       codes, scales, factors, amax, seed, offset);
  else
    hipLaunchKernelGGL(nv_rows_kernel<false>, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s, x, rows, cols, ldx,
                       codes, scales, factors, amax, seed, offset);
  return launch_status();
}

fp4_status fp4_nv_quantize_w2d16(const uint16_t* w, int64_t n, int64_t k, int64_t ldw, uint8_t* row_codes,
                                 uint8_t* row_scales, uint8_t* col_codes, uint8_t* col_scales, float* factor,
                                 float* amax_out, void* stream) {
  if (!mult32z(n) || !mult32z(k) || ldw < k) return FP4_ESHAPE;
  if (n == 0 || k == 0) return FP4_OK;
  if (!w || !row_codes || !row_scales || !col_codes || !col_scales || !factor || !amax_out) return FP4_EINVAL;
  const int64_t gxa = ceil_div(k / 8, 256), gya = n / 32;
  const int64_t gx = ceil_div(k, 64), gy = ceil_div(n, 64);
  if (gxa > 0x7FFFFFFF || gx > 0x7FFFFFFF || gya > 65535) return FP4_ESHAPE;
  if (!aligned16(w) || !aligned16(row_codes) || !aligned16(col_codes) || (ldw % 8) != 0) return FP4_EALIGN;
  hipStream_t s = as_stream(stream);
  uint32_t* amax = reinterpret_cast<uint32_t*>(amax_out);
  hipLaunchKernelGGL(nv_fill_kernel, dim3(1), dim3(256), 0, s, amax, (int64_t)1);
  hipLaunchKernelGGL(nv_amax_kernel, dim3((unsigned)gxa, (unsigned)gya), dim3(256), 0, s, w, n, k, ldw, amax, 0);
  hipLaunchKernelGGL(nv_w2d16_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s, w, n, k, ldw, row_codes,
                     row_scales, col_codes, col_scales, factor, amax);
  return launch_status();
}

fp4_status fp4_nv_gemm(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes, const uint8_t* a_scales,
                       const float* a_factors, int64_t a_factor_stride, const uint8_t* b_codes,
                       const uint8_t* b_scales, const float* b_factors, int64_t b_factor_stride, float* c,
                       int64_t ldc, int accumulate, void* stream) {
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
