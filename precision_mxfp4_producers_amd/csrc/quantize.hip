// MXFP4 operand producers for gfx950: row-facing (RTN / Philox SR),
// column-facing (optionally fixed-sign H32) and the fused 2D32 weight producer.
//
// "Format-Aware Fusion for Fast FP4 Pretraining":
//   §2.2.1  upward E8M0 scales over 32-value blocks; adaptive finer 2D32 scale
//   §2.3    row-facing / column-facing views (Eq. 4-6, Fig. 4)
//   §2.4    one 2D32 encoding emitted in both layouts (Eq. 7-8, Fig. 5)
//   §2.5    SR on the Dgrad-facing dY only (Eq. 9); paired H32 on the Wgrad
//           operands, applied in registers during column quantization (Eq. 10)
//
// All producers are HBM-bound: each reads its bf16 input once with coalesced
// 16-byte (rows, 2D32) or 4-byte-per-lane row segments (cols) and writes packed
// codes plus one scale byte per 32 values.
#include <hip/hip_runtime.h>

#include "abi_common.h"
#include "mx_device.h"

namespace mx {

thread_local int g_last_hip_error = 0;

constexpr int kThreads = 256;
constexpr int kMaxGridY = 65535;

typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// Largest 15-bit magnitude pattern among eight bf16 values (four words).
__device__ __forceinline__ uint32_t bf16_absmax8(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  const u16x2_t a = __builtin_bit_cast(u16x2_t, w0 & 0x7FFF7FFFu), b = __builtin_bit_cast(u16x2_t, w1 & 0x7FFF7FFFu);
  const u16x2_t c = __builtin_bit_cast(u16x2_t, w2 & 0x7FFF7FFFu), d = __builtin_bit_cast(u16x2_t, w3 & 0x7FFF7FFFu);
  const u16x2_t m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  return max((uint32_t)m[0], (uint32_t)m[1]);
}

// ------------------------------------------------------------------ rows
// One lane quantizes 8 consecutive values (one 16-byte load); four lanes share
// a 32-value block and reduce its maximum over the quad (DPP).  bf16
// magnitudes are ordered like their 15-bit integer patterns, so the maximum
// is an integer max.  RTN goes through the hardware converter; SR draws
// Philox words for the lane's 8 elements (two counters).
template <bool kSR>
__global__ __launch_bounds__(kThreads) void quant_rows_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint64_t seed, uint64_t offset) {
  const int64_t cpr = cols >> 3;                         // 8-value chunks per row
  const int64_t c8 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const bool col_ok = c8 < cpr;                          // quads are all-in or all-out
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (col_ok) v = *reinterpret_cast<const uint4*>(x + r * ldx + c8 * 8);
    const uint32_t m = max_quad(bf16_absmax8(v.x, v.y, v.z, v.w));
    const int e = upward_exp(m << 16);
    uint32_t packed;
    if constexpr (kSR) {
      const uint64_t idx0 = (uint64_t)r * (uint64_t)cols + (uint64_t)c8 * 8u;
      const u32x4 a = sr_words(idx0 >> 2, seed, offset);
      const u32x4 b = sr_words((idx0 >> 2) + 1u, seed, offset);
      const uint32_t u[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      const float inv = inv_pow2(e);
      packed = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t bits = (w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
        const uint32_t mag = bits & 0x7FFFu;
        const float y = bf16_bits_to_f32(mag) * inv;     // exact (power-of-two scale)
        packed |= (e2m1_sr(y, u[i], mag != 0u) | ((bits >> 12) & 8u)) << (4 * i);
      }
    } else {
      packed = rtn8_bf16(v.x, v.y, v.z, v.w, pow2_scale(e));
    }
    if (col_ok) {
      *reinterpret_cast<uint32_t*>(codes + r * (cols >> 1) + c8 * 4) = packed;
      if ((c8 & 3) == 0) scales[r * (cols >> 5) + (c8 >> 2)] = (uint8_t)(e + 127);
    }
  }
}

// ------------------------------------------------------------------ cols
// One lane owns two adjacent columns and one 32-row block: it reads 32 row
// segments of 4 bytes (64 lanes cover 256 contiguous bytes per row), optionally
// applies the fixed-sign H32 to each column in registers (fp32, stage order
// of the contract), and writes each column's 16 code bytes to the transposed
// output.
__device__ __forceinline__ void h32_inplace(float (&f)[32]) {
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

// RTN MXFP4 of one 32-value fp32 block: upward scale of its maximum, codes.
__device__ __forceinline__ uint4 encode32_f32(const float (&f)[32], int& e_out) {
  float am = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) am = fmaxf(am, fabsf(f[j]));
  const int e = upward_exp(__float_as_uint(am));
  const float sc = pow2_scale(e);
  e_out = e;
  return make_uint4(rtn8_f32(f, sc), rtn8_f32(f + 8, sc), rtn8_f32(f + 16, sc), rtn8_f32(f + 24, sc));
}

template <bool kH32>
__global__ __launch_bounds__(kThreads) void quant_cols_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
    uint8_t* __restrict__ codes_t, uint8_t* __restrict__ scales_t, uint32_t sign_mask16) {
  const int64_t pairs = cols >> 1;
  const int64_t p = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (p >= pairs) return;                                // no cross-lane work below
  const int64_t nrb = rows >> 5;
  for (int64_t rb = blockIdx.y; rb < nrb; rb += gridDim.y) {
    uint32_t v[32];
    const uint16_t* src = x + (rb * 32) * ldx + 2 * p;
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = *reinterpret_cast<const uint32_t*>(src + (int64_t)i * ldx);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float f[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        uint32_t b = (v[i] >> (16 * c)) & 0xFFFFu;
        if constexpr (kH32) b ^= ((sign_mask16 >> (i & 15)) & 1u) << 15;   // d_(i mod 16)
        f[i] = bf16_bits_to_f32(b);
      }
      if constexpr (kH32) h32_inplace(f);
      int e;
      const uint4 code = encode32_f32(f, e);
      const int64_t col = 2 * p + c;
      *reinterpret_cast<uint4*>(codes_t + col * (rows >> 1) + rb * 16) = code;
      scales_t[col * (rows >> 5) + rb] = (uint8_t)(e + 127);
    }
  }
}

// ------------------------------------------------------------------ 2D32
// A 256-lane workgroup owns a 128x128 weight macro tile (4x4 tiles of 32x32).
// Lane (r = tid/2, half = tid&1) loads 64 values of row r: two tiles.  Wave w
// holds exactly tile-row w, so each tile maximum is a wave reduction over the
// lanes with equal `half`.  Row codes are written from registers; the bf16
// tile is staged in LDS once and re-read by columns to write the column
// layout with the same tile exponent (the encoding is a pure function of
// value and exponent, so both layouts hold the same nibble).
constexpr int kWPitch = 68;                              // dwords per LDS row (64 + 4 pad)

__global__ __launch_bounds__(kThreads) void quant_w2d32_kernel(
    const uint16_t* __restrict__ w, int64_t N, int64_t K, int64_t ldw,
    uint8_t* __restrict__ row_codes, uint8_t* __restrict__ row_scales,
    uint8_t* __restrict__ col_codes, uint8_t* __restrict__ col_scales, float finer_ratio) {
  __shared__ uint32_t tile[128 * kWPitch];
  __shared__ int tile_e[4][4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t n0 = (int64_t)blockIdx.y * 128, k0 = (int64_t)blockIdx.x * 128;
  const int r = tid >> 1, half = tid & 1;
  const bool row_ok = n0 + 32 * wave < N;                // uniform per wave
  bool t_ok[2];
  t_ok[0] = k0 + 32 * (2 * half) < K;
  t_ok[1] = k0 + 32 * (2 * half + 1) < K;

  uint32_t v[32];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint4 d = make_uint4(0u, 0u, 0u, 0u);
    if (row_ok && t_ok[q >> 2])
      d = *reinterpret_cast<const uint4*>(w + (n0 + r) * ldw + k0 + half * 64 + q * 8);
    v[4 * q] = d.x; v[4 * q + 1] = d.y; v[4 * q + 2] = d.z; v[4 * q + 3] = d.w;
  }
  // tile maxima (bf16 magnitude patterns), reduced over the 32 rows of the wave
  uint32_t m[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
    m[t] = max(max(bf16_absmax8(v[16 * t], v[16 * t + 1], v[16 * t + 2], v[16 * t + 3]),
                   bf16_absmax8(v[16 * t + 4], v[16 * t + 5], v[16 * t + 6], v[16 * t + 7])),
               max(bf16_absmax8(v[16 * t + 8], v[16 * t + 9], v[16 * t + 10], v[16 * t + 11]),
                   bf16_absmax8(v[16 * t + 12], v[16 * t + 13], v[16 * t + 14], v[16 * t + 15])));
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int s = 2; s < 64; s <<= 1) m[t] = max(m[t], (uint32_t)__shfl_xor((int)m[t], s));
  }
  int e[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint32_t ab = m[t] << 16;
    const int e_up = upward_exp(ab);
    const float lhs = __uint_as_float(ab) * inv_pow2(e_up);      // exact, in (3, 6]
    const bool finer = ((double)lhs < 6.0 * (double)finer_ratio) && e_up > -127;
    e[t] = finer ? e_up - 1 : e_up;
  }
  if (lane < 2) {                                        // lane 0: tiles 0,1; lane 1: tiles 2,3
    tile_e[wave][2 * lane] = e[0];
    tile_e[wave][2 * lane + 1] = e[1];
  }
  // stage the bf16 values for the column pass
#pragma unroll
  for (int q = 0; q < 8; ++q)
    *reinterpret_cast<uint4*>(&tile[r * kWPitch + half * 32 + q * 4]) =
        make_uint4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);

  // row layout straight from registers (adjacent K values share a word)
  if (row_ok) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (!t_ok[t]) continue;
      const float sc = pow2_scale(e[t]);
      const uint32_t* q = v + 16 * t;
      const uint4 out = make_uint4(rtn8_bf16(q[0], q[1], q[2], q[3], sc), rtn8_bf16(q[4], q[5], q[6], q[7], sc),
                                   rtn8_bf16(q[8], q[9], q[10], q[11], sc), rtn8_bf16(q[12], q[13], q[14], q[15], sc));
      const int64_t kk = k0 + half * 64 + t * 32;
      *reinterpret_cast<uint4*>(row_codes + (n0 + r) * (K >> 1) + (kk >> 1)) = out;
      row_scales[(n0 + r) * (K >> 5) + (kk >> 5)] = (uint8_t)(e[t] + 127);
    }
  }
  __syncthreads();

  // column layout: wave q = tile-row, lane = column pair within the macro tile;
  // v_perm gathers (row 2j, row 2j+1) of one column into a bf16 pair
  {
    const int q = wave, pcol = lane;                     // columns 2*pcol, 2*pcol+1
    const int tc = pcol >> 4;
    if (n0 + 32 * q < N && k0 + 32 * tc < K) {
      const int et = tile_e[q][tc];
      const float sc = pow2_scale(et);
      uint32_t d[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) d[i] = tile[(32 * q + i) * kWPitch + pcol];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint32_t sel = c ? 0x07060302u : 0x05040100u;
        uint32_t pr[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) pr[j] = __builtin_amdgcn_perm(d[2 * j + 1], d[2 * j], sel);
        const uint4 out = make_uint4(rtn8_bf16(pr[0], pr[1], pr[2], pr[3], sc), rtn8_bf16(pr[4], pr[5], pr[6], pr[7], sc),
                                     rtn8_bf16(pr[8], pr[9], pr[10], pr[11], sc),
                                     rtn8_bf16(pr[12], pr[13], pr[14], pr[15], sc));
        const int64_t kcol = k0 + 2 * pcol + c;
        *reinterpret_cast<uint4*>(col_codes + kcol * (N >> 1) + ((n0 + 32 * q) >> 1)) = out;
        col_scales[kcol * (N >> 5) + ((n0 >> 5) + q)] = (uint8_t)(et + 127);
      }
    }
  }
}

}  // namespace mx

using namespace mx;

extern "C" {

fp4_status fp4_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                             uint8_t* codes, uint8_t* scales, int mode, uint64_t seed,
                             uint64_t offset, void* stream) {
  if (!x || !codes || !scales || (mode != FP4_RTN && mode != FP4_SR)) return FP4_EINVAL;
  if (rows <= 0 || !mult32(cols) || ldx < cols) return FP4_ESHAPE;
  if (!aligned16(x) || !aligned16(codes) || (ldx % 8) != 0) return FP4_EALIGN;
  const int64_t cpr = cols >> 3;
  dim3 grid((unsigned)((cpr + kThreads - 1) / kThreads), (unsigned)(rows < kMaxGridY ? rows : kMaxGridY));
  hipStream_t s = as_stream(stream);
  if (mode == FP4_SR)
    hipLaunchKernelGGL(quant_rows_kernel<true>, grid, dim3(kThreads), 0, s, x, rows, cols, ldx, codes,
                       scales, seed, offset);
  else
    hipLaunchKernelGGL(quant_rows_kernel<false>, grid, dim3(kThreads), 0, s, x, rows, cols, ldx, codes,
                       scales, seed, offset);
  return launch_status();
}

fp4_status fp4_quantize_cols(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                             uint8_t* codes_t, uint8_t* scales_t, int hadamard,
                             uint32_t sign_mask16, void* stream) {
  if (!x || !codes_t || !scales_t || (hadamard != 0 && hadamard != 32)) return FP4_EINVAL;
  if (!mult32(rows) || !mult32(cols) || ldx < cols) return FP4_ESHAPE;
  if (!aligned16(x) || !aligned16(codes_t) || (ldx % 8) != 0) return FP4_EALIGN;
  const int64_t pairs = cols >> 1, nrb = rows >> 5;
  dim3 grid((unsigned)((pairs + kThreads - 1) / kThreads), (unsigned)(nrb < kMaxGridY ? nrb : kMaxGridY));
  hipStream_t s = as_stream(stream);
  if (hadamard == 32)
    hipLaunchKernelGGL(quant_cols_kernel<true>, grid, dim3(kThreads), 0, s, x, rows, cols, ldx, codes_t,
                       scales_t, sign_mask16 & 0xFFFFu);
  else
    hipLaunchKernelGGL(quant_cols_kernel<false>, grid, dim3(kThreads), 0, s, x, rows, cols, ldx, codes_t,
                       scales_t, 0u);
  return launch_status();
}

fp4_status fp4_quantize_w2d32(const uint16_t* w, int64_t n, int64_t k, int64_t ldw,
                              uint8_t* row_codes, uint8_t* row_scales, uint8_t* col_codes,
                              uint8_t* col_scales, float finer_ratio, void* stream) {
  if (!w || !row_codes || !row_scales || !col_codes || !col_scales) return FP4_EINVAL;
  if (!(finer_ratio >= 0.0f && finer_ratio <= 1.0f)) return FP4_EINVAL;
  if (!mult32(n) || !mult32(k) || ldw < k) return FP4_ESHAPE;
  if (!aligned16(w) || !aligned16(row_codes) || !aligned16(col_codes) || (ldw % 8) != 0)
    return FP4_EALIGN;
  const int64_t gx = (k + 127) / 128, gy = (n + 127) / 128;
  if (gy > kMaxGridY) return FP4_ESHAPE;
  hipLaunchKernelGGL(quant_w2d32_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0,
                     as_stream(stream), w, n, k, ldw, row_codes, row_scales, col_codes, col_scales,
                     finer_ratio);
  return launch_status();
}

uint32_t fp4_sign_mask_from_seed(uint64_t seed) {
  // Host copy of Philox4x32-10 (same round function as the device code).
  uint32_t c0 = 0, c1 = 0, c2 = 0, c3 = 0;
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n1 = (uint32_t)p1;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1, n3 = (uint32_t)p0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c0 & 0xFFFFu;
}

int fp4_last_hip_error(void) { return g_last_hip_error; }

int fp4_abi_version(void) { return (1 << 16) | 0; }

}  // extern "C"
