// Elementwise SwiGLU backward (gated FFN of "Format-Aware Fusion for Fast FP4
// Pretraining", §3.2): from the fp32 W2 data gradient dH and the saved bf16
// gate/up outputs a, b,
//   sig = 1/(1+exp(-a)), s = a*sig
//   dA = bf16(((dH*b)*sig) * (1 + a*(1 - sig))),  dB = bf16(dH*s)
// with single fp32 roundings in this order and no FMA outside the exp (whose
// reduction and Horner steps are fused multiply-adds).  HBM-bound: 12 bytes
// per element (4 read dH, 2+2 read a/b, 2+2 written dA/dB).
//
// The fused backward producer applies the same arithmetic and emits dA and dB
// directly in the two representations their consumers read (§2.3, §2.5, §3.1:
// the producer completes every layout the next contractions need): row-facing
// with Philox SR for the W1/W3 Dgrad and column-facing with the fixed-sign H32
// for the W1/W3 Wgrad.  The bf16 dA, dB never leave the chip.
#include <hip/hip_runtime.h>

#include "abi_common.h"
#include "mx_device.h"

namespace mx {

constexpr int kBwdThreads = 256;
constexpr int kMaxGridY = 65535;
constexpr int64_t kMaxGridX = 0x7FFFFFFF;

// One lane handles 8 consecutive elements of a row.
__global__ __launch_bounds__(kBwdThreads) void swiglu_bwd_kernel(
    int64_t T, int64_t Fdim, const float* __restrict__ dh, int64_t lddh, const uint16_t* __restrict__ a,
    const uint16_t* __restrict__ b, uint16_t* __restrict__ da, uint16_t* __restrict__ db) {
  const int64_t cpr = Fdim >> 3;
  const int64_t c8 = (int64_t)blockIdx.x * kBwdThreads + threadIdx.x;
  if (c8 >= cpr) return;
  for (int64_t r = blockIdx.y; r < T; r += gridDim.y) {
    const float* dp = dh + r * lddh + c8 * 8;
    const float4 d0 = *reinterpret_cast<const float4*>(dp);
    const float4 d1 = *reinterpret_cast<const float4*>(dp + 4);
    const uint4 av = *reinterpret_cast<const uint4*>(a + r * Fdim + c8 * 8);
    const uint4 bv = *reinterpret_cast<const uint4*>(b + r * Fdim + c8 * 8);
    const float dv[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
    const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
    const uint32_t bw[4] = {bv.x, bv.y, bv.z, bv.w};
    uint32_t oa[4] = {0u, 0u, 0u, 0u}, ob[4] = {0u, 0u, 0u, 0u};
    float afv[8], sgv[8], slv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) afv[i] = bf16_bits_to_f32((aw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
    sigmoid_silu_n<8>(afv, sgv, slv);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float af = afv[i];
      const float bf = bf16_bits_to_f32((bw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
      const float sig = sgv[i], s = slv[i];
      const float g = __fadd_rn(1.0f, __fmul_rn(af, __fsub_rn(1.0f, sig)));
      const float dav = __fmul_rn(__fmul_rn(__fmul_rn(dv[i], bf), sig), g);
      const float dbv = __fmul_rn(dv[i], s);
      oa[i >> 1] |= f32_to_bf16_rne(dav) << (16 * (i & 1));
      ob[i >> 1] |= f32_to_bf16_rne(dbv) << (16 * (i & 1));
    }
    *reinterpret_cast<uint4*>(da + r * Fdim + c8 * 8) = make_uint4(oa[0], oa[1], oa[2], oa[3]);
    *reinterpret_cast<uint4*>(db + r * Fdim + c8 * 8) = make_uint4(ob[0], ob[1], ob[2], ob[3]);
  }
}


// ------------------------------------------------------------ fused producer
// A workgroup of kFbThreads lanes owns kFbCols FFN columns x kFbTok tokens,
// walked in chunks of kFbChunk tokens:
//   1. dA, dB of the chunk in bf16 into LDS (lane: 8 columns x 2 rows);
//   2. row-facing SR of every 32-column block (lane: one block of one row of
//      one tensor; four lanes cover a row's 64 code bytes), draws indexed by
//      the element's row-major index in the full [t][f] tensor;
//   3. column-facing H32 of every 32-token block (lane: one column of one
//      tensor), codes parked in LDS per column;
// and finally each column's kFbTok/2 code bytes -- a whole 128-byte line --
// go out with coalesced stores.  The kernel is ALU-bound (the exp chain, the
// Philox draws, the H32 butterflies): the LDS (two workgroups per CU) sets the
// occupancy, so each workgroup has eight waves and the per-lane work is
// split finely enough that a lane stays within 128 registers (four waves per
// SIMD).
constexpr int kFbThreads = 512;
constexpr int kFbCols = 128, kFbTok = 256, kFbChunk = 64;
constexpr int kFbRowsPerLane = kFbChunk * (kFbCols / 8) / kFbThreads;   // 2
constexpr int kFbPitch = 272;                            // bytes per staged bf16 row (256 + 16)
constexpr int kFbCodePitch = kFbTok / 2 + 16;            // bytes per staged column of codes
static_assert(kFbRowsPerLane * kFbThreads == kFbChunk * (kFbCols / 8), "phase 1 covers the chunk");
static_assert(2 * kFbChunk * (kFbCols / 32) == kFbThreads, "phase 2: one (tensor, row, block) per lane");
static_assert(2 * (kFbChunk / 32) * kFbCols == kFbThreads, "phase 3: one (tensor, token block, column) per lane");

struct FbOut {
  uint8_t* codes;                                        // row-facing [t][f/2]
  uint8_t* scales;                                       // [t][f/32]
  uint8_t* codes_t;                                      // column-facing [f][t/2]
  uint8_t* scales_t;                                     // [f][t/32]
  uint64_t offset;                                       // SR counter offset
};

// Inputs of one chunk for one lane: rows rg + 32k (k < kFbRowsPerLane), 8 columns.
struct FbIn {
  float4 d[kFbRowsPerLane][2];
  uint4 a[kFbRowsPerLane], b[kFbRowsPerLane];
};

// Chunk `ck` of the workgroup's tile (t0, c0): buffer resources span the
// chunk's rows that lie inside the tensor (none for a chunk past the tile), so
// loads of later rows return zero; columns past f are sent past every
// resource (kOffNone).  Byte offsets stay below 2^31: 64 rows x lddh x 4 with
// lddh < 2^23, checked on the host.
__device__ __forceinline__ void fb_load(FbIn& in, const float* dh, int64_t lddh, const uint16_t* a,
                                        const uint16_t* b, int64_t Fdim, int64_t t0, int64_t c0, int ntok, int ck,
                                        int rg, int cc, bool col_ok) {
  const int rows = max(0, min(kFbChunk, ntok - ck * kFbChunk));
  const int64_t r0 = t0 + (int64_t)ck * kFbChunk;
  const int64_t base = rows > 0 ? r0 : t0;               // keep the base inside the tensor
  const __amdgpu_buffer_rsrc_t rd = buffer_rsrc(dh + base * lddh + c0, (int64_t)rows * lddh * 4);
  const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(a + base * Fdim + c0, (int64_t)rows * Fdim * 2);
  const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(b + base * Fdim + c0, (int64_t)rows * Fdim * 2);
#pragma unroll
  for (int k = 0; k < kFbRowsPerLane; ++k) {
    const uint32_t r = (uint32_t)(rg + 32 * k);
    const uint32_t od = col_ok ? r * (uint32_t)lddh * 4u + (uint32_t)cc * 32u : kOffNone;
    const uint32_t oab = col_ok ? r * (uint32_t)Fdim * 2u + (uint32_t)cc * 16u : kOffNone;
    in.d[k][0] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rd, od, 0, 0));
    in.d[k][1] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rd, od + 16u, 0, 0));
    in.a[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, oab, 0, 0));
    in.b[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rb, oab, 0, 0));
  }
}

// kIdx32: the tensors hold at most 2^34 elements, so every Philox counter's
// second word is 0 (sr_words32).
template <bool kIdx32>
__global__ __launch_bounds__(kFbThreads) void swiglu_bwd_producer_kernel(
    int64_t T, int64_t Fdim, const float* __restrict__ dh, int64_t lddh, const uint16_t* __restrict__ a,
    const uint16_t* __restrict__ b, FbOut oa, FbOut ob, uint64_t seed, uint32_t sign_mask16) {
  __shared__ __attribute__((aligned(16))) uint8_t gs[2][kFbChunk * kFbPitch];          // dA, dB chunk
  __shared__ __attribute__((aligned(16))) uint8_t cs[2][kFbCols * kFbCodePitch];       // column codes
  __shared__ uint8_t ss[2][kFbCols][kFbTok / 32];                                      // column scales
  const int tid = threadIdx.x;
  // neighbouring column tiles write the two halves of each row-code line:
  // keep them on one XCD
  uint32_t bx, by;
  xcd_block(0, bx, by);
  const int64_t c0 = (int64_t)bx * kFbCols, t0 = (int64_t)by * kFbTok;
  const int ncol = (int)min<int64_t>(kFbCols, Fdim - c0);          // multiple of 32
  const int ntok = (int)min<int64_t>(kFbTok, T - t0);              // multiple of 32

  // 1. dA, dB inputs of a chunk: lane (8 columns from cc*8, rows rg + 32k)
  // through buffer resources over the chunk's valid rows, so rows past T and
  // columns past f read zero and need no branch; the next chunk's loads are
  // issued right after this chunk's values are consumed and arrive while its
  // SR and H32 passes run.
  const int cc = tid & 15, rg = tid >> 4;
  const bool col_ok = cc * 8 < ncol;
  const int nchunks = (ntok + kFbChunk - 1) / kFbChunk;
  FbIn in;
  fb_load(in, dh, lddh, a, b, Fdim, t0, c0, ntok, 0, rg, cc, col_ok);
  for (int ck = 0; ck < nchunks; ++ck) {
    const int nrow = min(kFbChunk, ntok - ck * kFbChunk);           // 32 or 64
    const int64_t r0 = t0 + ck * kFbChunk;
    {
#pragma unroll
      for (int k = 0; k < kFbRowsPerLane; ++k) {
        const int r = rg + 32 * k;
        // zero inputs (rows or columns past the tensor) give +0 for dA and dB
        const float dv[8] = {in.d[k][0].x, in.d[k][0].y, in.d[k][0].z, in.d[k][0].w,
                             in.d[k][1].x, in.d[k][1].y, in.d[k][1].z, in.d[k][1].w};
        const uint32_t aw[4] = {in.a[k].x, in.a[k].y, in.a[k].z, in.a[k].w};
        const uint32_t bw[4] = {in.b[k].x, in.b[k].y, in.b[k].z, in.b[k].w};
        uint32_t oa4[4], ob4[4];
        float afv[8], sig[8], sl[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) afv[i] = bf16_bits_to_f32((aw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
        sigmoid_silu_n<8>(afv, sig, sl);
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          float dav[2], dbv[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const float af = afv[i + u];
            const float bf = bf16_bits_to_f32((bw[i >> 1] >> (16 * u)) & 0xFFFFu);
            const float g = __fadd_rn(1.0f, __fmul_rn(af, __fsub_rn(1.0f, sig[i + u])));
            dav[u] = __fmul_rn(__fmul_rn(__fmul_rn(dv[i + u], bf), sig[i + u]), g);
            dbv[u] = __fmul_rn(dv[i + u], sl[i + u]);
          }
          oa4[i >> 1] = bf16_pack2_rne(dav[0], dav[1]);
          ob4[i >> 1] = bf16_pack2_rne(dbv[0], dbv[1]);
        }
        *reinterpret_cast<uint4*>(gs[0] + r * kFbPitch + cc * 16) = make_uint4(oa4[0], oa4[1], oa4[2], oa4[3]);
        *reinterpret_cast<uint4*>(gs[1] + r * kFbPitch + cc * 16) = make_uint4(ob4[0], ob4[1], ob4[2], ob4[3]);
      }
    }
    // the next chunk's inputs (a chunk past the tile reads zero: empty resources)
    fb_load(in, dh, lddh, a, b, Fdim, t0, c0, ntok, ck + 1, rg, cc, col_ok);
    __syncthreads();
    // 2. row-facing SR: lane (tensor tid/256, row (tid/4)%64, block tid%4);
    // the tensor is uniform over each wave
    {
      const int k = tid >> 8, r = (tid >> 2) & 63, blk = tid & 3;
      const FbOut& o = __builtin_amdgcn_readfirstlane(k) ? ob : oa;       // wave-uniform
      const int64_t row = r0 + r, col0 = c0 + 32 * blk;
      const bool ok = r < nrow && 32 * blk < ncol;
      uint32_t w[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 d = *reinterpret_cast<const uint4*>(gs[k] + r * kFbPitch + blk * 64 + q * 16);
        w[4 * q] = d.x; w[4 * q + 1] = d.y; w[4 * q + 2] = d.z; w[4 * q + 3] = d.w;
      }
      uint32_t m = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) m = max(m, bf16_absmax8(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]));
      const int e = upward_exp(m << 16);
      const uint64_t blk0 = ((uint64_t)row * (uint64_t)Fdim + (uint64_t)col0) >> 2;   // first Philox counter
      uint32_t packed[4];
      sr_encode<16>(w, e, [&](int q, uint32_t* u) {
        u32x4 a, b;
        if constexpr (kIdx32) {
          a = sr_words32((uint32_t)blk0 + 2u * q, seed, o.offset);
          b = sr_words32((uint32_t)blk0 + 2u * q + 1u, seed, o.offset);
        } else {
          a = sr_words(blk0 + 2 * q, seed, o.offset);
          b = sr_words(blk0 + 2 * q + 1, seed, o.offset);
        }
        u[0] = a.x; u[1] = a.y; u[2] = a.z; u[3] = a.w; u[4] = b.x; u[5] = b.y; u[6] = b.z; u[7] = b.w;
      }, packed);
      if (ok) {
        *reinterpret_cast<uint4*>(o.codes + row * (Fdim >> 1) + (col0 >> 1)) =
            make_uint4(packed[0], packed[1], packed[2], packed[3]);
        o.scales[row * (Fdim >> 5) + (col0 >> 5)] = (uint8_t)(e + 127);
      }
    }
    // 3. column-facing H32: lane (tensor tid/256, column-in-pair (tid/128)%2,
    // token block (tid/64)%2, column pair tid%64); all but the pair index are
    // uniform over each wave
    {
      const int k = tid >> 8, c = (tid >> 7) & 1, tb = (tid >> 6) & 1, cp = tid & 63;
      if (32 * tb < nrow && 2 * cp < ncol) {
        // value i of column 2cp+c as fp32 with the fixed sign d_(i mod 16):
        // the low half by a shift and an add of the sign bit (adding bit 31
        // flips it), the high half by one and-xor; c is uniform over the wave
        float f[32];
        const uint8_t* src = gs[k] + (32 * tb) * kFbPitch + cp * 4;
        if (__builtin_amdgcn_readfirstlane(c) == 0) {
#pragma unroll
          for (int i = 0; i < 32; ++i) {
            const uint32_t v = *reinterpret_cast<const uint32_t*>(src + i * kFbPitch);
            f[i] = __uint_as_float((v << 16) + (((sign_mask16 >> (i & 15)) & 1u) << 31));
          }
        } else {
#pragma unroll
          for (int i = 0; i < 32; ++i) {
            const uint32_t v = *reinterpret_cast<const uint32_t*>(src + i * kFbPitch);
            f[i] = __uint_as_float((v & 0xFFFF0000u) ^ (((sign_mask16 >> (i & 15)) & 1u) << 31));
          }
        }
        h32_fp32(f);
        int e;
        const uint4 code = encode32_rtn(f, e);
        const int tblk = ck * (kFbChunk / 32) + tb;     // token block within the workgroup
        *reinterpret_cast<uint4*>(cs[k] + (2 * cp + c) * kFbCodePitch + tblk * 16) = code;
        ss[k][2 * cp + c][tblk] = (uint8_t)(e + 127);
      }
    }
    __syncthreads();
  }
  // 4. column codes out: piece p = (tensor, column, 16-byte piece); 8 lanes per column
#pragma unroll
  for (int pass = 0; pass < 2 * kFbCols * (kFbTok / 32) / kFbThreads; ++pass) {
    const int p = tid + kFbThreads * pass;
    const int k = p >> 10, col = (p >> 3) & 127, q = p & 7;
    if (col < ncol && 32 * q < ntok) {
      const FbOut& o = k ? ob : oa;
      *reinterpret_cast<uint4*>(o.codes_t + (c0 + col) * (T >> 1) + (t0 >> 1) + 16 * q) =
          *reinterpret_cast<const uint4*>(cs[k] + col * kFbCodePitch + 16 * q);
    }
  }
  if (tid < 2 * kFbCols) {
    const int k = tid >> 7, col = tid & 127;
    if (col < ncol) {
      const FbOut& o = k ? ob : oa;
      uint8_t* dst = o.scales_t + (c0 + col) * (T >> 5) + (t0 >> 5);
      for (int tb = 0; tb < ntok / 32; ++tb) dst[tb] = ss[k][col][tb];
    }
  }
}

}  // namespace mx

using namespace mx;

extern "C" fp4_status fp4_swiglu_backward(int64_t t, int64_t f, const float* dh, int64_t lddh,
                                          const uint16_t* a_bf16, const uint16_t* b_bf16, uint16_t* da_bf16,
                                          uint16_t* db_bf16, hipStream_t stream) {
  if (!mult32z(t) || !mult32z(f) || lddh < f) return FP4_ESHAPE;
  if (t == 0 || f == 0) return FP4_OK;
  if (!dh || !a_bf16 || !b_bf16 || !da_bf16 || !db_bf16) return FP4_EINVAL;
  if (!aligned16(dh) || !aligned16(a_bf16) || !aligned16(b_bf16) || !aligned16(da_bf16) || !aligned16(db_bf16) ||
      (lddh % 4) != 0)
    return FP4_EALIGN;
  const int64_t cpr = f >> 3;
  const int64_t gx = (cpr + kBwdThreads - 1) / kBwdThreads;
  if (gx > kMaxGridX) return FP4_ESHAPE;
  dim3 grid((unsigned)gx, (unsigned)(t < kMaxGridY ? t : kMaxGridY));
  hipLaunchKernelGGL(swiglu_bwd_kernel, grid, dim3(kBwdThreads), 0, as_stream(stream), t, f, dh, lddh, a_bf16,
                     b_bf16, da_bf16, db_bf16);
  return launch_status();
}

extern "C" fp4_status fp4_swiglu_backward_producer(
    int64_t t, int64_t f, const float* dh, int64_t lddh, const uint16_t* a_bf16, const uint16_t* b_bf16,
    uint64_t seed, uint64_t offset_a, uint64_t offset_b, uint32_t sign_mask16,
    uint8_t* da_codes, uint8_t* da_scales, uint8_t* db_codes, uint8_t* db_scales,
    uint8_t* dat_codes, uint8_t* dat_scales, uint8_t* dbt_codes, uint8_t* dbt_scales, hipStream_t stream) {
  if (!mult32z(t) || !mult32z(f) || lddh < f) return FP4_ESHAPE;
  if (t == 0 || f == 0) return FP4_OK;
  if (!dh || !a_bf16 || !b_bf16 || !da_codes || !da_scales || !db_codes || !db_scales || !dat_codes ||
      !dat_scales || !dbt_codes || !dbt_scales)
    return FP4_EINVAL;
  if (!aligned16(dh) || !aligned16(a_bf16) || !aligned16(b_bf16) || !aligned16(da_codes) ||
      !aligned16(db_codes) || !aligned16(dat_codes) || !aligned16(dbt_codes) || (lddh % 4) != 0)
    return FP4_EALIGN;
  const int64_t gx = (f + kFbCols - 1) / kFbCols, gy = (t + kFbTok - 1) / kFbTok;
  if (gy > kMaxGridY || gx > kMaxGridX || lddh >= (int64_t(1) << 23)) return FP4_ESHAPE;   // 32-bit buffer offsets
  const FbOut oa{da_codes, da_scales, dat_codes, dat_scales, offset_a};
  const FbOut ob{db_codes, db_scales, dbt_codes, dbt_scales, offset_b};
  if (t <= (int64_t(1) << 34) / f)                        // t * f <= 2^34: counters below 2^32
    hipLaunchKernelGGL(swiglu_bwd_producer_kernel<true>, dim3((unsigned)gx, (unsigned)gy), dim3(kFbThreads), 0,
                       as_stream(stream), t, f, dh, lddh, a_bf16, b_bf16, oa, ob, seed, sign_mask16 & 0xFFFFu);
  else
    hipLaunchKernelGGL(swiglu_bwd_producer_kernel<false>, dim3((unsigned)gx, (unsigned)gy), dim3(kFbThreads), 0,
                       as_stream(stream), t, f, dh, lddh, a_bf16, b_bf16, oa, ob, seed, sign_mask16 & 0xFFFFu);
  return launch_status();
}
