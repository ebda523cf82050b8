// W2 data gradient with the SwiGLU backward and the dA/dB producers in its
// epilogue ("Format-Aware Fusion for Fast FP4 Pretraining", §3.2: the gate's
// derivative is applied to the W2 Dgrad output within the fused backward step,
// which emits the operands of the W1/W3 Dgrad and Wgrad contractions; §3.1:
// a producer completes every layout its consumers read).
//
// One workgroup owns a 256-token x 256-column tile of dH = dec(dY_r) dec(W2_c)^T
// (the fast main loop of the GEMM, 8 waves).  The fp32 dH never leaves the
// chip: the epilogue takes the tile in two halves of 128 columns.  For each
// half
//   1. the four waves that hold the half's accumulators park them in LDS
//      (256 rows x 128 fp32, 16-byte chunks of 8 values XOR-swizzled by the
//      row's 32-token block so that the column reads of step 4 are
//      conflict-free);
//   2. every lane takes 8 columns x 8 rows: dH from LDS, the saved a, b from
//      HBM with coalesced 16-byte loads (the first four rows' issued before
//      the half's dH is staged), and writes dA and dB in bf16 over the dH
//      chunk it read (8 fp32 in, 8 + 8 bf16 out: the same 32 bytes);
//   3. row-facing SR of dA and dB (lane: one 32-column block of one row of one
//      tensor), with the Philox words of the element's row-major index in the
//      [t][f] tensor;
//   4. column-facing fixed-sign H32 of dA and dB (lane: one column pair x one
//      32-token block of one tensor); the eight token blocks of a column sit
//      in eight neighbouring lanes, so each store instruction writes whole
//      128-byte lines of column codes.
// The arithmetic of steps 2-4 is that of fp4_swiglu_backward followed by
// fp4_quantize_rows (SR) and fp4_quantize_cols (H32), and dH is the same fp32
// sum fp4_gemm computes (same main loop, same K order), so every output byte
// equals the unfused calls'.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "abi_common.h"
#include "gemm_core.h"
#include "mx_device.h"

namespace mx {

constexpr int kDbPitch = 528;                 // bytes per staged row: 128 fp32 + 16
constexpr int kDbRowsPerLane = 8;             // step 2: 256 rows x 16 chunks / 512 lanes
constexpr int kDbBatch = 4;                   // rows per batch of a, b loads
static_assert(256 * kDbPitch <= kSmemBytes, "a half tile of dH fits in the stage buffers");

struct DbOut {
  uint8_t* codes;                             // row-facing [t][f/2]
  uint8_t* scales;                            // [t][f/32]
  uint8_t* codes_t;                           // column-facing [f][t/2]
  uint8_t* scales_t;                          // [f][t/32]
  uint64_t offset;                            // SR counter offset
};

// Byte offset of 8-value chunk c8 (0..15) of staged row r: chunks are
// XOR-swizzled by the row's 32-token block.
__device__ __forceinline__ uint32_t db_chunk(int r, int c8) {
  return (uint32_t)(r * kDbPitch + 32 * (c8 ^ ((r >> 5) & 7)));
}

// Loads of the saved a, b for step 2 of half h: lane rows rg + 32k, 8 columns
// from 8*cc; rows past t read zero (buffer range), columns past f read values
// of the next row that no store uses.
struct DbAB {
  uint4 a[kDbBatch], b[kDbBatch];
};

// Rows rg + 32 (kb * kDbBatch + k), k < kDbBatch, of half h.
__device__ __forceinline__ void db_load_ab(DbAB& x, const uint16_t* a, const uint16_t* b, int64_t T, int64_t Fdim,
                                           int64_t m0, int64_t n0, int h, int kb, int rg, int cc) {
  const int64_t rows = std::min<int64_t>(256, T - m0);
  const int64_t c0 = n0 + 128 * h;
  const int64_t bytes = (rows - 1) * Fdim * 2 + std::min<int64_t>(128, Fdim - c0) * 2;
  const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(a + m0 * Fdim + c0, bytes);
  const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(b + m0 * Fdim + c0, bytes);
#pragma unroll
  for (int k = 0; k < kDbBatch; ++k) {
    const uint32_t off = (uint32_t)((rg + 32 * (kb * kDbBatch + k)) * Fdim * 2 + cc * 16);
    x.a[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0));
    x.b[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0));
  }
}

// Step 1: wave (wm, wn) with wn in {2h, 2h+1} parks its 128 x 64 accumulators.
__device__ __forceinline__ void db_stage_dh(uint8_t* smem, const v16f (&acc)[4][2], int wm, int wn, int h, int lane) {
  const int hl = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wm * 128 + 32 * i + (lane & 31);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = wn * 64 + 32 * j + 8 * g + 4 * hl - 128 * h;     // column within the half
        *reinterpret_cast<float4*>(smem + db_chunk(r, c >> 3) + 4 * (c & 7)) =
            make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
      }
  }
}

// Step 2: dA, dB of one 8-value chunk, fp32 dH in LDS -> bf16 in place.
__device__ __forceinline__ void db_backward_chunk(uint8_t* p, uint4 av, uint4 bv) {
  const float4 d0 = *reinterpret_cast<const float4*>(p);
  const float4 d1 = *reinterpret_cast<const float4*>(p + 16);
  const float dv[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
  const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
  const uint32_t bw[4] = {bv.x, bv.y, bv.z, bv.w};
  float afv[8], sig[8], sl[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) afv[i] = bf16_bits_to_f32((aw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
  sigmoid_silu_n<8>(afv, sig, sl);
  uint32_t oa[4], ob[4];
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
    oa[i >> 1] = bf16_pack2_rne(dav[0], dav[1]);
    ob[i >> 1] = bf16_pack2_rne(dbv[0], dbv[1]);
  }
  *reinterpret_cast<uint4*>(p) = make_uint4(oa[0], oa[1], oa[2], oa[3]);
  *reinterpret_cast<uint4*>(p + 16) = make_uint4(ob[0], ob[1], ob[2], ob[3]);
}

__global__ __launch_bounds__(kFastThreads) void dgrad_swiglu_bwd_kernel(
    int64_t T, int64_t Fdim, int64_t D, const uint8_t* __restrict__ dy_codes, const uint8_t* __restrict__ dy_scales,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, const uint16_t* __restrict__ a,
    const uint16_t* __restrict__ b, DbOut oa, DbOut ob, uint64_t seed, uint32_t sign_mask16) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
  int64_t tm, tn;
  tile_coords((T + BM - 1) / BM, (Fdim + BN - 1) / BN, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;
  Operand A{dy_codes, dy_scales, T}, B{w_codes, w_scales, Fdim};
  v16f acc[4][2];
  main_loop_fast<false>(smem, A, B, m0, n0, 0, D, acc, wm, wn);
  const int nrow = (int)std::min<int64_t>(256, T - m0);                 // multiple of 32
  const int cc = tid & 15, rg = tid >> 4;                                 // step 2 lane: chunk, first row
  const int nhalf = Fdim - n0 > 128 ? 2 : 1;                            // uniform
#pragma unroll 1
  for (int h = 0; h < nhalf; ++h) {
    const int64_t c0 = n0 + 128 * h;                                      // first column of the half
    const int ncol = (int)std::min<int64_t>(128, Fdim - c0);              // multiple of 32
    DbAB ab;
    db_load_ab(ab, a, b, T, Fdim, m0, n0, h, 0, rg, cc);
    // 1. park the half's dH (the barrier at the end of the previous half, or
    //    of the main loop, freed the buffer)
    if ((wn >> 1) == h) db_stage_dh(smem, acc, wm, wn, h, lane);
    __syncthreads();
    // 2. dA, dB in bf16 over the staged dH
#pragma unroll
    for (int kb = 0; kb < kDbRowsPerLane / kDbBatch; ++kb) {
      if (kb > 0) db_load_ab(ab, a, b, T, Fdim, m0, n0, h, kb, rg, cc);
#pragma unroll
      for (int k = 0; k < kDbBatch; ++k)
        db_backward_chunk(smem + db_chunk(rg + 32 * (kb * kDbBatch + k), cc), ab.a[k], ab.b[k]);
    }
    __syncthreads();
    // 3. row-facing SR: item (tensor, row, 32-column block), block fastest
#pragma unroll 1
    for (int p = 0; p < 4; ++p) {
      const int item = tid + 512 * p;
      const int blk = item & 3, r = (item >> 2) & 255, k = item >> 10;  // k uniform per pass
      const DbOut& o = k ? ob : oa;
      uint32_t w[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 d = *reinterpret_cast<const uint4*>(smem + db_chunk(r, 4 * blk + q) + 16 * k);
        w[4 * q] = d.x; w[4 * q + 1] = d.y; w[4 * q + 2] = d.z; w[4 * q + 3] = d.w;
      }
      uint32_t m = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) m = max(m, bf16_absmax8(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]));
      const int e = upward_exp(m << 16);
      const int64_t row = m0 + r, col0 = c0 + 32 * blk;
      const uint64_t blkc = ((uint64_t)row * (uint64_t)Fdim + (uint64_t)col0) >> 2;   // first Philox counter
      uint32_t packed[4];
      sr_encode<16>(w, e, [&](int q, uint32_t* u) {
        const u32x4 x = sr_words(blkc + 2 * q, seed, o.offset), y = sr_words(blkc + 2 * q + 1, seed, o.offset);
        u[0] = x.x; u[1] = x.y; u[2] = x.z; u[3] = x.w; u[4] = y.x; u[5] = y.y; u[6] = y.z; u[7] = y.w;
      }, packed);
      if (r < nrow && 32 * blk < ncol) {
        *reinterpret_cast<uint4*>(o.codes + row * (Fdim >> 1) + (col0 >> 1)) =
            make_uint4(packed[0], packed[1], packed[2], packed[3]);
        o.scales[row * (Fdim >> 5) + (col0 >> 5)] = (uint8_t)(e + 127);
      }
    }
    // 4. column-facing H32: item (tensor, column pair, token block), token
    //    block fastest
#pragma unroll 1
    for (int p = 0; p < 2; ++p) {
      const int item = tid + 512 * p;
      const int tb = item & 7, cp = (item >> 3) & 63, k = item >> 9;     // k uniform per pass
      const DbOut& o = k ? ob : oa;
      uint32_t v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i)
        v[i] = *reinterpret_cast<const uint32_t*>(smem + db_chunk(32 * tb + i, cp >> 2) + 16 * k + 4 * (cp & 3));
      const int64_t t0 = m0 + 32 * tb;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float f[32];
        h32_column(v, c, sign_mask16, f);
        h32_fp32(f);
        int e;
        const uint4 code = encode32_rtn(f, e);
        const int64_t col = c0 + 2 * cp + c;
        if (32 * tb < nrow && 2 * cp < ncol) {
          *reinterpret_cast<uint4*>(o.codes_t + col * (T >> 1) + (t0 >> 1)) = code;
          o.scales_t[col * (T >> 5) + (t0 >> 5)] = (uint8_t)(e + 127);
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace mx

using namespace mx;

extern "C" fp4_status fp4_gemm_swiglu_backward_producer(
    int64_t t, int64_t f, int64_t d, const uint8_t* dy_codes, const uint8_t* dy_scales, const uint8_t* w2c_codes,
    const uint8_t* w2c_scales, const uint16_t* a_bf16, const uint16_t* b_bf16, uint64_t seed, uint64_t offset_a,
    uint64_t offset_b, uint32_t sign_mask16, uint8_t* da_codes, uint8_t* da_scales, uint8_t* db_codes,
    uint8_t* db_scales, uint8_t* dat_codes, uint8_t* dat_scales, uint8_t* dbt_codes, uint8_t* dbt_scales,
    hipStream_t stream) {
  if (!mult32z(t) || !mult32z(f) || !mult32z(d)) return FP4_ESHAPE;
  if (t == 0 || f == 0) return FP4_OK;                                  // empty outputs
  if ((d % 256) != 0 || d == 0) return FP4_ESHAPE;                      // the fast main loop's K steps
  if (!dy_codes || !dy_scales || !w2c_codes || !w2c_scales || !a_bf16 || !b_bf16 || !da_codes || !da_scales ||
      !db_codes || !db_scales || !dat_codes || !dat_scales || !dbt_codes || !dbt_scales)
    return FP4_EINVAL;
  if (!aligned16(dy_codes) || !aligned16(dy_scales) || !aligned16(w2c_codes) || !aligned16(w2c_scales) ||
      !aligned16(a_bf16) || !aligned16(b_bf16) || !aligned16(da_codes) || !aligned16(db_codes) ||
      !aligned16(dat_codes) || !aligned16(dbt_codes))
    return FP4_EALIGN;
  // 32-bit buffer offsets: a 256-row panel of a, b and of the operands
  if (f >= ((int64_t)1 << 22) || d >= ((int64_t)1 << 24)) return FP4_ESHAPE;
  const int64_t tm = (t + BM - 1) / BM, tn = (f + BN - 1) / BN;
  if (tm > 0x7FFFFFFF / tn) return FP4_ESHAPE;
  const DbOut oa{da_codes, da_scales, dat_codes, dat_scales, offset_a};
  const DbOut ob{db_codes, db_scales, dbt_codes, dbt_scales, offset_b};
  hipLaunchKernelGGL(dgrad_swiglu_bwd_kernel, dim3((unsigned)(tm * tn)), dim3(kFastThreads), 0, as_stream(stream), t,
                     f, d, dy_codes, dy_scales, w2c_codes, w2c_scales, a_bf16, b_bf16, oa, ob, seed,
                     sign_mask16 & 0xFFFFu);
  return launch_status();
}
