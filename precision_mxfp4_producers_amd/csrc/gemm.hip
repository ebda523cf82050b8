// Block-scaled E2M1 GEMM on the gfx950 scaled MFMA, and the fused SwiGLU
// producer built on the same main loops.
//
// "Format-Aware Fusion for Fast FP4 Pretraining":
//   §2.3 (Eq. 4-6)  Fprop, Dgrad and Wgrad are all C = dec(A) dec(B)^T with
//                   both operands K-major and 1x32 E8M0 scales along K.
//   §3.2            the gated FFN pairs W1 and W3 and emits the SiLU-gated
//                   output directly as the FP4 input of W2.
//
// A workgroup owns a 256x256 output tile (256 tokens x 128 FFN columns for
// the SwiGLU producer, whose B tile holds the matching W1 and W3 rows) and
// walks K in steps of 256 values: 128 code bytes + 8 scale bytes per row.
// MFMA: v_mfma_scale_f32_32x32x64_f8f6f4 with both operands FP4 (E2M1) and
// E8M0 scales, fp32 accumulate.  A lane supplies 32 K-values of one row plus
// their scale byte; lanes 0-31 and 32-63 supply two different 32-blocks.
// Within a K step, lane half h takes blocks 4h..4h+3 for the four sub-steps,
// so each lane's four scale bytes are one aligned dword and the sub-step
// selects the byte (op_sel).  Applying the same block assignment to A and B
// leaves the sum over K unchanged.  B enters the instruction as its first
// operand and A as its second, so each 32x32 result is the transposed tile: a
// lane holds one row of C and, per group of four registers, four consecutive
// columns, which the epilogues write with 16- or 8-byte stores.
//
// Two main loops:
//   generic  (any K multiple of 32): 4 waves of 128x128, global -> registers
//            -> LDS with per-chunk predicates.
//   fast     (K % 256 == 0): 8 waves of 128x64, two per SIMD taking turns:
//            one issues a half step of MFMAs while the other reads its next
//            fragments, writes staged registers to LDS and issues raw buffer
//            loads (rows beyond M/N read as zero).
// Both stage tiles through the same LDS layout family: 128-byte rows whose
// 16-byte chunks are XOR-swizzled so that 16 consecutive rows read at one
// logical chunk hit 16 distinct bank groups.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "abi_common.h"
#include "gemm_core.h"
#include "mx_device.h"

namespace mx {

// ------------------------------------------------------------------ epilogues
// Result layout (operands entered as (B, A)): lane holds row (lane & 31) of A
// sub-tile i; registers 4g..4g+3 hold columns 8g + 4*(lane/32) + 0..3 of B
// sub-tile j.  `cols` is the tile-local first column of sub-tile j.
__device__ __forceinline__ void store_c_row(float* crow, const v16f& acc, int hl, bool accumulate) {
  float* p = crow + 4 * hl;
  if (accumulate) {
    float4 prev[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) prev[g] = *reinterpret_cast<const float4*>(p + 8 * g);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float4 v;
      v.x = __fadd_rn(prev[g].x, acc[4 * g]);
      v.y = __fadd_rn(prev[g].y, acc[4 * g + 1]);
      v.z = __fadd_rn(prev[g].z, acc[4 * g + 2]);
      v.w = __fadd_rn(prev[g].w, acc[4 * g + 3]);
      *reinterpret_cast<float4*>(p + 8 * g) = v;
    }
  } else {
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<float4*>(p + 8 * g) = make_float4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
  }
}

// SwiGLU: from the fp32 a (acc_a) and b (acc_b) of one row segment of four
// columns, save bf16 a and b and stage bf16 h = bf16(SiLU(a) * b) in LDS.
__device__ __forceinline__ void swiglu_quad(const v16f& acc_a, const v16f& acc_b, int g, uint8_t* hdst, uint16_t* adst,
                                            uint16_t* bdst, bool store) {
  uint32_t ab[4], bb[4], hb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    ab[u] = f32_to_bf16_rne(acc_a[4 * g + u]);
    bb[u] = f32_to_bf16_rne(acc_b[4 * g + u]);
    float sig, sl;
    sigmoid_silu(bf16_bits_to_f32(ab[u]), sig, sl);
    hb[u] = f32_to_bf16_rne(__fmul_rn(sl, bf16_bits_to_f32(bb[u])));
  }
  *reinterpret_cast<uint2*>(hdst) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
  if (store) {
    *reinterpret_cast<uint2*>(adst) = make_uint2(ab[0] | (ab[1] << 16), ab[2] | (ab[3] << 16));
    *reinterpret_cast<uint2*>(bdst) = make_uint2(bb[0] | (bb[1] << 16), bb[2] | (bb[3] << 16));
  }
}

// RTN MXFP4 of one 32-value bf16 block given as 16 packed words.
__device__ __forceinline__ uint4 encode_block_bf16(const uint32_t (&w)[16], int& e_out) {
  // largest 15-bit magnitude pattern: packed 16-bit maxima, one final pair
  u16x2_t mm = {0, 0};
#pragma unroll
  for (int j = 0; j < 16; ++j) mm = __builtin_elementwise_max(mm, __builtin_bit_cast(u16x2_t, w[j] & 0x7FFF7FFFu));
  const uint32_t m = max((uint32_t)mm[0], (uint32_t)mm[1]);
  const int e = upward_exp(m << 16);
  const float sc = pow2_scale(e);
  e_out = e;
  return make_uint4(rtn8_bf16(w[0], w[1], w[2], w[3], sc), rtn8_bf16(w[4], w[5], w[6], w[7], sc),
                    rtn8_bf16(w[8], w[9], w[10], w[11], sc), rtn8_bf16(w[12], w[13], w[14], w[15], sc));
}

// Quantize the staged 256 x 128 bf16 h tile: row-facing RTN (1024 blocks of
// 32 columns) and, if requested, column-facing with the fixed-sign H32 (128
// columns x 8 token blocks).  NT threads share the blocks.
template <int NT>
__device__ __forceinline__ void quantize_h_tile(const uint8_t* smem, int64_t m0, int64_t n0, int64_t T, int64_t Fdim,
                                                uint8_t* h_codes, uint8_t* h_scales, uint8_t* ht_codes,
                                                uint8_t* ht_scales, uint32_t sign_mask16) {
  const int tid = threadIdx.x;
  for (int b = tid; b < 1024; b += NT) {
    const int lr = b & 255, blk = b >> 8;
    const int64_t row = m0 + lr, col0 = n0 + 32 * blk;
    if (row >= T || col0 >= Fdim) continue;
    uint32_t wv[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 d = *reinterpret_cast<const uint4*>(smem + lr * kHPitch + blk * 64 + q * 16);
      wv[4 * q] = d.x; wv[4 * q + 1] = d.y; wv[4 * q + 2] = d.z; wv[4 * q + 3] = d.w;
    }
    int e;
    const uint4 code = encode_block_bf16(wv, e);
    *reinterpret_cast<uint4*>(h_codes + row * (Fdim >> 1) + (col0 >> 1)) = code;
    h_scales[row * (Fdim >> 5) + (col0 >> 5)] = (uint8_t)(e + 127);
  }
  if (ht_codes == nullptr) return;
  for (int b = tid; b < 512; b += NT) {
    const int cp = b & 63, tb = b >> 6;                  // columns 2cp, 2cp+1; tokens 32tb..
    const int64_t r0 = m0 + 32 * tb;
    if (r0 >= T) continue;
    uint32_t v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = *reinterpret_cast<const uint32_t*>(smem + (32 * tb + i) * kHPitch + cp * 4);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int64_t col = n0 + 2 * cp + c;
      if (col >= Fdim) continue;
      float fv[32];
      h32_column(v, c, sign_mask16, fv);
      h32_fp32(fv);
      int e;
      const uint4 code = encode32_rtn(fv, e);
      *reinterpret_cast<uint4*>(ht_codes + col * (T >> 1) + (r0 >> 1)) = code;
      ht_scales[col * (T >> 5) + (r0 >> 5)] = (uint8_t)(e + 127);
    }
  }
}

// ------------------------------------------------------------------ kernels
// C out through a private LDS slice per wave (LDS is free after the main
// loop): each 32x32 sub-tile is parked row-major (144-byte pitch: eight rows
// at one column land on distinct banks) and read back eight lanes per row, so
// every 16-byte store instruction writes eight whole 128-byte lines (a
// lane-per-row pattern leaves 32 partly written lines per instruction, which
// drains at about half the rate).  No workgroup barrier: waves stage and store
// independently.  Measured on 8192 x 14336 x 4096: the whole-tile staging with
// two workgroup-wide passes cost about 5 us per round of tiles.
constexpr int kCWPitch = 144;               // bytes per staged sub-tile row (128 + 16)
constexpr int kCWSlice = 32 * kCWPitch;     // bytes per wave
static_assert(8 * kCWSlice <= kSmemBytes, "C staging slices fit in the stage buffers");

__device__ __forceinline__ void store_c_tile_wave(uint8_t* smem, const v16f (&acc)[4][2], float* __restrict__ c,
                                                  int64_t ldc, int64_t M, int64_t N, int64_t m0, int64_t n0,
                                                  int wave, int lane, int wm, int wn, int hl, bool accumulate,
                                                  bool stream_c) {
  uint8_t* buf = smem + wave * kCWSlice;
  const int r = lane & 31, rr0 = lane >> 3, ch = lane & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row0 = m0 + wm * 128 + 32 * i;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col0 = n0 + wn * 64 + 32 * j;
      const v16f& a = acc[i][j];
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(buf + r * kCWPitch + (8 * g + 4 * hl) * 4) =
            make_float4(a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]);
      // the wave's LDS operations run in order: the reads see the writes, and
      // the next sub-tile's writes come after these reads
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int rr = rr0 + 8 * k;
        float4 v = *reinterpret_cast<const float4*>(buf + rr * kCWPitch + ch * 16);
        const int64_t row = row0 + rr;
        if (row < M && col0 < N) {                       // N % 32 == 0: the sub-tile's columns are all in
          float* p = c + row * ldc + col0 + 4 * ch;
          if (accumulate) {
            const float4 prev = *reinterpret_cast<const float4*>(p);
            v.x = __fadd_rn(prev.x, v.x);
            v.y = __fadd_rn(prev.y, v.y);
            v.z = __fadd_rn(prev.z, v.z);
            v.w = __fadd_rn(prev.w, v.w);
          }
          if (stream_c) __builtin_nontemporal_store(v4f{v.x, v.y, v.z, v.w}, reinterpret_cast<v4f*>(p));
          else *reinterpret_cast<float4*>(p) = v;
        }
      }
    }
  }
}

// SwiGLU producer epilogue for the 8-wave tile (256 tokens x 128 FFN columns;
// wave (wm, wn) holds a in sub-tile 0 and b in sub-tile 1 for FFN columns
// wn*32 ..).  LDS (free after the main loop) holds two staged bf16 tiles of
// 256 rows x kHPitch bytes: h in the first, a then b in the second.  Within a
// row, dword d sits at d ^ hswz(row) so that the column-pair reads of the H32
// pass (8 lanes per column pair, one per token block) hit distinct banks; the
// XOR moves whole 8-dword groups, so 16-byte chunks stay contiguous.
//   pass 1  a, b, h in bf16 (a and b are the rounded GEMM outputs)
//   pass 2  a out with whole-row stores; h row codes (4 lanes per row: 64
//           contiguous bytes); h column codes with H32 (8 lanes per column:
//           one whole 128-byte line)
//   pass 3  b through the same buffer as a
__device__ __forceinline__ int hswz(int row) { return ((row >> 5) & 7) << 3; }

__device__ __forceinline__ void swiglu_epilogue_staged(
    uint8_t* smem, const v16f (&acc)[4][2], int64_t T, int64_t Fdim, int64_t m0, int64_t n0, int wave, int lane,
    int wm, int wn, int hl, uint16_t* __restrict__ a_out, uint16_t* __restrict__ b_out,
    uint8_t* __restrict__ h_codes, uint8_t* __restrict__ h_scales, uint8_t* __restrict__ ht_codes,
    uint8_t* __restrict__ ht_scales, uint32_t sign_mask16) {
  uint8_t* hs = smem;
  uint8_t* as = smem + 256 * kHPitch;
  const int tid = threadIdx.x;
  uint32_t bpk[4][4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lr = wm * 128 + 32 * i + (lane & 31);
    // a and b of the lane's 16 columns of row lr in bf16, then SiLU of all 16
    // in one batch
    uint32_t ab[4][2], bb[4][2];
    float av[16], sg[16], sl[16];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        ab[g][u] = bf16_pack2_rne(acc[i][0][4 * g + 2 * u], acc[i][0][4 * g + 2 * u + 1]);
        bb[g][u] = bf16_pack2_rne(acc[i][1][4 * g + 2 * u], acc[i][1][4 * g + 2 * u + 1]);
        av[4 * g + 2 * u] = __uint_as_float(ab[g][u] << 16);
        av[4 * g + 2 * u + 1] = __uint_as_float(ab[g][u] & 0xFFFF0000u);
      }
    sigmoid_silu_n<16>(av, sg, sl);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dw = (wn * 32 + 8 * g + 4 * hl) >> 1;     // first dword of the lane's 4 columns
      uint32_t hb[2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
        hb[u] = bf16_pack2_rne(__fmul_rn(sl[4 * g + 2 * u], __uint_as_float(bb[g][u] << 16)),
                               __fmul_rn(sl[4 * g + 2 * u + 1], __uint_as_float(bb[g][u] & 0xFFFF0000u)));
      const int off = lr * kHPitch + 4 * (dw ^ hswz(lr));
      *reinterpret_cast<uint2*>(hs + off) = make_uint2(hb[0], hb[1]);
      *reinterpret_cast<uint2*>(as + off) = make_uint2(ab[g][0], ab[g][1]);
      bpk[i][g][0] = bb[g][0];
      bpk[i][g][1] = bb[g][1];
    }
  }
  __syncthreads();
  // a out: 16 lanes per row (256 bytes), 32 rows per pass of the workgroup
  const int ch = tid & 15;
#pragma unroll 4
  for (int p = 0; p < 8; ++p) {
    const int r = 32 * p + (tid >> 4);
    const int64_t row = m0 + r, col = n0 + 8 * ch;
    if (row < T && col < Fdim)
      __builtin_nontemporal_store(*reinterpret_cast<const v4i*>(as + r * kHPitch + 4 * ((4 * ch) ^ hswz(r))),
                                  reinterpret_cast<v4i*>(a_out + row * Fdim + col));
  }
  // h row codes: thread (row b/4, block b%4)
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int b = tid + 512 * k, lr = b >> 2, blk = b & 3;
    const int64_t row = m0 + lr, col0 = n0 + 32 * blk;
    uint32_t wv[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 d = *reinterpret_cast<const uint4*>(hs + lr * kHPitch + 4 * ((16 * blk + 4 * q) ^ hswz(lr)));
      wv[4 * q] = d.x; wv[4 * q + 1] = d.y; wv[4 * q + 2] = d.z; wv[4 * q + 3] = d.w;
    }
    int e;
    const uint4 code = encode_block_bf16(wv, e);
    if (row < T && col0 < Fdim) {
      *reinterpret_cast<uint4*>(h_codes + row * (Fdim >> 1) + (col0 >> 1)) = code;
      h_scales[row * (Fdim >> 5) + (col0 >> 5)] = (uint8_t)(e + 127);
    }
  }
  // h column codes with H32: thread (column pair tid/8, token block tid%8)
  if (ht_codes != nullptr) {
    const int cp = tid >> 3, tb = tid & 7;
    const int64_t r0 = m0 + 32 * tb;
    uint32_t v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = *reinterpret_cast<const uint32_t*>(hs + (32 * tb + i) * kHPitch + 4 * (cp ^ (tb << 3)));
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int64_t col = n0 + 2 * cp + c;
      float fv[32];
      h32_column(v, c, sign_mask16, fv);
      h32_fp32(fv);
      int e;
      const uint4 code = encode32_rtn(fv, e);
      if (r0 < T && col < Fdim) {
        __builtin_nontemporal_store(v4i{(int)code.x, (int)code.y, (int)code.z, (int)code.w},
                                    reinterpret_cast<v4i*>(ht_codes + col * (T >> 1) + (r0 >> 1)));
        ht_scales[col * (T >> 5) + (r0 >> 5)] = (uint8_t)(e + 127);
      }
    }
  }
  __syncthreads();
  // b through the a buffer
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lr = wm * 128 + 32 * i + (lane & 31);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dw = (wn * 32 + 8 * g + 4 * hl) >> 1;
      *reinterpret_cast<uint2*>(as + lr * kHPitch + 4 * (dw ^ hswz(lr))) = make_uint2(bpk[i][g][0], bpk[i][g][1]);
    }
  }
  __syncthreads();
#pragma unroll 4
  for (int p = 0; p < 8; ++p) {
    const int r = 32 * p + (tid >> 4);
    const int64_t row = m0 + r, col = n0 + 8 * ch;
    if (row < T && col < Fdim)
      __builtin_nontemporal_store(*reinterpret_cast<const v4i*>(as + r * kHPitch + 4 * ((4 * ch) ^ hswz(r))),
                                  reinterpret_cast<v4i*>(b_out + row * Fdim + col));
  }
}

__global__ __launch_bounds__(kGemmThreads) void gemm_generic_kernel(
    int64_t M, int64_t N, int64_t K, const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_scales, float* __restrict__ c, int64_t ldc,
    int accumulate) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
  int64_t tm, tn;
  tile_coords((M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1, hl = lane >> 5;
  Operand A{a_codes, a_scales, M}, B{b_codes, b_scales, N};
  v16f acc[4][4];
  main_loop_generic<false>(smem, smem + kStageBytes, A, B, m0, n0, 0, K, acc, wm, wn);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = m0 + wm * 128 + 32 * i + (lane & 31);
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn * 128 + 32 * j;
      if (col < N) store_c_row(c + row * ldc + col, acc[i][j], hl, accumulate != 0);
    }
  }
}

// One product of a launch: C (+)= A B^T, or with a2c set C (+)= A B^T + A2 B2^T
// as one fp32 accumulation over both K ranges (each K long).  `flags`: bit 0
// accumulate, bit 1 write C with non-temporal (streaming) stores.
struct GemmJob {
  const uint8_t* ac;
  const uint8_t* as;
  const uint8_t* bc;
  const uint8_t* bs;
  const uint8_t* a2c;
  const uint8_t* a2s;
  const uint8_t* b2c;
  const uint8_t* b2s;
  float* c;
  int64_t M, N, K, ldc;
  int64_t tiles;                            // 256 x 256 output tiles of this product
  int flags;
};
constexpr int kMaxGemmJobs = 4;
struct GemmGroup {
  GemmJob job[kMaxGemmJobs];
  int count;
};

// Up to kMaxGemmJobs independent products in one launch: job q owns the
// workgroups after those of jobs 0 .. q-1, and the workgroup dispatcher hands
// them out in that order, so a job that leaves the last round of tiles part
// empty is followed at once by the next job's tiles on the idle CUs.  Every
// tile runs the same loop and epilogue as in a launch of its own.
__global__ __launch_bounds__(kFastThreads) void gemm_fast_kernel(const GemmGroup g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
  GemmJob J = g.job[0];
  int64_t pid = blockIdx.x;
#pragma unroll
  for (int q = 1; q < kMaxGemmJobs; ++q) {
    if (q < g.count && pid >= J.tiles) {
      pid -= J.tiles;
      J = g.job[q];
    }
  }
  int64_t tm, tn;
  tile_coords_of(pid, J.tiles, (J.M + BM - 1) / BM, (J.N + BN - 1) / BN, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 2, wn = wave & 3, hl = lane >> 5;
  Operand A{J.ac, J.as, J.M}, B{J.bc, J.bs, J.N};
  Operand A2{J.a2c, J.a2s, J.M}, B2{J.b2c, J.b2s, J.N};
  v16f acc[4][2];
  main_loop_fast<false>(smem, A, B, m0, n0, 0, J.K, acc, wm, wn, &A2, &B2);
  store_c_tile_wave(smem, acc, J.c, J.ldc, J.M, J.N, m0, n0, wave, lane, wm, wn, hl, (J.flags & 1) != 0,
                    (J.flags & 2) != 0);
}

// SwiGLU producer output tile: 256 tokens x 128 FFN columns.
__global__ __launch_bounds__(kGemmThreads) void swiglu_generic_kernel(
    int64_t T, int64_t Fdim, int64_t D, const uint8_t* __restrict__ x_codes, const uint8_t* __restrict__ x_scales,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, uint16_t* __restrict__ a_out,
    uint16_t* __restrict__ b_out, uint8_t* __restrict__ h_codes, uint8_t* __restrict__ h_scales,
    uint8_t* __restrict__ ht_codes, uint8_t* __restrict__ ht_scales, uint32_t sign_mask16) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
  int64_t tm, tn;
  tile_coords((T + BM - 1) / BM, (Fdim + 127) / 128, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * 128;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1, hl = lane >> 5;
  Operand A{x_codes, x_scales, T}, B{w_codes, w_scales, 2 * Fdim};
  v16f acc[4][4];
  main_loop_generic<true>(smem, smem + kStageBytes, A, B, m0, n0, Fdim, D, acc, wm, wn);
  // wave (wm, wn): a in sub-tiles j = 0, 1 and b in j + 2, FFN columns wn*64 + 32j ..
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lr = wm * 128 + 32 * i + (lane & 31);
    const int64_t row = m0 + lr;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int lc = wn * 64 + 32 * j + 8 * g + 4 * hl;
        const int64_t col = n0 + lc;
        swiglu_quad(acc[i][j], acc[i][j + 2], g, smem + lr * kHPitch + lc * 2, a_out + row * Fdim + col,
                    b_out + row * Fdim + col, row < T && col < Fdim);
      }
  }
  __syncthreads();
  quantize_h_tile<kGemmThreads>(smem, m0, n0, T, Fdim, h_codes, h_scales, ht_codes, ht_scales, sign_mask16);
}

__global__ __launch_bounds__(kFastThreads) void swiglu_fast_kernel(
    int64_t T, int64_t Fdim, int64_t D, const uint8_t* __restrict__ x_codes, const uint8_t* __restrict__ x_scales,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, uint16_t* __restrict__ a_out,
    uint16_t* __restrict__ b_out, uint8_t* __restrict__ h_codes, uint8_t* __restrict__ h_scales,
    uint8_t* __restrict__ ht_codes, uint8_t* __restrict__ ht_scales, uint32_t sign_mask16) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
  int64_t tm, tn;
  tile_coords((T + BM - 1) / BM, (Fdim + 127) / 128, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * 128;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 2, wn = wave & 3, hl = lane >> 5;
  Operand A{x_codes, x_scales, T}, B{w_codes, w_scales, 2 * Fdim};
  v16f acc[4][2];
  main_loop_fast<true>(smem, A, B, m0, n0, Fdim, D, acc, wm, wn);
  swiglu_epilogue_staged(smem, acc, T, Fdim, m0, n0, wave, lane, wm, wn, hl, a_out, b_out, h_codes, h_scales,
                         ht_codes, ht_scales, sign_mask16);
}

// A contraction with K = 0 (every sum empty) writes zeros; a plain kernel
// rather than a memset so that the call stays capturable in graphs.
__global__ __launch_bounds__(256) void fill_rows_f32_kernel(float* __restrict__ c, int64_t m, int64_t n, int64_t ldc) {
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (col >= n) return;
  for (int64_t r = blockIdx.y; r < m; r += gridDim.y) c[r * ldc + col] = 0.0f;
}

}  // namespace mx

using namespace mx;

// Kernel flags of the fast GEMM: accumulate, and streaming (non-temporal) C
// stores when C is larger than three quarters of the 256 MB Infinity Cache.
// Such an output cannot stay cached for its reader anyway, and written
// through the cache it evicts the operands of the next launches (same-box
// A/B over the FFN step: the 235 and 470 MB Wgrad and Dgrad outputs gained
// 5-15 us each, and the kernels after them too; the 134 MB outputs lost
// about 7 us each, so they keep ordinary stores).
// Number of (bm x bn) output tiles of an m x n result, or -1 when it exceeds
// the 2^31 - 1 workgroups of a one-dimensional grid (checked before the
// product, which could overflow int64 for huge m, n).
static int64_t grid_tiles(int64_t m, int64_t bm, int64_t n, int64_t bn) {
  const int64_t tm = (m + bm - 1) / bm, tn = (n + bn - 1) / bn;
  if (tm == 0 || tn == 0) return 0;
  if (tm > 0x7FFFFFFF / tn) return -1;
  return tm * tn;
}

static int fast_flags(int64_t m, int64_t n, int accumulate) {
  constexpr int64_t kStreamCBytes = (int64_t)192 << 20;
  return accumulate | (m * n * 4 > kStreamCBytes ? 2 : 0);
}

// The fast kernel needs K % 256 == 0 and buffer offsets below 2^31 per tile.
static bool fast_k(int64_t k) { return k > 0 && (k % 256) == 0 && 256 * (k / 2) < 0x7FFFFFFF; }

static GemmJob make_job(const fp4_gemm_problem& p, int64_t tiles) {
  GemmJob j{};
  j.ac = p.a_codes;
  j.as = p.a_scales;
  j.bc = p.b_codes;
  j.bs = p.b_scales;
  j.a2c = p.a2_codes;
  j.a2s = p.a2_scales;
  j.b2c = p.b2_codes;
  j.b2s = p.b2_scales;
  j.c = p.c;
  j.M = p.m;
  j.N = p.n;
  j.K = p.k;
  j.ldc = p.ldc;
  j.tiles = tiles;
  j.flags = fast_flags(p.m, p.n, p.accumulate);
  return j;
}

// Argument checks of one product (plain or pair form); `tiles` gets its
// number of 256 x 256 output tiles (0 when C is empty).
static fp4_status check_problem(const fp4_gemm_problem& p, int64_t& tiles) {
  tiles = 0;
  if (p.accumulate != 0 && p.accumulate != 1) return FP4_EINVAL;
  if (!mult32z(p.m) || !mult32z(p.n) || !mult32z(p.k) || p.ldc < p.n) return FP4_ESHAPE;
  if (p.m == 0 || p.n == 0) return FP4_OK;                // empty C
  if (!p.c) return FP4_EINVAL;
  if (p.k == 0) {                                         // C = 0, or unchanged when accumulating
    if (!p.accumulate && (p.n + 255) / 256 > 0x7FFFFFFF) return FP4_ESHAPE;
    return FP4_OK;
  }
  const bool pair = p.a2_codes || p.a2_scales || p.b2_codes || p.b2_scales;
  if (!p.a_codes || !p.a_scales || !p.b_codes || !p.b_scales) return FP4_EINVAL;
  if (pair && !(p.a2_codes && p.a2_scales && p.b2_codes && p.b2_scales)) return FP4_EINVAL;
  if (!aligned16(p.a_codes) || !aligned16(p.b_codes) || !aligned16(p.a_scales) || !aligned16(p.b_scales) ||
      !aligned16(p.c) || (p.ldc % 4) != 0)
    return FP4_EALIGN;
  if (pair && (!aligned16(p.a2_codes) || !aligned16(p.b2_codes) || !aligned16(p.a2_scales) ||
               !aligned16(p.b2_scales)))
    return FP4_EALIGN;
  tiles = grid_tiles(p.m, BM, p.n, BN);
  if (tiles < 0) return FP4_ESHAPE;
  return FP4_OK;
}

static fp4_status launch_fast(const GemmGroup& g, int64_t total_tiles, hipStream_t s) {
  hipLaunchKernelGGL(gemm_fast_kernel, dim3((unsigned)total_tiles), dim3(kFastThreads), 0, s, g);
  return launch_status();
}

// One checked product on its own: the fill kernel for K = 0, the fast kernel,
// or the generic kernel(s).
static fp4_status run_problem(const fp4_gemm_problem& p, int64_t tiles, hipStream_t s) {
  if (p.m == 0 || p.n == 0) return FP4_OK;
  if (p.k == 0) {
    if (p.accumulate) return FP4_OK;
    const int64_t gx = (p.n + 255) / 256, gy = std::min<int64_t>(p.m, 65535);
    hipLaunchKernelGGL(fill_rows_f32_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s, p.c, p.m, p.n,
                       p.ldc);
    return launch_status();
  }
  if (fast_k(p.k)) {
    GemmGroup g{};
    g.job[0] = make_job(p, tiles);
    g.count = 1;
    return launch_fast(g, tiles, s);
  }
  hipLaunchKernelGGL(gemm_generic_kernel, dim3((unsigned)tiles), dim3(kGemmThreads), 0, s, p.m, p.n, p.k,
                     p.a_codes, p.a_scales, p.b_codes, p.b_scales, p.c, p.ldc, p.accumulate);
  fp4_status st = launch_status();
  if (st != FP4_OK || !p.a2_codes) return st;
  // pair form with K not a multiple of 256: the second product is added to the first's result
  hipLaunchKernelGGL(gemm_generic_kernel, dim3((unsigned)tiles), dim3(kGemmThreads), 0, s, p.m, p.n, p.k,
                     p.a2_codes, p.a2_scales, p.b2_codes, p.b2_scales, p.c, p.ldc, 1);
  return launch_status();
}

extern "C" {

fp4_status fp4_gemm(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes, const uint8_t* a_scales,
                    const uint8_t* b_codes, const uint8_t* b_scales, float* c, int64_t ldc, int accumulate,
                    hipStream_t stream) {
  const fp4_gemm_problem p{m, n, k, a_codes, a_scales, b_codes, b_scales, nullptr, nullptr, nullptr, nullptr,
                           c, ldc, accumulate};
  int64_t tiles;
  const fp4_status st = check_problem(p, tiles);
  if (st != FP4_OK) return st;
  return run_problem(p, tiles, as_stream(stream));
}

fp4_status fp4_gemm_pair(int64_t m, int64_t n, int64_t k, const uint8_t* a1_codes, const uint8_t* a1_scales,
                         const uint8_t* b1_codes, const uint8_t* b1_scales, const uint8_t* a2_codes,
                         const uint8_t* a2_scales, const uint8_t* b2_codes, const uint8_t* b2_scales, float* c,
                         int64_t ldc, int accumulate, hipStream_t stream) {
  // with all four second operands NULL the checks below would take the plain
  // form; here that is a missing operand
  if (!a2_codes && !a2_scales && !b2_codes && !b2_scales && mult32z(m) && mult32z(n) && mult32z(k) && k > 0 &&
      ldc >= n && m > 0 && n > 0)
    return FP4_EINVAL;
  const fp4_gemm_problem p{m, n, k, a1_codes, a1_scales, b1_codes, b1_scales, a2_codes, a2_scales, b2_codes,
                           b2_scales, c, ldc, accumulate};
  int64_t tiles;
  const fp4_status st = check_problem(p, tiles);
  if (st != FP4_OK) return st;
  return run_problem(p, tiles, as_stream(stream));
}

fp4_status fp4_gemm_grouped(const fp4_gemm_problem* problems, int count, hipStream_t stream) {
  if (count < 0 || count > FP4_GEMM_GROUP_MAX) return FP4_EINVAL;
  if (count == 0) return FP4_OK;
  if (!problems) return FP4_EINVAL;
  int64_t tiles[FP4_GEMM_GROUP_MAX];
  int64_t total = 0;
  for (int q = 0; q < count; ++q) {
    const fp4_status st = check_problem(problems[q], tiles[q]);
    if (st != FP4_OK) return st;
    if (fast_k(problems[q].k)) total += tiles[q];
  }
  if (total > 0x7FFFFFFF) return FP4_ESHAPE;
  hipStream_t s = as_stream(stream);
  // the shared launch: longest K per tile first (pair form: both K ranges)
  int order[FP4_GEMM_GROUP_MAX];
  int nfast = 0;
  for (int q = 0; q < count; ++q)
    if (fast_k(problems[q].k) && tiles[q] > 0) order[nfast++] = q;
  auto steps = [&](int q) { return problems[q].k * (problems[q].a2_codes ? 2 : 1); };
  for (int i = 1; i < nfast; ++i)                         // stable insertion sort, descending
    for (int j = i; j > 0 && steps(order[j]) > steps(order[j - 1]); --j) std::swap(order[j], order[j - 1]);
  if (nfast > 0) {
    GemmGroup g{};
    for (int i = 0; i < nfast; ++i) g.job[i] = make_job(problems[order[i]], tiles[order[i]]);
    g.count = nfast;
    const fp4_status st = launch_fast(g, total, s);
    if (st != FP4_OK) return st;
  }
  for (int q = 0; q < count; ++q) {
    if (fast_k(problems[q].k)) continue;
    const fp4_status st = run_problem(problems[q], tiles[q], s);
    if (st != FP4_OK) return st;
  }
  return FP4_OK;
}

fp4_status fp4_swiglu_producer(int64_t t, int64_t f, int64_t d, const uint8_t* x_codes, const uint8_t* x_scales,
                               const uint8_t* w13_codes, const uint8_t* w13_scales, uint16_t* a_bf16,
                               uint16_t* b_bf16, uint8_t* h_codes, uint8_t* h_scales, uint8_t* ht_codes,
                               uint8_t* ht_scales, uint32_t sign_mask16, hipStream_t stream) {
  if ((ht_codes == nullptr) != (ht_scales == nullptr)) return FP4_EINVAL;
  if (!mult32z(t) || !mult32z(f) || !mult32z(d)) return FP4_ESHAPE;
  if (t == 0 || f == 0) return FP4_OK;                    // empty outputs
  if (!a_bf16 || !b_bf16 || !h_codes || !h_scales) return FP4_EINVAL;
  // d = 0 (empty sums) runs the ordinary kernel: its operand loads go through
  // empty buffer resources and read zero, and the epilogue then produces the
  // definition (a = b = +0, h = +0; the H32 signs still decide the sign of
  // each transformed zero)
  if (d > 0 && (!x_codes || !x_scales || !w13_codes || !w13_scales)) return FP4_EINVAL;
  if (!aligned16(x_codes) || !aligned16(w13_codes) || !aligned16(h_codes) || !aligned16(x_scales) ||
      !aligned16(w13_scales) || !aligned16(a_bf16) || !aligned16(b_bf16) || (ht_codes && !aligned16(ht_codes)))
    return FP4_EALIGN;
  const int64_t tiles = grid_tiles(t, BM, f, 128);
  if (tiles < 0) return FP4_ESHAPE;
  hipStream_t s = as_stream(stream);
  if ((d % 256) == 0 && 256 * (d / 2) < 0x7FFFFFFF)
    hipLaunchKernelGGL(swiglu_fast_kernel, dim3((unsigned)tiles), dim3(kFastThreads), 0, s, t, f, d, x_codes, x_scales,
                       w13_codes, w13_scales, a_bf16, b_bf16, h_codes, h_scales, ht_codes, ht_scales,
                       sign_mask16 & 0xFFFFu);
  else
    hipLaunchKernelGGL(swiglu_generic_kernel, dim3((unsigned)tiles), dim3(kGemmThreads), 0, s, t, f, d, x_codes,
                       x_scales, w13_codes, w13_scales, a_bf16, b_bf16, h_codes, h_scales, ht_codes, ht_scales,
                       sign_mask16 & 0xFFFFu);
  return launch_status();
}

}  // extern "C"
