// Block-scaled E2M1 GEMM core shared by the GEMM, the SwiGLU producer and
// the Dgrad + SwiGLU-backward producer: LDS layout, operand staging, the
// generic and the fast (ping-pong) main loops, and the tile order; each loop's
// schedule is described beside it.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>

#include "mx_device.h"

namespace mx {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256;
constexpr int BKB = 128;                    // code bytes per row per K step (256 values)
constexpr int kGemmThreads = 256;           // generic path
constexpr int kFastThreads = 512;           // fast path
constexpr int kStageBytes = BM * BKB + BN * BKB + BM * 8 + BN * 8;    // 69632
constexpr int kSmemBytes = 2 * kStageBytes;                            // 139264
constexpr int kHPitch = 272;                // bytes per row of the staged h tile (256 + 16)
static_assert(2 * 256 * kHPitch <= kSmemBytes, "h and a/b tiles fit in the stage buffers");

__device__ __forceinline__ int swz(int row, int chunk) {
  return chunk ^ ((row & 7) ^ ((row >> 3) & 1));
}

struct Operand {
  const uint8_t* codes;     // [rows][K/2]
  const uint8_t* scales;    // [rows][K/32]
  int64_t rows;
};

// Global row of LDS row `lr` of the B tile: plain GEMM maps n0 + lr; the SwiGLU
// producer maps LDS rows 0..127 to W1 rows n0.. and 128..255 to W3 rows f+n0..
template <bool kSwiGLU>
__device__ __forceinline__ int64_t b_global_row(int lr, int64_t n0, int64_t f, bool& ok, int64_t nrows) {
  if constexpr (kSwiGLU) {
    const int64_t col = n0 + (lr & 127);
    ok = col < f;
    return (lr < 128) ? col : f + col;
  } else {
    const int64_t g = n0 + lr;
    ok = g < nrows;
    return g;
  }
}

// LDS row base of B sub-tile j for wave column wn.
template <bool kSwiGLU>
__device__ __forceinline__ int b_sub_row(int wn, int j) {
  if constexpr (kSwiGLU) return (j < 2) ? (wn * 64 + 32 * j) : (128 + wn * 64 + 32 * (j - 2));
  else return wn * 128 + 32 * j;
}

struct Staged {
  uint4 a[8], b[8];
  uint2 sa, sb;
};

template <bool kSwiGLU>
__device__ __forceinline__ void load_stage(Staged& st, const Operand& A, const Operand& B, int64_t m0,
                                           int64_t n0, int64_t f, int64_t K, int kit, bool k_full,
                                           bool vec_scales) {
  const int t = threadIdx.x;
  const int64_t kb0 = (int64_t)kit * BKB;              // byte offset along K
  const int64_t ldb = K >> 1, lds_ = K >> 5;
  const int c = t & 7;
  const bool chunk_ok = k_full || (kb0 + c * 16 < ldb);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = (t >> 3) + 32 * j;
    const int64_t ga = m0 + row;
    uint4 va = make_uint4(0u, 0u, 0u, 0u);
    if (ga < A.rows && chunk_ok) va = *reinterpret_cast<const uint4*>(A.codes + ga * ldb + kb0 + c * 16);
    st.a[j] = va;
    bool okb;
    const int64_t gb = b_global_row<kSwiGLU>(row, n0, f, okb, B.rows);
    uint4 vb = make_uint4(0u, 0u, 0u, 0u);
    if (okb && chunk_ok) vb = *reinterpret_cast<const uint4*>(B.codes + gb * ldb + kb0 + c * 16);
    st.b[j] = vb;
  }
  // scales: lane t owns row t of each operand, 8 bytes per K step
  const int64_t sb0 = (int64_t)kit * 8;
  {
    const int64_t ga = m0 + t;
    bool okb;
    const int64_t gb = b_global_row<kSwiGLU>(t, n0, f, okb, B.rows);
    if (vec_scales) {                                    // K % 256 == 0: rows 8-byte aligned
      st.sa = ga < A.rows ? *reinterpret_cast<const uint2*>(A.scales + ga * lds_ + sb0) : make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
      st.sb = okb ? *reinterpret_cast<const uint2*>(B.scales + gb * lds_ + sb0) : make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
    } else {
      uint32_t w[2][2] = {{0u, 0u}, {0u, 0u}};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const bool kok = sb0 + q < lds_;
        const uint32_t va = (ga < A.rows && kok) ? A.scales[ga * lds_ + sb0 + q] : 0x7Fu;
        const uint32_t vb = (okb && kok) ? B.scales[gb * lds_ + sb0 + q] : 0x7Fu;
        w[0][q >> 2] |= va << (8 * (q & 3));
        w[1][q >> 2] |= vb << (8 * (q & 3));
      }
      st.sa = make_uint2(w[0][0], w[0][1]);
      st.sb = make_uint2(w[1][0], w[1][1]);
    }
  }
}

__device__ __forceinline__ void store_stage(const Staged& st, uint8_t* stage) {
  const int t = threadIdx.x;
  uint8_t* la = stage;
  uint8_t* lb = stage + BM * BKB;
  uint32_t* lsa = reinterpret_cast<uint32_t*>(stage + BM * BKB + BN * BKB);
  uint32_t* lsb = lsa + BM * 2;
  const int c = t & 7;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = (t >> 3) + 32 * j;
    *reinterpret_cast<uint4*>(la + row * BKB + swz(row, c) * 16) = st.a[j];
    *reinterpret_cast<uint4*>(lb + row * BKB + swz(row, c) * 16) = st.b[j];
  }
  *reinterpret_cast<uint2*>(lsa + 2 * t) = st.sa;
  *reinterpret_cast<uint2*>(lsb + 2 * t) = st.sb;
}

__device__ __forceinline__ v8i widen(v4i x) {
  v8i r = {x[0], x[1], x[2], x[3], 0, 0, 0, 0};
  return r;
}

// One 64-value sub-step: op_sel S picks byte S of each lane's scale dword.
template <bool kSwiGLU, int S>
__device__ __forceinline__ void compute_substep(const uint8_t* la, const uint8_t* lb, const uint32_t (&sa)[4],
                                                const uint32_t (&sb)[4], v16f (&acc)[4][4], int wm, int wn,
                                                int r, int h) {
  const int c = 4 * h + S;
  v4i af[4], bf[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = wm * 128 + 32 * i + r;
    af[i] = *reinterpret_cast<const v4i*>(la + row * BKB + swz(row, c) * 16);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = b_sub_row<kSwiGLU>(wn, j) + r;
    bf[j] = *reinterpret_cast<const v4i*>(lb + row * BKB + swz(row, c) * 16);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          widen(bf[j]), widen(af[i]), acc[i][j], 4, 4, S, (int)sb[j], S, (int)sa[i]);
    }
  }
}

template <bool kSwiGLU>
__device__ __forceinline__ void compute_stage(const uint8_t* stage, v16f (&acc)[4][4], int wm, int wn) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 31, h = lane >> 5;
  const uint8_t* la = stage;
  const uint8_t* lb = stage + BM * BKB;
  const uint32_t* lsa = reinterpret_cast<const uint32_t*>(stage + BM * BKB + BN * BKB);
  const uint32_t* lsb = lsa + BM * 2;
  uint32_t sa[4], sb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = wm * 128 + 32 * i + r;
    sa[i] = lsa[2 * row + h];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = b_sub_row<kSwiGLU>(wn, j) + r;
    sb[j] = lsb[2 * row + h];
  }
  compute_substep<kSwiGLU, 0>(la, lb, sa, sb, acc, wm, wn, r, h);
  compute_substep<kSwiGLU, 1>(la, lb, sa, sb, acc, wm, wn, r, h);
  compute_substep<kSwiGLU, 2>(la, lb, sa, sb, acc, wm, wn, r, h);
  compute_substep<kSwiGLU, 3>(la, lb, sa, sb, acc, wm, wn, r, h);
}

// Tile order: XCD-aware (the hardware deals workgroups round-robin to 8 XCDs;
// remap so that consecutive logical tiles share an XCD and its L2), then
// grouped along M so neighbouring tiles reuse A rows and B columns.  `pid` is
// the workgroup's index among the `num` workgroups of its product.
__device__ __forceinline__ void tile_coords_of(int64_t pid, int64_t num, int64_t tiles_m, int64_t tiles_n,
                                               int64_t& tm, int64_t& tn) {
  if ((num & 7) == 0) pid = (pid & 7) * (num >> 3) + (pid >> 3);
  const int64_t GM = 8;
  const int64_t width = GM * tiles_n;
  const int64_t group = pid / width;
  const int64_t first_m = group * GM;
  const int64_t gsz = min(tiles_m - first_m, GM);
  const int64_t in_group = pid - group * width;
  tm = first_m + in_group % gsz;
  tn = in_group / gsz;
}

__device__ __forceinline__ void tile_coords(int64_t tiles_m, int64_t tiles_n, int64_t& tm, int64_t& tn) {
  tile_coords_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
}

// Generic main loop (any K that is a multiple of 32): global -> registers ->
// LDS staging with per-chunk predicates.
template <bool kSwiGLU>
__device__ __forceinline__ void main_loop_generic(uint8_t* buf0, uint8_t* buf1, const Operand& A,
                                                  const Operand& B, int64_t m0, int64_t n0, int64_t f, int64_t K,
                                                  v16f (&acc)[4][4], int wm, int wn) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
  const int nk = (int)((K + 255) / 256);
  const bool all_full = (K & 255) == 0;
  Staged st;
  load_stage<kSwiGLU>(st, A, B, m0, n0, f, K, 0, all_full || nk > 1, all_full);
  store_stage(st, buf0);
  __syncthreads();
  for (int it = 0; it < nk; ++it) {
    const bool more = it + 1 < nk;
    if (more) load_stage<kSwiGLU>(st, A, B, m0, n0, f, K, it + 1, all_full || it + 2 < nk, all_full);
    compute_stage<kSwiGLU>((it & 1) ? buf1 : buf0, acc, wm, wn);
    if (more) store_stage(st, (it & 1) ? buf0 : buf1);
    __syncthreads();
  }
}


// ------------------------------------------------------------------ fast main loop
// K % 256 == 0.  LDS holds two K-256 stages, stage-major per operand:
//   A[2] 32 KB each (256 rows x 128 B) | B[2] | SA[2] 2 KB (256 rows x 8 B) | SB[2]
// The two waves on a SIMD (w and w + 4) take turns: while one issues the 16
// MFMAs of a half K step (two 64-deep sub-steps) back to back, the other does
// its memory work -- reads its fragments for its next half step, writes its
// share of a later stage from registers to LDS, and issues the global loads of
// the stage after that.  Group 0 (waves 0-3, tile rows 0-127) computes in the
// even phases of the global numbering, group 1 (rows 128-255) in the odd ones.
// Per K step s (phases 4s .. 4s+3) and wave, its share of a stage is an A part
// (4 code loads) and a B part (4 code loads + its scale rows):
//   phase  group 0                               group 1
//   4s     half 0 of s                           frags half 0 of s; write A of s+1; load A of s+2
//   4s+1   frags half 1 of s; write B of s+1;    half 0 of s
//          load B of s+2
//   4s+2   half 1 of s                           frags half 1 of s; write B of s+1; load B of s+2
//   4s+3   frags half 0 of s+1; write A of s+2;  half 1 of s
//          load A of s+3
// One workgroup barrier per K step, at the end of phase 4s+2, covers every
// LDS hazard: stage s+1 is written in phases 4s-1 .. 4s+2 and first read in
// 4s+3; stage s (the buffer that A of s+2 overwrites in 4s+3) is last read in
// 4s+2; stage s-1 (the buffer of s+1) is last read in 4s-2, before the
// previous barrier.  The barrier also pulls the groups back into opposite
// phases once per step.  A part is loaded four phases before it is written;
// loads past the last step are clamped to it and land in a buffer nobody reads
// again.
//
// Measured alternatives (one MI355X, 8192 x 4096 x 14336, random codes):
//   - the same schedule with a barrier at every phase end: 293 us; every
//     other phase: 283 us; once per step (this loop): 273 us;
//   - all eight waves interleaving fragment reads, LDS writes and MFMAs in
//     one instruction stream with a barrier per step: 300-324 us;
//   - direct global -> LDS transfers (buffer_load ... lds) into four K-128
//     stages, which frees the staging registers and the LDS write
//     instructions: 365 us (the transfers run at about half the rate of
//     register-staged loads);
//   - four waves of 128 x 128 (one per SIMD): 4-8% slower than the
//     interleaved eight-wave loop.
// Ablations of this loop: without the global loads 251 us, without the LDS
// writes 225 us, with all-zero operands (less power, higher clock) 209 us; the
// MFMA pipe itself sustains about 5.6 PFLOP/s on random FP4 data.  (These
// figures date from when the loop was written; the same launch now takes
// about 230 us.)  Later, with every load an L2 hit (all K steps reading the
// lines of step 0): 4% faster at this shape and up to 15% on the short-K ones,
// at the same clock -- load latency beyond L2, which the one K step between a
// part's load and its LDS write does not always cover.  Prefetching the lines
// of step s+6 (one dword per line, into an LDS sink or into registers) ran
// 11-12% slower: vector loads complete in order, so the prefetch's own miss
// holds up the next real load.
constexpr int kLdsA = 0, kLdsB = 2 * BM * BKB, kLdsSA = 4 * BM * BKB, kLdsSB = kLdsSA + 2 * BM * 8;
static_assert(kLdsSB + 2 * BN * 8 == kSmemBytes, "fast path LDS layout");

// s_waitcnt immediate (gfx9 encoding: vmcnt[3:0]+[15:14], expcnt[6:4], lgkmcnt[11:8])
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 0xF) | ((vm >> 4) << 14) | 0x70 | ((lgkm & 0xF) << 8); }

struct FastPlan {
  __amdgpu_buffer_rsrc_t ra, rb, rs;   // A codes, this wave's B codes, this wave's scales
  __amdgpu_buffer_rsrc_t ra2, rb2, rs2;  // the same for the second operand pair (K steps nk1 ..)
  int nk1;                             // K steps of the first pair
  uint32_t va, vb;                     // lane code offsets of load j = 0 (j adds 8 rows)
  uint32_t vs;                         // lane scale offset
  uint32_t ldb8;                       // 8 code rows (bytes)
  uint32_t wa0, wa1;                   // lane LDS offsets (even / odd j) of its code chunk
  uint32_t ws;                         // lane LDS offset of its scale row (stage 0)
};

// Wave w loads code rows 32w..32w+31 of both tiles (load j: rows 32w + 8j +
// l/8, chunk l&7; 8 lanes cover a 128-byte row) and the scale rows 64(w&3) +
// l of A (waves 0-3) or B (waves 4-7).  For the SwiGLU producer, B tile rows
// 0..127 are W1 rows n0.. and rows 128..255 are W3 rows f+n0..
template <bool kSwiGLU>
__device__ __forceinline__ void make_fast_plan(FastPlan& p, const Operand& A, const Operand& B, int64_t m0,
                                               int64_t n0, int64_t f, int64_t K, const Operand* A2 = nullptr,
                                               const Operand* B2 = nullptr) {
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int l = threadIdx.x & 63;
  const int64_t ldb = K >> 1, lsc = K >> 5;
  const int64_t rows_a = min((int64_t)BM, A.rows - m0);
  const int64_t rows_b = kSwiGLU ? min((int64_t)128, f - n0) : min((int64_t)BN, B.rows - n0);
  p.ra = buffer_rsrc(A.codes + m0 * ldb, rows_a * ldb);
  int bshift = 0;
  if constexpr (kSwiGLU) {
    const int64_t g0 = (w >= 4 ? f : 0) + n0;
    p.rb = buffer_rsrc(B.codes + g0 * ldb, rows_b * ldb);
    bshift = w >= 4 ? 128 : 0;
  } else {
    p.rb = buffer_rsrc(B.codes + n0 * ldb, rows_b * ldb);
  }
  const int srow = 64 * (w & 3) + l;
  if (w < 4) {
    p.rs = buffer_rsrc(A.scales + m0 * lsc, rows_a * lsc);
    p.vs = (uint32_t)(srow * lsc);
    p.ws = (uint32_t)(kLdsSA + srow * 8);
  } else {
    int sshift = 0;
    if constexpr (kSwiGLU) {
      const int64_t g0 = (w >= 6 ? f : 0) + n0;
      p.rs = buffer_rsrc(B.scales + g0 * lsc, rows_b * lsc);
      sshift = w >= 6 ? 128 : 0;
    } else {
      p.rs = buffer_rsrc(B.scales + n0 * lsc, rows_b * lsc);
    }
    p.vs = (uint32_t)((srow - sshift) * lsc);
    p.ws = (uint32_t)(kLdsSB + srow * 8);
  }
  const int row0 = 32 * w + (l >> 3), c = l & 7;
  p.va = (uint32_t)(row0 * ldb + c * 16);
  p.vb = (uint32_t)((row0 - bshift) * ldb + c * 16);
  p.ldb8 = (uint32_t)(8 * ldb);
  // LDS slot of the chunk: c ^ ((row & 7) ^ ((row >> 3) & 1)) with row & 7 = l/8
  // and (row >> 3) & 1 = j & 1
  p.wa0 = (uint32_t)(row0 * BKB + ((c ^ (l >> 3)) * 16));
  p.wa1 = (uint32_t)(row0 * BKB + ((c ^ (l >> 3) ^ 1) * 16));
  // second pair (plain GEMM only): same shapes, so the same lane offsets
  if constexpr (!kSwiGLU) {
    if (A2 != nullptr && A2->codes != nullptr) {
      p.ra2 = buffer_rsrc(A2->codes + m0 * ldb, rows_a * ldb);
      p.rb2 = buffer_rsrc(B2->codes + n0 * ldb, rows_b * ldb);
      p.rs2 = w < 4 ? buffer_rsrc(A2->scales + m0 * lsc, rows_a * lsc) : buffer_rsrc(B2->scales + n0 * lsc, rows_b * lsc);
      p.nk1 = (int)(K / 256);
      return;
    }
  }
  p.ra2 = p.ra;
  p.rb2 = p.rb;
  p.rs2 = p.rs;
  p.nk1 = 0x7FFFFFFF;
}

struct Frags8 {
  v4i a[4], b[2];
};

template <bool kSwiGLU>
__device__ __forceinline__ constexpr int bsub8(int j) { return kSwiGLU ? 128 * j : 32 * j; }

template <int S, int I0, int I1>
__device__ __forceinline__ void mfma8(const Frags8& fr, const uint32_t (&sa)[4], const uint32_t (&sb)[2],
                                      v16f (&acc)[4][2]) {
#pragma unroll
  for (int i = I0; i < I1; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(fr.b[j]), widen(fr.a[i]), acc[i][j], 4, 4, S,
                                                                 (int)sb[j], S, (int)sa[i]);
    }
  }
  // Pin the group here: MFMAs are pure, and without a consumer at this point
  // the optimizer sinks them below the stage barrier.  Emits no code.
#pragma unroll
  for (int i = I0; i < I1; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) asm volatile("" : "+a"(acc[i][j]));
}

struct PartA {
  v4i a[4];
};
struct PartB {
  v4i b[4];
  uint2 s;
};

// Load j of a part reads 8 rows further down.  The row offset stays in the
// lane offset: the buffer range check (rows past the operand read zero) covers
// the lane offset, not the scalar one, which carries only the K position.
// K step `kit` of the concatenated K range: steps from nk1 on come from the
// second operand pair (a wave-uniform choice of buffer resources).
__device__ __forceinline__ void load_part_a(const FastPlan& p, int kit, PartA& x) {
  const bool second = kit >= p.nk1;
  const __amdgpu_buffer_rsrc_t ra = second ? p.ra2 : p.ra;
  const uint32_t so = (uint32_t)(second ? kit - p.nk1 : kit) * BKB;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    x.a[j] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ra, p.va + (uint32_t)j * p.ldb8, so, 0));
}

__device__ __forceinline__ void load_part_b(const FastPlan& p, int kit, PartB& x) {
  const bool second = kit >= p.nk1;
  const __amdgpu_buffer_rsrc_t rb = second ? p.rb2 : p.rb;
  const __amdgpu_buffer_rsrc_t rs = second ? p.rs2 : p.rs;
  const int k1 = second ? kit - p.nk1 : kit;
  const uint32_t so = (uint32_t)k1 * BKB, sso = (uint32_t)k1 * 8u;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    x.b[j] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rb, p.vb + (uint32_t)j * p.ldb8, so, 0));
  x.s = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, p.vs, sso, 0));
}

// Stage `stg` (0 or 1, wave-uniform) of the part: 32 KB per code stage, 2 KB
// per scale stage.
__device__ __forceinline__ void write_part_a(uint8_t* smem, const FastPlan& p, uint32_t stg, const PartA& x) {
  uint8_t* b0 = smem + (p.wa0 + (stg << 15));
  uint8_t* b1 = smem + (p.wa1 + (stg << 15));
#pragma unroll
  for (int j = 0; j < 4; ++j) *reinterpret_cast<v4i*>(((j & 1) ? b1 : b0) + (kLdsA + j * 1024)) = x.a[j];
}

__device__ __forceinline__ void write_part_b(uint8_t* smem, const FastPlan& p, uint32_t stg, const PartB& x) {
  uint8_t* b0 = smem + (p.wa0 + (stg << 15));
  uint8_t* b1 = smem + (p.wa1 + (stg << 15));
#pragma unroll
  for (int j = 0; j < 4; ++j) *reinterpret_cast<v4i*>(((j & 1) ? b1 : b0) + (kLdsB + j * 1024)) = x.b[j];
  *reinterpret_cast<uint2*>(smem + (p.ws + (stg << 11))) = x.s;
}

// Fragment addresses without per-sub-step registers: the chunk swizzle only
// touches address bits 4-6 and the sub-step XORs bits 4-5, so sub-step s of a
// fragment is its sub-step 0 address XOR 16 s; stage 1 sets bit 15 (codes) or
// bit 11 (scales), which no stage-0 address has set.
struct PPAddr {
  uint32_t a, b;      // sub-step 0, stage 0 byte address of this lane's first A and B fragment rows
  uint32_t sa, sb;    // scale dwords, stage 0
};

template <bool kSwiGLU>
__device__ __forceinline__ void make_pp_addr(PPAddr& q, int wm, int wn, int r, int h) {
  const int g = (r & 7) ^ ((r >> 3) & 1);
  const int x = (4 * h) ^ g;
  const int arow = wm * 128 + r;
  const int brow = (kSwiGLU ? wn * 32 : wn * 64) + r;
  q.a = (uint32_t)(kLdsA + arow * BKB + x * 16);
  q.b = (uint32_t)(kLdsB + brow * BKB + x * 16);
  q.sa = (uint32_t)(kLdsSA + (2 * arow + h) * 4);
  q.sb = (uint32_t)(kLdsSB + (2 * brow + h) * 4);
}

template <bool kSwiGLU, int S>
__device__ __forceinline__ void pp_read_frags(const uint8_t* smem, const PPAddr& q, uint32_t stg, Frags8& fr) {
  const uint8_t* pa = smem + ((q.a ^ (uint32_t)(16 * S)) | (stg << 15));
  const uint8_t* pb = smem + ((q.b ^ (uint32_t)(16 * S)) | (stg << 15));
#pragma unroll
  for (int i = 0; i < 4; ++i) fr.a[i] = *reinterpret_cast<const v4i*>(pa + i * 32 * BKB);
#pragma unroll
  for (int j = 0; j < 2; ++j) fr.b[j] = *reinterpret_cast<const v4i*>(pb + bsub8<kSwiGLU>(j) * BKB);
}

template <bool kSwiGLU>
__device__ __forceinline__ void pp_read_scales(const uint8_t* smem, const PPAddr& q, uint32_t stg, uint32_t (&sa)[4],
                                               uint32_t (&sb)[2]) {
  const uint8_t* pa = smem + (q.sa | (stg << 11));
  const uint8_t* pb = smem + (q.sb | (stg << 11));
#pragma unroll
  for (int i = 0; i < 4; ++i) sa[i] = *reinterpret_cast<const uint32_t*>(pa + i * 32 * 8);
#pragma unroll
  for (int j = 0; j < 2; ++j) sb[j] = *reinterpret_cast<const uint32_t*>(pb + bsub8<kSwiGLU>(j) * 8);
}

// Phase ends.  pp_sync: this wave's LDS traffic has landed, then the
// workgroup barrier; pp_next: no synchronisation, only an ordering fence
// (MFMAs are pure, and the optimizer would otherwise move them across phases).
__device__ __forceinline__ void pp_sync() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void pp_next() { __builtin_amdgcn_sched_barrier(0); }

template <int H, bool kSync>
__device__ __forceinline__ void pp_compute(const Frags8& f0, const Frags8& f1, const uint32_t (&sa)[4],
                                           const uint32_t (&sb)[2], v16f (&acc)[4][2]) {
  mfma8<2 * H, 0, 4>(f0, sa, sb, acc);
  mfma8<2 * H + 1, 0, 4>(f1, sa, sb, acc);
  if constexpr (kSync) pp_sync();
  else pp_next();
}

// Memory work of a phase: fragments of half H of stage `frs` (for H = 0 also
// the stage's scale dwords), one part written to stage `wst`, the same part of
// K step `lkit` loaded.
template <bool kSwiGLU, int H, bool kPartA, bool kSync>
__device__ __forceinline__ void pp_memory(uint8_t* smem, const FastPlan& p, const PPAddr& q, uint32_t frs,
                                          uint32_t wst, int lkit, Frags8& f0, Frags8& f1, uint32_t (&sa)[4],
                                          uint32_t (&sb)[2], PartA& xa, PartB& xb) {
  pp_read_frags<kSwiGLU, 2 * H>(smem, q, frs, f0);
  pp_read_frags<kSwiGLU, 2 * H + 1>(smem, q, frs, f1);
  if constexpr (H == 0) pp_read_scales<kSwiGLU>(smem, q, frs, sa, sb);
  // the part's registers are written out before they are loaded again: kept
  // in this order, one set of staging registers per part suffices
  if constexpr (kPartA) write_part_a(smem, p, wst, xa);
  else write_part_b(smem, p, wst, xb);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (kPartA) load_part_a(p, lkit, xa);
  else load_part_b(p, lkit, xb);
  if constexpr (kSync) pp_sync();
  else pp_next();
}

// With A2/B2 (plain GEMM only) the loop runs over K of (A, B) and then K of
// (A2, B2) into the same accumulators: one fp32 sum over the concatenated K.
template <bool kSwiGLU>
__device__ __forceinline__ void main_loop_fast(uint8_t* smem, const Operand& A, const Operand& B, int64_t m0,
                                               int64_t n0, int64_t f, int64_t K, v16f (&acc)[4][2], int wm, int wn,
                                               const Operand* A2 = nullptr, const Operand* B2 = nullptr) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
  const int lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
  const int nk = (int)(K / 256) * ((A2 != nullptr && A2->codes != nullptr) ? 2 : 1), last = nk - 1;
  FastPlan p;
  make_fast_plan<kSwiGLU>(p, A, B, m0, n0, f, K, A2, B2);
  PPAddr q;
  make_pp_addr<kSwiGLU>(q, wm, wn, r, h);
  PartA xa;
  PartB xb;
  Frags8 f0, f1;
  uint32_t sa[4], sb[2];
  // every wave: stage 0 whole, then its stage-1 parts in registers
  load_part_a(p, 0, xa);
  load_part_b(p, 0, xb);
  write_part_a(smem, p, 0u, xa);
  write_part_b(smem, p, 0u, xb);
  __builtin_amdgcn_sched_barrier(0);
  load_part_a(p, min(1, last), xa);
  load_part_b(p, min(1, last), xb);
  if (__builtin_amdgcn_readfirstlane(wm) == 0) {
    // group 0 writes its A part of stage 1 now (its phase 4s-1 for s = 0),
    // loads A of stage 2, and reads its first fragments after the barrier
    write_part_a(smem, p, 1u, xa);
    __builtin_amdgcn_sched_barrier(0);
    load_part_a(p, min(2, last), xa);
    pp_sync();
    pp_read_frags<kSwiGLU, 0>(smem, q, 0u, f0);
    pp_read_frags<kSwiGLU, 1>(smem, q, 0u, f1);
    pp_read_scales<kSwiGLU>(smem, q, 0u, sa, sb);
    for (int s = 0; s < nk; ++s) {
      const uint32_t cur = (uint32_t)(s & 1), nxt = cur ^ 1u;
      pp_compute<0, false>(f0, f1, sa, sb, acc);
      pp_memory<kSwiGLU, 1, false, false>(smem, p, q, cur, nxt, min(s + 2, last), f0, f1, sa, sb, xa, xb);
      pp_compute<1, true>(f0, f1, sa, sb, acc);
      pp_memory<kSwiGLU, 0, true, false>(smem, p, q, nxt, cur, min(s + 3, last), f0, f1, sa, sb, xa, xb);
    }
  } else {
    pp_sync();
    for (int s = 0; s < nk; ++s) {
      const uint32_t cur = (uint32_t)(s & 1), nxt = cur ^ 1u;
      pp_memory<kSwiGLU, 0, true, false>(smem, p, q, cur, nxt, min(s + 2, last), f0, f1, sa, sb, xa, xb);
      pp_compute<0, false>(f0, f1, sa, sb, acc);
      pp_memory<kSwiGLU, 1, false, true>(smem, p, q, cur, nxt, min(s + 2, last), f0, f1, sa, sb, xa, xb);
      pp_compute<1, false>(f0, f1, sa, sb, acc);
    }
  }
  __syncthreads();
}


}  // namespace mx
