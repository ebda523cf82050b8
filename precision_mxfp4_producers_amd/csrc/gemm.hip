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
// grouped along M so neighbouring tiles reuse A rows and B columns.
__device__ __forceinline__ void tile_coords(int64_t tiles_m, int64_t tiles_n, int64_t& tm, int64_t& tn) {
  int64_t pid = blockIdx.x;
  const int64_t num = gridDim.x;
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
// MFMA pipe itself sustains about 5.6 PFLOP/s on random FP4 data.
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
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) m = max(m, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
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
    h32_sign_words(v, sign_mask16);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int64_t col = n0 + 2 * cp + c;
      if (col >= Fdim) continue;
      float fv[32];
      h32_half(v, c, fv);
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
    h32_sign_words(v, sign_mask16);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int64_t col = n0 + 2 * cp + c;
      float fv[32];
      h32_half(v, c, fv);
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

// a2_codes == nullptr: C (+)= A B^T.  Otherwise C (+)= A B^T + A2 B2^T as one
// fp32 accumulation over both K ranges (each K long).  `flags`: bit 0
// accumulate, bit 1 write C with non-temporal (streaming) stores.
__global__ __launch_bounds__(kFastThreads) void gemm_fast_kernel(
    int64_t M, int64_t N, int64_t K, const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_scales, const uint8_t* __restrict__ a2_codes,
    const uint8_t* __restrict__ a2_scales, const uint8_t* __restrict__ b2_codes,
    const uint8_t* __restrict__ b2_scales, float* __restrict__ c, int64_t ldc, int flags) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
  int64_t tm, tn;
  tile_coords((M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 2, wn = wave & 3, hl = lane >> 5;
  Operand A{a_codes, a_scales, M}, B{b_codes, b_scales, N};
  Operand A2{a2_codes, a2_scales, M}, B2{b2_codes, b2_scales, N};
  v16f acc[4][2];
  main_loop_fast<false>(smem, A, B, m0, n0, 0, K, acc, wm, wn, &A2, &B2);
  store_c_tile_wave(smem, acc, c, ldc, M, N, m0, n0, wave, lane, wm, wn, hl, (flags & 1) != 0,
                    (flags & 2) != 0);
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

extern "C" {

fp4_status fp4_gemm(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes, const uint8_t* a_scales,
                    const uint8_t* b_codes, const uint8_t* b_scales, float* c, int64_t ldc, int accumulate,
                    void* stream) {
  if (accumulate != 0 && accumulate != 1) return FP4_EINVAL;
  if (!mult32z(m) || !mult32z(n) || !mult32z(k) || ldc < n) return FP4_ESHAPE;
  if (m == 0 || n == 0) return FP4_OK;                    // empty C
  if (!c) return FP4_EINVAL;
  if (k == 0) {                                           // empty sums: C = 0, or C unchanged when accumulating
    if (accumulate) return FP4_OK;
    const int64_t gx = (n + 255) / 256, gy = std::min<int64_t>(m, 65535);
    if (gx > 0x7FFFFFFF) return FP4_ESHAPE;
    hipLaunchKernelGGL(fill_rows_f32_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0,
                       as_stream(stream), c, m, n, ldc);
    return launch_status();
  }
  if (!a_codes || !a_scales || !b_codes || !b_scales) return FP4_EINVAL;
  if (!aligned16(a_codes) || !aligned16(b_codes) || !aligned16(a_scales) || !aligned16(b_scales) ||
      !aligned16(c) || (ldc % 4) != 0)
    return FP4_EALIGN;
  const int64_t tiles = grid_tiles(m, BM, n, BN);
  if (tiles < 0) return FP4_ESHAPE;
  hipStream_t s = as_stream(stream);
  // the fast path needs K % 256 == 0 and buffer offsets below 2^31 per tile
  if ((k % 256) == 0 && 256 * (k / 2) < 0x7FFFFFFF)
    hipLaunchKernelGGL(gemm_fast_kernel, dim3((unsigned)tiles), dim3(kFastThreads), 0, s, m, n, k, a_codes, a_scales,
                       b_codes, b_scales, nullptr, nullptr, nullptr, nullptr, c, ldc, fast_flags(m, n, accumulate));
  else
    hipLaunchKernelGGL(gemm_generic_kernel, dim3((unsigned)tiles), dim3(kGemmThreads), 0, s, m, n, k, a_codes,
                       a_scales, b_codes, b_scales, c, ldc, accumulate);
  return launch_status();
}

fp4_status fp4_gemm_pair(int64_t m, int64_t n, int64_t k, const uint8_t* a1_codes, const uint8_t* a1_scales,
                         const uint8_t* b1_codes, const uint8_t* b1_scales, const uint8_t* a2_codes,
                         const uint8_t* a2_scales, const uint8_t* b2_codes, const uint8_t* b2_scales, float* c,
                         int64_t ldc, int accumulate, void* stream) {
  if (accumulate != 0 && accumulate != 1) return FP4_EINVAL;
  if (!mult32z(m) || !mult32z(n) || !mult32z(k) || ldc < n) return FP4_ESHAPE;
  if (m == 0 || n == 0) return FP4_OK;
  if (k == 0) return fp4_gemm(m, n, 0, nullptr, nullptr, nullptr, nullptr, c, ldc, accumulate, stream);
  if (!c || !a1_codes || !a1_scales || !b1_codes || !b1_scales || !a2_codes || !a2_scales || !b2_codes ||
      !b2_scales)
    return FP4_EINVAL;
  if (!aligned16(a1_codes) || !aligned16(b1_codes) || !aligned16(a1_scales) || !aligned16(b1_scales) ||
      !aligned16(a2_codes) || !aligned16(b2_codes) || !aligned16(a2_scales) || !aligned16(b2_scales) ||
      !aligned16(c) || (ldc % 4) != 0)
    return FP4_EALIGN;
  const int64_t tiles = grid_tiles(m, BM, n, BN);
  if (tiles < 0) return FP4_ESHAPE;
  if ((k % 256) == 0 && 256 * (k / 2) < 0x7FFFFFFF) {
    hipLaunchKernelGGL(gemm_fast_kernel, dim3((unsigned)tiles), dim3(kFastThreads), 0, as_stream(stream), m, n, k,
                       a1_codes, a1_scales, b1_codes, b1_scales, a2_codes, a2_scales, b2_codes, b2_scales, c, ldc,
                       fast_flags(m, n, accumulate));
    return launch_status();
  }
  // K not a multiple of 256: the second product is added to the first's result
  const fp4_status st = fp4_gemm(m, n, k, a1_codes, a1_scales, b1_codes, b1_scales, c, ldc, accumulate, stream);
  if (st != FP4_OK) return st;
  return fp4_gemm(m, n, k, a2_codes, a2_scales, b2_codes, b2_scales, c, ldc, 1, stream);
}

fp4_status fp4_swiglu_producer(int64_t t, int64_t f, int64_t d, const uint8_t* x_codes, const uint8_t* x_scales,
                               const uint8_t* w13_codes, const uint8_t* w13_scales, uint16_t* a_bf16,
                               uint16_t* b_bf16, uint8_t* h_codes, uint8_t* h_scales, uint8_t* ht_codes,
                               uint8_t* ht_scales, uint32_t sign_mask16, void* stream) {
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
