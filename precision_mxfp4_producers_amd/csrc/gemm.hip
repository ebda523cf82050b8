// Block-scaled E2M1 GEMM on the gfx950 scaled MFMA, and the fused SwiGLU
// producer built on the same main loop.
//
// "Format-Aware Fusion for Fast FP4 Pretraining":
//   §2.3 (Eq. 4-6)  Fprop, Dgrad and Wgrad are all C = dec(A) dec(B)^T with
//                   both operands K-major and 1x32 E8M0 scales along K.
//   §3.2            the gated FFN pairs W1 and W3 and emits the SiLU-gated
//                   output directly as the FP4 input of W2.
//
// Main loop.  A 256-lane workgroup owns a 256x256 output tile and walks K in
// steps of 256 values (128 code bytes + 8 scale bytes per row).  Each step is
// staged global -> registers -> LDS (double-buffered, one barrier per step);
// 16-byte chunks are XOR-swizzled so that the fragment reads of 16 consecutive
// rows hit distinct banks.  Each wave computes a 128x128 sub-tile as 4x4
// v_mfma_scale_f32_32x32x64_f8f6f4 tiles (both operands FP4, fp32 accumulate).
// A lane of that instruction supplies 32 K-values of one row plus their E8M0
// scale byte; lanes 0-31 and 32-63 supply two different 32-blocks.  Within a
// K step, lane half h takes blocks 4h..4h+3 for the four sub-steps, so each
// lane's four scale bytes are one aligned dword and the sub-step selects the
// byte (op_sel).  Applying the same block assignment to A and B leaves the
// sum over K unchanged.
#include <hip/hip_runtime.h>

#include "abi_common.h"
#include "mx_device.h"

namespace mx {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256;
constexpr int BKB = 128;                    // code bytes per row per K step (256 values)
constexpr int kGemmThreads = 256;
constexpr int kStageBytes = BM * BKB + BN * BKB + BM * 8 + BN * 8;    // 69632
constexpr int kHPitch = 272;
static_assert(2 * kStageBytes == 139264, "LDS budget");                // bytes per row of the staged h tile (256 + 16)

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
          widen(af[i]), widen(bf[j]), acc[i][j], 4, 4, S, (int)sa[i], S, (int)sb[j]);
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

// ------------------------------------------------------------------ DMA main loop
// Fast path for K % 128 == 0.  Code and scale tiles move global -> LDS with
// buffer_load ... lds: no staging registers; rows beyond M/N and chunks beyond
// K get an out-of-range buffer offset and read as zero.  The DMA is issued
// with inline asm so that the compiler's wait-count pass, which cannot tell
// the two stage buffers apart, does not stall every LDS read behind it; the
// single wait it needs (vmcnt(0) before each stage barrier) is explicit.
//
// LDS layout (stage-interleaved per operand so the stage is an immediate
// offset of the fragment reads):
//   A stage 0 | A stage 1 | B stage 0 | B stage 1 | SA 0 | SA 1 | SB 0 | SB 1
//   32 KB each (256 rows x 128 B, 16-byte chunks swizzled), 2 KB per scale tile
// Per K step each wave issues 8 + 8 16-byte code DMAs (1 KB blocks of 8 rows)
// and 2 + 2 4-byte scale DMAs (256 B blocks of 32 rows x 2 dwords).  Fragments
// are read from LDS one sub-step ahead of the MFMAs that use them; the DMA of
// step it+2 is issued right after the barrier that ends step it and overlaps
// a whole step of MFMA work.
constexpr int kLdsA = 0, kLdsB = 2 * BM * BKB, kLdsSA = 4 * BM * BKB, kLdsSB = kLdsSA + 2 * BM * 8;
constexpr int kLdsTotal = kLdsSB + 2 * BN * 8;          // 139264
constexpr uint32_t kOOB = 0x80000000u;                  // beyond every num_records below
constexpr int kDmaPerStage = 20;                        // DMA instructions per wave per K step

// s_waitcnt immediate (gfx9 encoding: vmcnt[3:0]+[15:14], expcnt[6:4], lgkmcnt[11:8])
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 0xF) | ((vm >> 4) << 14) | 0x70 | ((lgkm & 0xF) << 8); }

// Raw buffer descriptor (stride 0, range-checked on the byte offset), uniform.
__device__ __forceinline__ v4i buffer_rsrc(const void* base, int64_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const int64_t n = bytes < 0 ? 0 : (bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF);
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32) & 0xFFFF);
  r[2] = __builtin_amdgcn_readfirstlane((int)n);
  r[3] = 0x00020000;
  return r;
}

__device__ __forceinline__ void dma_b128(v4i rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}
__device__ __forceinline__ void dma_b32(v4i rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}

struct DmaPlan {
  v4i ra, rb, rsa, rsb;          // this wave's descriptors (B: W1 or W3 half for the SwiGLU producer)
  uint32_t va0, va1, vb0, vb1;   // lane code offsets for even / odd DMA j
  uint32_t vsa, vsb;             // lane scale offsets
  uint32_t ldb8, lds32;          // 8 code rows, 32 scale rows (bytes)
  uint32_t lds_base;             // LDS address of the tile buffers
  bool hi0, hi1;                 // lane's chunk (even / odd j) lies in the upper half of a K step
  int w;                         // wave index (uniform)
};

template <bool kSwiGLU>
__device__ __forceinline__ void make_plan(DmaPlan& p, const uint8_t* smem, const Operand& A, const Operand& B,
                                          int64_t m0, int64_t n0, int64_t f, int64_t K) {
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int l = threadIdx.x & 63;
  const int64_t ldb = K >> 1, lsc = K >> 5;
  const int64_t rows_a = min((int64_t)BM, A.rows - m0);
  p.ra = buffer_rsrc(A.codes + m0 * ldb, rows_a * ldb);
  p.rsa = buffer_rsrc(A.scales + m0 * lsc, rows_a * lsc);
  int brow_shift = 0;                                    // B tile rows handled by this wave start here
  if constexpr (kSwiGLU) {
    const int64_t rows_b = min((int64_t)128, f - n0);
    const int64_t g0 = (w >= 2 ? f : 0) + n0;            // W1 rows n0.. or W3 rows f+n0..
    p.rb = buffer_rsrc(B.codes + g0 * ldb, rows_b * ldb);
    p.rsb = buffer_rsrc(B.scales + g0 * lsc, rows_b * lsc);
    brow_shift = w >= 2 ? 128 : 0;
  } else {
    const int64_t rows_b = min((int64_t)BN, B.rows - n0);
    p.rb = buffer_rsrc(B.codes + n0 * ldb, rows_b * ldb);
    p.rsb = buffer_rsrc(B.scales + n0 * lsc, rows_b * lsc);
  }
  // DMA j of wave w covers rows 8i..8i+7, i = 8w + j; lane l takes row 8i + l/8
  // and LDS slot l&7, which holds logical chunk (l&7) ^ swizzle(row).
  const int row0 = 64 * w + (l >> 3);
  const int c0 = (l & 7) ^ (l >> 3);                     // j even (swizzle bit 3 of the row is 0)
  const int c1 = c0 ^ 1;                                 // j odd
  p.va0 = (uint32_t)(row0 * ldb + c0 * 16);
  p.va1 = (uint32_t)(row0 * ldb + c1 * 16);
  p.vb0 = (uint32_t)((row0 - brow_shift) * ldb + c0 * 16);
  p.vb1 = (uint32_t)((row0 - brow_shift) * ldb + c1 * 16);
  p.hi0 = c0 >= 4;
  p.hi1 = c1 >= 4;
  // scale DMA j of wave w covers rows 32i..32i+31 (i = 2w + j), lane l: row 32i + l/2, dword l&1
  const int srow0 = 64 * w + (l >> 1);
  p.vsa = (uint32_t)(srow0 * lsc + 4 * (l & 1));
  p.vsb = (uint32_t)((srow0 - brow_shift) * lsc + 4 * (l & 1));
  p.ldb8 = (uint32_t)(8 * ldb);
  p.lds32 = (uint32_t)(32 * lsc);
  p.lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)smem;
  p.w = w;
}

// `none` (uniform) turns every offset out of range: the DMA then only writes
// zeros into a stage that is no longer read, which keeps the loop branch-free.
__device__ __forceinline__ void dma_stage(const DmaPlan& p, int stg, int kit, bool half, bool none = false) {
  const uint32_t so = (uint32_t)kit * BKB, sso = (uint32_t)kit * 8u;
  const bool odd_lane = (threadIdx.x & 1) != 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = 8 * p.w + j;
    uint32_t va = ((j & 1) ? p.va1 : p.va0) + (uint32_t)j * p.ldb8;
    uint32_t vb = ((j & 1) ? p.vb1 : p.vb0) + (uint32_t)j * p.ldb8;
    if (none || (half && ((j & 1) ? p.hi1 : p.hi0))) va = vb = kOOB;
    dma_b128(p.ra, p.lds_base + kLdsA + stg * BM * BKB + i * 1024, va, so);
    dma_b128(p.rb, p.lds_base + kLdsB + stg * BN * BKB + i * 1024, vb, so);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = 2 * p.w + j;
    uint32_t va = p.vsa + (uint32_t)j * p.lds32;
    uint32_t vb = p.vsb + (uint32_t)j * p.lds32;
    if (none || (half && odd_lane)) va = vb = kOOB;
    dma_b32(p.rsa, p.lds_base + kLdsSA + stg * BM * 8 + i * 256, va, sso);
    dma_b32(p.rsb, p.lds_base + kLdsSB + stg * BN * 8 + i * 256, vb, sso);
  }
}

struct Frags {
  v4i a[4], b[4];
};

// Lane-constant LDS offsets of this wave's fragments for sub-step s (chunk
// 4h + s of its row, swizzled) and of its scale dwords.
struct FragAddr {
  uint32_t a[4], b[4];
  uint32_t sa, sb;
};

template <bool kSwiGLU>
__device__ __forceinline__ void make_frag_addr(FragAddr& fa, int wm, int wn, int r, int h) {
  const int g = (r & 7) ^ ((r >> 3) & 1);                // swizzle of rows r + 32k (same low 4 bits)
  const int x = (4 * h) ^ g;
  const int arow = wm * 128 + r;
  const int brow = (kSwiGLU ? wn * 64 : wn * 128) + r;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    fa.a[s] = (uint32_t)(kLdsA + arow * BKB + ((x ^ s) * 16));
    fa.b[s] = (uint32_t)(kLdsB + brow * BKB + ((x ^ s) * 16));
  }
  fa.sa = (uint32_t)(kLdsSA + (2 * arow + h) * 4);
  fa.sb = (uint32_t)(kLdsSB + (2 * brow + h) * 4);
}

template <bool kSwiGLU>
__device__ __forceinline__ constexpr int b_sub_off(int j) {
  // byte offset of B sub-tile j relative to the wave's first B row
  return kSwiGLU ? ((j < 2) ? 32 * j * BKB : (128 + 32 * (j - 2)) * BKB) : 32 * j * BKB;
}

template <bool kSwiGLU>
__device__ __forceinline__ void read_frags(const uint8_t* smem, const FragAddr& fa, Frags& fr, int s, uint32_t soff) {
  const uint8_t* pa = smem + (fa.a[s] + soff);
  const uint8_t* pb = smem + (fa.b[s] + soff);
#pragma unroll
  for (int i = 0; i < 4; ++i) fr.a[i] = *reinterpret_cast<const v4i*>(pa + i * 32 * BKB);
#pragma unroll
  for (int j = 0; j < 4; ++j) fr.b[j] = *reinterpret_cast<const v4i*>(pb + b_sub_off<kSwiGLU>(j));
}

template <bool kSwiGLU>
__device__ __forceinline__ void read_scales(const uint8_t* smem, const FragAddr& fa, uint32_t (&sa)[4],
                                            uint32_t (&sb)[4], uint32_t stg) {
  const uint8_t* pa = smem + (fa.sa + stg * (BM * 8));
  const uint8_t* pb = smem + (fa.sb + stg * (BN * 8));
#pragma unroll
  for (int i = 0; i < 4; ++i) sa[i] = *reinterpret_cast<const uint32_t*>(pa + i * 32 * 8);
#pragma unroll
  for (int j = 0; j < 4; ++j) sb[j] = *reinterpret_cast<const uint32_t*>(pb + (b_sub_off<kSwiGLU>(j) / BKB) * 8);
}

template <int S, int I0, int I1>
__device__ __forceinline__ void mfma_rows(const Frags& fr, const uint32_t (&sa)[4], const uint32_t (&sb)[4],
                                          v16f (&acc)[4][4]) {
#pragma unroll
  for (int i = I0; i < I1; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(fr.a[i]), widen(fr.b[j]), acc[i][j], 4, 4, S,
                                                                 (int)sa[i], S, (int)sb[j]);
    }
  }
  // Pin the group here: MFMAs are pure, and without a consumer at this point
  // the optimizer sinks them below the stage barrier.  Emits no code.
#pragma unroll
  for (int i = I0; i < I1; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" : "+a"(acc[i][j]));
}

// Scheduling region: the 8 fragment reads of the next sub-step go out first,
// then the 16 MFMAs of this one (which cover their latency).
__device__ __forceinline__ void reads_then_mfma() {
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // DS read
  __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);  // MFMA
  __builtin_amdgcn_sched_barrier(0);
}

// One K step on stage `stg` (its sub-step 0 fragments and scales are already
// in registers): prefetches sub-step 0 of the next step from the other stage
// and issues the DMA of step it+2 into this stage once every wave is done with
// it.  No branch encloses MFMA work, so the accumulators stay in AGPRs.
template <bool kSwiGLU>
__device__ __forceinline__ void dma_step(const uint8_t* smem, const DmaPlan& p, const FragAddr& fa, int it, int nk,
                                         bool k_half, int stg, Frags& f0, Frags& f1, uint32_t (&sa)[4],
                                         uint32_t (&sb)[4], v16f (&acc)[4][4]) {
  const uint32_t cur = (uint32_t)stg * (BM * BKB), nxt = (uint32_t)(stg ^ 1) * (BM * BKB);
  // sched_barrier(0) fences keep each sub-step's LDS reads ahead of the
  // previous sub-step's MFMAs (the scheduler would otherwise hoist every read
  // and sink every MFMA below the stage barrier).
  read_frags<kSwiGLU>(smem, fa, f1, 1, cur);
  mfma_rows<0, 0, 4>(f0, sa, sb, acc);
  reads_then_mfma();
  read_frags<kSwiGLU>(smem, fa, f0, 2, cur);
  mfma_rows<1, 0, 4>(f1, sa, sb, acc);
  reads_then_mfma();
  read_frags<kSwiGLU>(smem, fa, f1, 3, cur);
  mfma_rows<2, 0, 4>(f0, sa, sb, acc);
  reads_then_mfma();
  mfma_rows<3, 0, 2>(f1, sa, sb, acc);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));       // own DMA of step it+1 landed, own reads done
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  uint32_t sa_n[4], sb_n[4];
  read_frags<kSwiGLU>(smem, fa, f0, 0, nxt);             // harmless past the last step
  read_scales<kSwiGLU>(smem, fa, sa_n, sb_n, (uint32_t)(stg ^ 1));
  dma_stage(p, stg, it + 2, k_half && it + 2 == nk - 1, it + 2 >= nk);
  __builtin_amdgcn_sched_barrier(0);
  mfma_rows<3, 2, 4>(f1, sa, sb, acc);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sa[i] = sa_n[i];
    sb[i] = sb_n[i];
  }
}

template <bool kSwiGLU>
__device__ __forceinline__ void main_loop_dma(uint8_t* smem, const Operand& A, const Operand& B, int64_t m0,
                                              int64_t n0, int64_t f, int64_t K, v16f (&acc)[4][4], int wm, int wn) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
  const int lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
  const int nk = (int)((K + 255) / 256);
  const bool k_half = (K & 255) != 0;                    // the last step holds 128 values
  DmaPlan p;
  make_plan<kSwiGLU>(p, smem, A, B, m0, n0, f, K);
  FragAddr fa;
  make_frag_addr<kSwiGLU>(fa, wm, wn, r, h);
  dma_stage(p, 0, 0, k_half && nk == 1);
  if (nk > 1) {
    dma_stage(p, 1, 1, k_half && nk == 2);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(kDmaPerStage, 15));
  } else {
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
  }
  __builtin_amdgcn_s_barrier();
  Frags f0, f1;
  uint32_t sa[4], sb[4];
  read_frags<kSwiGLU>(smem, fa, f0, 0, 0u);
  read_scales<kSwiGLU>(smem, fa, sa, sb, 0u);
  for (int it = 0; it < nk; ++it)
    dma_step<kSwiGLU>(smem, p, fa, it, nk, k_half, it & 1, f0, f1, sa, sb, acc);
  __syncthreads();
}

// ------------------------------------------------------------------ GEMM
template <bool kDMA>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(
    int64_t M, int64_t N, int64_t K, const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_scales, float* __restrict__ c,
    int64_t ldc, int accumulate) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStageBytes];
  const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int64_t tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  Operand A{a_codes, a_scales, M}, B{b_codes, b_scales, N};
  v16f acc[4][4];
  if constexpr (kDMA) main_loop_dma<false>(smem, A, B, m0, n0, 0, K, acc, wm, wn);
  else main_loop_generic<false>(smem, smem + kStageBytes, A, B, m0, n0, 0, K, acc, wm, wn);

  // 32x32 accumulator layout: lane holds column (lane & 31); register q holds
  // row 8*(q/4) + 4*(lane/32) + (q%4).
  const int hl = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn * 128 + 32 * j + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t row = m0 + wm * 128 + 32 * i + 8 * (q >> 2) + 4 * hl + (q & 3);
        if (row < M) {
          float* p = c + row * ldc + col;
          *p = accumulate ? __fadd_rn(*p, acc[i][j][q]) : acc[i][j][q];
        }
      }
    }
  }
}

// ------------------------------------------------------------------ SwiGLU producer
// Output tile: 256 tokens x 128 FFN columns.  Wave (wm, wn) holds a and b for
// tokens wm*128.. and columns wn*64.. in matching registers (sub-tiles j and
// j+2), so h is formed in registers; a and b are saved as bf16 and h is staged
// in LDS as bf16, then quantized row-facing (32 columns per block) and, if
// requested, column-facing with H32 (32 tokens per block).
__device__ __forceinline__ void h32_block(float (&f)[32]) {
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
  const float cn = 0x1.6a09e6p-3f;                       // RN_fp32(2^-2.5)
#pragma unroll
  for (int j = 0; j < 32; ++j) f[j] = __fmul_rn(f[j], cn);
}

__device__ __forceinline__ uint4 encode_block_rtn(const float (&f)[32], int& e_out) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) m = max(m, __float_as_uint(f[j]) & 0x7FFFFFFFu);
  const int e = upward_exp(m);
  const float inv = inv_pow2(e);
  uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const uint32_t b = __float_as_uint(f[j]);
    const float y = __uint_as_float(b & 0x7FFFFFFFu) * inv;
    out[j >> 3] |= (e2m1_rtn(y) | ((b >> 28) & 8u)) << (4 * (j & 7));
  }
  e_out = e;
  return make_uint4(out[0], out[1], out[2], out[3]);
}

template <bool kDMA>
__global__ __launch_bounds__(kGemmThreads) void swiglu_producer_kernel(
    int64_t T, int64_t Fdim, int64_t D, const uint8_t* __restrict__ x_codes, const uint8_t* __restrict__ x_scales,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, uint16_t* __restrict__ a_out,
    uint16_t* __restrict__ b_out, uint8_t* __restrict__ h_codes, uint8_t* __restrict__ h_scales,
    uint8_t* __restrict__ ht_codes, uint8_t* __restrict__ ht_scales, uint32_t sign_mask16) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStageBytes];   // h tile staged here afterwards
  const int64_t tiles_m = (T + BM - 1) / BM, tiles_n = (Fdim + 127) / 128;
  int64_t tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * 128;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  Operand A{x_codes, x_scales, T}, B{w_codes, w_scales, 2 * Fdim};
  v16f acc[4][4];
  if constexpr (kDMA) main_loop_dma<true>(smem, A, B, m0, n0, Fdim, D, acc, wm, wn);
  else main_loop_generic<true>(smem, smem + kStageBytes, A, B, m0, n0, Fdim, D, acc, wm, wn);
  // (main_loop ends with a barrier: LDS is free for the h tile)

  const int hl = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int lc = wn * 64 + 32 * j + (lane & 31);            // column within the 128-wide tile
      const int64_t col = n0 + lc;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int lr = wm * 128 + 32 * i + 8 * (q >> 2) + 4 * hl + (q & 3);
        const int64_t row = m0 + lr;
        const uint32_t ab = f32_to_bf16_rne(acc[i][j][q]);
        const uint32_t bb = f32_to_bf16_rne(acc[i][j + 2][q]);
        float sig, s;
        sigmoid_silu(bf16_bits_to_f32(ab), sig, s);
        const uint32_t hb = f32_to_bf16_rne(__fmul_rn(s, bf16_bits_to_f32(bb)));
        *reinterpret_cast<uint16_t*>(smem + lr * kHPitch + lc * 2) = (uint16_t)hb;
        if (row < T && col < Fdim) {
          a_out[row * Fdim + col] = (uint16_t)ab;
          b_out[row * Fdim + col] = (uint16_t)bb;
        }
      }
    }
  }
  __syncthreads();

  // row-facing h: lane tid owns token row tid, four 32-column blocks
  {
    const int lr = tid;
    const int64_t row = m0 + lr;
    if (row < T) {
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const int64_t col0 = n0 + 32 * blk;
        if (col0 >= Fdim) break;
        float fv[32];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 d = *reinterpret_cast<const uint4*>(smem + lr * kHPitch + blk * 64 + q * 16);
          const uint32_t w4[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            fv[8 * q + 2 * u] = bf16_bits_to_f32(w4[u] & 0xFFFFu);
            fv[8 * q + 2 * u + 1] = bf16_bits_to_f32(w4[u] >> 16);
          }
        }
        int e;
        const uint4 code = encode_block_rtn(fv, e);
        *reinterpret_cast<uint4*>(h_codes + row * (Fdim >> 1) + (col0 >> 1)) = code;
        h_scales[row * (Fdim >> 5) + (col0 >> 5)] = (uint8_t)(e + 127);
      }
    }
  }

  // column-facing h with H32: lane owns columns 2cp, 2cp+1 and token blocks 2g, 2g+1
  if (ht_codes != nullptr) {
    const int cp = tid & 63, g = tid >> 6;
#pragma unroll
    for (int tb2 = 0; tb2 < 2; ++tb2) {
      const int tb = 2 * g + tb2;
      const int64_t r0 = m0 + 32 * tb;
      if (r0 >= T) continue;
      uint32_t v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i)
        v[i] = *reinterpret_cast<const uint32_t*>(smem + (32 * tb + i) * kHPitch + cp * 4);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int64_t col = n0 + 2 * cp + c;
        if (col >= Fdim) continue;
        float fv[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          uint32_t b = (v[i] >> (16 * c)) & 0xFFFFu;
          b ^= ((sign_mask16 >> (i & 15)) & 1u) << 15;
          fv[i] = bf16_bits_to_f32(b);
        }
        h32_block(fv);
        int e;
        const uint4 code = encode_block_rtn(fv, e);
        *reinterpret_cast<uint4*>(ht_codes + col * (T >> 1) + (r0 >> 1)) = code;
        ht_scales[col * (T >> 5) + (r0 >> 5)] = (uint8_t)(e + 127);
      }
    }
  }
}

}  // namespace mx

using namespace mx;

extern "C" {

fp4_status fp4_gemm(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes, const uint8_t* a_scales,
                    const uint8_t* b_codes, const uint8_t* b_scales, float* c, int64_t ldc, int accumulate,
                    void* stream) {
  if (!a_codes || !a_scales || !b_codes || !b_scales || !c || (accumulate != 0 && accumulate != 1))
    return FP4_EINVAL;
  if (!mult32(m) || !mult32(n) || !mult32(k) || ldc < n) return FP4_ESHAPE;
  if (!aligned16(a_codes) || !aligned16(b_codes) || !aligned16(a_scales) || !aligned16(b_scales) ||
      !aligned16(c) || (ldc % 4) != 0)
    return FP4_EALIGN;
  const int64_t tiles = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
  if (tiles > 0x7FFFFFFF) return FP4_ESHAPE;
  // the DMA path needs K % 128 == 0 and byte offsets below 2^31
  const bool dma = (k % 128) == 0 && m * (k / 2) < 0x7FFFFFFF && n * (k / 2) < 0x7FFFFFFF;
  if (dma)
    hipLaunchKernelGGL(gemm_kernel<true>, dim3((unsigned)tiles), dim3(kGemmThreads), 0, as_stream(stream), m, n, k,
                       a_codes, a_scales, b_codes, b_scales, c, ldc, accumulate);
  else
    hipLaunchKernelGGL(gemm_kernel<false>, dim3((unsigned)tiles), dim3(kGemmThreads), 0, as_stream(stream), m, n, k,
                       a_codes, a_scales, b_codes, b_scales, c, ldc, accumulate);
  return launch_status();
}

fp4_status fp4_swiglu_producer(int64_t t, int64_t f, int64_t d, const uint8_t* x_codes, const uint8_t* x_scales,
                               const uint8_t* w13_codes, const uint8_t* w13_scales, uint16_t* a_bf16,
                               uint16_t* b_bf16, uint8_t* h_codes, uint8_t* h_scales, uint8_t* ht_codes,
                               uint8_t* ht_scales, uint32_t sign_mask16, void* stream) {
  if (!x_codes || !x_scales || !w13_codes || !w13_scales || !a_bf16 || !b_bf16 || !h_codes || !h_scales)
    return FP4_EINVAL;
  if ((ht_codes == nullptr) != (ht_scales == nullptr)) return FP4_EINVAL;
  if (!mult32(t) || !mult32(f) || !mult32(d)) return FP4_ESHAPE;
  if (!aligned16(x_codes) || !aligned16(w13_codes) || !aligned16(h_codes) || !aligned16(x_scales) ||
      !aligned16(w13_scales) ||
      (ht_codes && !aligned16(ht_codes)))
    return FP4_EALIGN;
  const int64_t tiles = ((t + BM - 1) / BM) * ((f + 127) / 128);
  if (tiles > 0x7FFFFFFF) return FP4_ESHAPE;
  const bool dma = (d % 128) == 0 && t * (d / 2) < 0x7FFFFFFF && 2 * f * (d / 2) < 0x7FFFFFFF;
  if (dma)
    hipLaunchKernelGGL(swiglu_producer_kernel<true>, dim3((unsigned)tiles), dim3(kGemmThreads), 0, as_stream(stream),
                       t, f, d, x_codes, x_scales, w13_codes, w13_scales, a_bf16, b_bf16, h_codes, h_scales, ht_codes,
                       ht_scales, sign_mask16 & 0xFFFFu);
  else
    hipLaunchKernelGGL(swiglu_producer_kernel<false>, dim3((unsigned)tiles), dim3(kGemmThreads), 0, as_stream(stream),
                       t, f, d, x_codes, x_scales, w13_codes, w13_scales, a_bf16, b_bf16, h_codes, h_scales, ht_codes,
                       ht_scales, sign_mask16 & 0xFFFFu);
  return launch_status();
}

}  // extern "C"
