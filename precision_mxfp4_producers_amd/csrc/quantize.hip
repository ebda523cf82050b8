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
// The RTN producers are HBM-bound: each reads its bf16 input once with
// coalesced 16-byte loads (the column, dual and 2D32 producers stage the tile
// in LDS and read it back by columns) and writes packed codes plus one scale
// byte per 32 values.  The SR producers are bound by the Philox draws.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "abi_common.h"
#include "mx_device.h"

namespace mx {

thread_local int g_last_hip_error = 0;

constexpr int kThreads = 256;
constexpr int kMaxGridY = 65535;
constexpr int64_t kMaxGridX = 0x7FFFFFFF;
constexpr int64_t kTargetBlocks = 8192;                  // 32 workgroups per CU

typedef int v4i __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ rows
// One lane quantizes 8 consecutive values (one 16-byte load); four lanes share
// a 32-value block and reduce its maximum over the quad (DPP).  bf16
// magnitudes are ordered like their 15-bit integer patterns, so the maximum
// is an integer max.  RTN goes through the hardware converter; SR draws
// Philox words for the lane's 8 elements (two counters).  Each pass of the
// row loop issues the loads of kRowsPerPass rows before using any of them.
constexpr int kRowsPerPass = 2;

// kIdx32 (SR only): the tensor holds at most 2^34 elements, so every Philox
// counter's second word is 0 (sr_words32).
template <bool kSR, bool kIdx32 = false>
__device__ __forceinline__ uint32_t encode_row_chunk(uint4 v, int e, int64_t r, int64_t cols, int64_t c8,
                                                     uint64_t seed, uint64_t offset) {
  if constexpr (kSR) {
    const uint64_t blk0 = ((uint64_t)r * (uint64_t)cols + (uint64_t)c8 * 8u) >> 2;   // first Philox counter
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t packed;
    sr_encode<4>(w, e, [&](int, uint32_t* u) {
      u32x4 a, b;
      if constexpr (kIdx32) {
        a = sr_words32((uint32_t)blk0, seed, offset);
        b = sr_words32((uint32_t)blk0 + 1u, seed, offset);
      } else {
        a = sr_words(blk0, seed, offset);
        b = sr_words(blk0 + 1u, seed, offset);
      }
      u[0] = a.x; u[1] = a.y; u[2] = a.z; u[3] = a.w; u[4] = b.x; u[5] = b.y; u[6] = b.z; u[7] = b.w;
    }, &packed);
    return packed;
  } else {
    return rtn8_bf16(v.x, v.y, v.z, v.w, pow2_scale(e));
  }
}

template <bool kSR, bool kIdx32 = false>
__global__ __launch_bounds__(kThreads) void quant_rows_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint64_t seed, uint64_t offset) {
  const int64_t cpr = cols >> 3;                         // 8-value chunks per row
  const int64_t c8 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const bool col_ok = c8 < cpr;                          // quads are all-in or all-out
  const int64_t rstep = gridDim.y;
  for (int64_t r0 = blockIdx.y; r0 < rows; r0 += kRowsPerPass * rstep) {
    uint4 v[kRowsPerPass];
#pragma unroll
    for (int j = 0; j < kRowsPerPass; ++j) {
      const int64_t r = r0 + j * rstep;
      v[j] = make_uint4(0u, 0u, 0u, 0u);
      if (col_ok && r < rows) v[j] = load_once_u4(x + r * ldx + c8 * 8);
    }
#pragma unroll
    for (int j = 0; j < kRowsPerPass; ++j) {
      const int64_t r = r0 + j * rstep;
      const uint32_t m = max_quad(bf16_absmax8(v[j].x, v[j].y, v[j].z, v[j].w));
      const int e = upward_exp(m << 16);
      if (col_ok && r < rows) {
        const uint32_t packed = encode_row_chunk<kSR, kIdx32>(v[j], e, r, cols, c8, seed, offset);
        *reinterpret_cast<uint32_t*>(codes + r * (cols >> 1) + c8 * 4) = packed;
        if ((c8 & 3) == 0) scales[r * (cols >> 5) + (c8 >> 2)] = (uint8_t)(e + 127);
      }
    }
  }
}

// ------------------------------------------------------------------ cols
// A workgroup owns kColTok tokens x kColW columns: it loads the bf16 tile
// row-contiguously into LDS, encodes column pairs from LDS (optional H32 per
// 32-token block), parks the codes in LDS and writes each column's kColTok/2
// code bytes as one contiguous run with coalesced 16-byte stores (16-byte
// pieces of many lines per store instruction drain at a fraction of the rate).
// 128 x 128 measured best among 128-512 tokens x 32-128 columns on one MI355X
// (it trades whole 128-byte code lines for more workgroups per CU).
#ifndef MX_COL_TOK
#define MX_COL_TOK 128
#endif
#ifndef MX_COL_W
#define MX_COL_W 128
#endif
constexpr int kColTok = MX_COL_TOK, kColW = MX_COL_W;
constexpr int kColChunks = kColW / 8;                    // 16-byte chunks per token row
constexpr int kColRowsPerLoad = kThreads / kColChunks;   // token rows one load instruction round covers
constexpr int kColPitch = kColW * 2 + 16;                // bytes per staged token row (16-byte aligned rows)
constexpr int kColCodePitch = kColTok / 2 + 16;          // bytes per staged column of codes
static_assert(kColTok % kColRowsPerLoad == 0 && kColTok % 32 == 0 && kColW % 32 == 0, "column tile shape");
static_assert((kColW / 2) * (kColTok / 32) == kThreads, "one column item per lane");
static_assert(kColW * kColCodePitch <= kColTok * kColPitch, "column codes fit in the tile buffer");

template <bool kH32>
__global__ __launch_bounds__(kThreads) void quant_cols_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
    uint8_t* __restrict__ codes_t, uint8_t* __restrict__ scales_t, uint32_t sign_mask16) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kColTok * kColPitch];
  __shared__ uint8_t stile[kColW][kColTok / 32];
  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * kColW, t0 = (int64_t)blockIdx.y * kColTok;
  const int ntok = (int)min<int64_t>(kColTok, rows - t0);          // multiple of 32
  const int ncol = (int)min<int64_t>(kColW, cols - c0);            // multiple of 32

  // load: thread (row tid/kColChunks + kColRowsPerLoad j, 16-byte chunk tid%kColChunks)
  {
    constexpr int kJ = kColTok / kColRowsPerLoad;
    const int ch = tid % kColChunks;
    const bool col_ok = ch * 8 < ncol;
    uint4 v[kJ];
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int r = tid / kColChunks + kColRowsPerLoad * j;
      v[j] = make_uint4(0u, 0u, 0u, 0u);
      if (col_ok && r < ntok) v[j] = load_once_u4(x + (t0 + r) * ldx + c0 + ch * 8);
    }
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int r = tid / kColChunks + kColRowsPerLoad * j;
      *reinterpret_cast<uint4*>(tile + r * kColPitch + ch * 16) = v[j];
    }
  }
  __syncthreads();

  // encode: one item (column pair tid % (kColW/2), token block tid / (kColW/2))
  // per lane; the codes are kept in registers until every lane has read its
  // values, then parked in the tile buffer (one LDS array: four workgroups
  // per CU)
  const int cp = tid % (kColW / 2), tb = tid / (kColW / 2);
  const bool live = 2 * cp < ncol && 32 * tb < ntok;
  uint4 code[2];
  int ex[2];
  {
    uint32_t v[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) v[k] = *reinterpret_cast<const uint32_t*>(tile + (32 * tb + k) * kColPitch + cp * 4);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float f[32];
      h32_column(v, c, kH32 ? sign_mask16 : 0u, f);     // d_(k mod 16) with H32
      if constexpr (kH32) h32_fp32(f);
      code[c] = encode32_rtn(f, ex[c]);
    }
  }
  __syncthreads();
  uint8_t* ctile = tile;
  if (live) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      *reinterpret_cast<uint4*>(ctile + (2 * cp + c) * kColCodePitch + tb * 16) = code[c];
      stile[2 * cp + c][tb] = (uint8_t)(ex[c] + 127);
    }
  }
  __syncthreads();

  // store: consecutive threads cover one column's kColTok/2 code bytes (one
  // whole 128-byte line when kColTok == 256); then one thread per column
  // writes its scale bytes
  constexpr int kPieces = kColTok / 32;                  // 16-byte pieces per column
  for (int i = tid; i < kColW * kPieces; i += kThreads) {
    const int col = i / kPieces, piece = i % kPieces;
    if (col < ncol && piece * 32 < ntok) {
      const uint4 d = *reinterpret_cast<const uint4*>(ctile + col * kColCodePitch + piece * 16);
      *reinterpret_cast<uint4*>(codes_t + (c0 + col) * (rows >> 1) + (t0 >> 1) + piece * 16) = d;
    }
  }
  for (int col = tid; col < ncol; col += kThreads) {
    uint8_t* dst = scales_t + (c0 + col) * (rows >> 5) + (t0 >> 5);
    for (int tb = 0; tb < ntok / 32; ++tb) dst[tb] = stile[col][tb];
  }
}

// ------------------------------------------------------------------ dual (rows + cols, one read)
// Both views of one tensor from a single read (the dY of a linear layer: row
// SR for Dgrad, column H32 for Wgrad).  A workgroup stages kDualTok tokens x
// kDualW columns of bf16 in LDS, then
//   rows: lane (row ci/32, 8-value chunk ci%32) encodes with the rows
//         kernel's own code (quad max, SR words of the element's row-major
//         index); a wave stores two whole 128-byte code lines;
//   cols: as the column kernel (column pairs x 32-token blocks, optional H32),
//         codes staged in the tile buffer once every lane has read its values,
//         then stored as 64-byte runs per column.
// Bytes are those of fp4_quantize_rows and fp4_quantize_cols on the same
// tensor: the same per-block encoders run on the same values.
constexpr int kDualTok = 128, kDualW = 256;
constexpr int kDualThreads = 512;                        // one column item per lane
constexpr int kDualPitch = kDualW * 2 + 16;              // bytes per staged token row (16-byte aligned rows)
constexpr int kDualCodePitch = kDualTok / 2 + 16;        // bytes per staged column of codes
static_assert(kDualW * kDualCodePitch <= kDualTok * kDualPitch, "column codes fit in the tile buffer");

template <bool kSR, bool kH32, bool kIdx32 = false>
__global__ __launch_bounds__(kDualThreads) void quant_dual_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* __restrict__ row_codes,
    uint8_t* __restrict__ row_scales, uint64_t seed, uint64_t offset, uint8_t* __restrict__ codes_t,
    uint8_t* __restrict__ scales_t, uint32_t sign_mask16) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kDualTok * kDualPitch];
  __shared__ uint8_t stile[kDualW][kDualTok / 32];
  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * kDualW, t0 = (int64_t)blockIdx.y * kDualTok;
  const int ntok = (int)min<int64_t>(kDualTok, rows - t0);         // multiple of 32
  const int ncol = (int)min<int64_t>(kDualW, cols - c0);           // multiple of 32

  // load: thread (row tid/32 + 16j, 16-byte chunk tid%32); rows beyond the
  // tensor and chunks beyond its columns stage zeros (never encoded)
  {
    constexpr int kJ = kDualTok / (kDualThreads / 32);
    const int ch = tid & 31;
    const bool col_ok = ch * 8 < ncol;
#pragma unroll
    for (int j0 = 0; j0 < kJ; j0 += 4) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = (tid >> 5) + (kDualThreads / 32) * (j0 + u);
        v[u] = make_uint4(0u, 0u, 0u, 0u);
        if (col_ok && r < ntok) v[u] = load_once_u4(x + (t0 + r) * ldx + c0 + ch * 8);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = (tid >> 5) + (kDualThreads / 32) * (j0 + u);
        *reinterpret_cast<uint4*>(tile + r * kDualPitch + ch * 16) = v[u];
      }
    }
  }
  __syncthreads();

  // rows: 128 rows x 32 chunks; a quad covers one 32-value block
  {
#pragma unroll 2
    for (int k = 0; k < kDualTok * 32 / kDualThreads; ++k) {
      const int ci = tid + k * kDualThreads;
      const int r = ci >> 5, ch = ci & 31;
      const uint4 v = *reinterpret_cast<const uint4*>(tile + r * kDualPitch + ch * 16);
      const uint32_t m = max_quad(bf16_absmax8(v.x, v.y, v.z, v.w));
      const int e = upward_exp(m << 16);
      if (r < ntok && ch * 8 < ncol) {
        const int64_t gr = t0 + r, c8 = (c0 >> 3) + ch;
        const uint32_t packed = encode_row_chunk<kSR, kIdx32>(v, e, gr, cols, c8, seed, offset);
        *reinterpret_cast<uint32_t*>(row_codes + gr * (cols >> 1) + c8 * 4) = packed;
        if ((ch & 3) == 0) row_scales[gr * (cols >> 5) + (c8 >> 2)] = (uint8_t)(e + 127);
      }
    }
  }

  // cols: items (column pair, token block); all lanes read before any code
  // overwrites the tile
  constexpr int kItems = (kDualW / 2) * (kDualTok / 32);
  static_assert(kItems == kDualThreads, "one column item per lane");
  uint4 code[1][2];
  int ex[1][2];
  bool live[1];
#pragma unroll
  for (int u = 0; u < 1; ++u) {
    const int i = tid + u * kDualThreads;
    const int cp = i % (kDualW / 2), tb = i / (kDualW / 2);
    live[u] = 2 * cp < ncol && 32 * tb < ntok;
    uint32_t v[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) v[k] = *reinterpret_cast<const uint32_t*>(tile + (32 * tb + k) * kDualPitch + cp * 4);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float f[32];
      h32_column(v, c, kH32 ? sign_mask16 : 0u, f);     // d_(k mod 16) with H32
      if constexpr (kH32) h32_fp32(f);
      code[u][c] = encode32_rtn(f, ex[u][c]);
    }
  }
  __syncthreads();
  uint8_t* ctile = tile;
#pragma unroll
  for (int u = 0; u < 1; ++u) {
    const int i = tid + u * kDualThreads;
    const int cp = i % (kDualW / 2), tb = i / (kDualW / 2);
    if (live[u]) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        *reinterpret_cast<uint4*>(ctile + (2 * cp + c) * kDualCodePitch + tb * 16) = code[u][c];
        stile[2 * cp + c][tb] = (uint8_t)(ex[u][c] + 127);
      }
    }
  }
  __syncthreads();
  constexpr int kPieces = kDualTok / 32;                 // 16-byte pieces per column
  for (int i = tid; i < kDualW * kPieces; i += kDualThreads) {
    const int col = i / kPieces, piece = i % kPieces;
    if (col < ncol && piece * 32 < ntok) {
      const uint4 d = *reinterpret_cast<const uint4*>(ctile + col * kDualCodePitch + piece * 16);
      *reinterpret_cast<uint4*>(codes_t + (c0 + col) * (rows >> 1) + (t0 >> 1) + piece * 16) = d;
    }
  }
  for (int col = tid; col < ncol; col += kDualThreads) {
    uint8_t* dst = scales_t + (c0 + col) * (rows >> 5) + (t0 >> 5);
    for (int tb = 0; tb < ntok / 32; ++tb) dst[tb] = stile[col][tb];
  }
}

// ------------------------------------------------------------------ 2D32
// A 256-lane workgroup walks consecutive 128x128 weight macro tiles (4x4 tiles
// of 32x32) along K; the loads of the next macro tile are in flight while the
// current one is encoded.  Wave w holds tile-row w: lane l loads rows
// 4q + l/16 (q = 0..7) of it, 8 values at column chunk l%16, so each load
// covers four whole 256-byte row segments and each lane's values lie in
// tile l%16/4.  A tile maximum is a reduction over the lane's rows, its quad
// and lane bits 4-5.  Row codes go out from registers as 64-byte runs per row;
// the bf16 tile is staged in LDS, re-read by columns with the same tile
// exponent (the encoding is a pure function of value and exponent, so both
// layouts hold the same nibble), and the column codes are staged again so
// that four lanes write each column's 64 bytes together.
constexpr int kWPitch = 68;                              // dwords per staged bf16 row (64 + 4 pad)
constexpr int kWCodePitch = 80;                          // bytes per staged column of codes (64 + 16 pad)

// Loads of macro tile (n0, k0) through the strip's buffer resource (rows >= N
// and columns >= K read zero).
__device__ __forceinline__ void w2d32_load(__amdgpu_buffer_rsrc_t rs, int64_t N, int64_t K, int64_t ldw,
                                           int64_t n0, int64_t k0, uint32_t (&v)[32]) {
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

__device__ __forceinline__ void w2d32_tile(const uint32_t (&v)[32], int64_t N, int64_t K, int64_t n0, int64_t k0,
                                           uint8_t* __restrict__ row_codes, uint8_t* __restrict__ row_scales,
                                           uint8_t* __restrict__ col_codes, uint8_t* __restrict__ col_scales,
                                           float finer_ratio, uint32_t* tile, uint8_t* ccodes, int (*tile_e)[4]) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int t = (l & 15) >> 2;                           // this lane's tile within the tile-row
  const int64_t col = k0 + (l & 15) * 8;
  const bool tile_ok = n0 + 32 * w < N && k0 + 32 * t < K;
  // tile maximum (bf16 magnitude patterns): own 8 rows, quad, lane bits 4-5
  uint32_t m = 0;
#pragma unroll
  for (int q = 0; q < 8; ++q) m = max(m, bf16_absmax8(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]));
  m = max_quad(m);
  m = max(m, (uint32_t)__shfl_xor((int)m, 16));
  m = max(m, (uint32_t)__shfl_xor((int)m, 32));
  const uint32_t ab = m << 16;
  const int e_up = upward_exp(ab);
  const float lhs = __uint_as_float(ab) * inv_pow2(e_up);          // exact, in (3, 6]
  const bool finer = ((double)lhs < 6.0 * (double)finer_ratio) && e_up > -127;
  const int e = finer ? e_up - 1 : e_up;
  if (l < 16 && (l & 3) == 0) tile_e[w][t] = e;
  // stage the bf16 values for the column pass
#pragma unroll
  for (int q = 0; q < 8; ++q)
    *reinterpret_cast<uint4*>(&tile[(32 * w + 4 * q + (l >> 4)) * kWPitch + (l & 15) * 4]) =
        make_uint4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  // row layout from registers: 16 lanes write 64 contiguous bytes of a row
  if (tile_ok) {
    const float sc = pow2_scale(e);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int64_t row = n0 + 32 * w + 4 * q + (l >> 4);
      *reinterpret_cast<uint32_t*>(row_codes + row * (K >> 1) + (col >> 1)) =
          rtn8_bf16(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3], sc);
      if ((l & 3) == 0) row_scales[row * (K >> 5) + (col >> 5)] = (uint8_t)(e + 127);
    }
  }
  __syncthreads();

  // column pass: wave q = tile-row, lane = column pair; codes staged per column
  {
    const int qr = w, pcol = l;                          // columns 2*pcol, 2*pcol+1
    const int tc = pcol >> 4;
    const int et = tile_e[qr][tc];
    const float sc = pow2_scale(et);
    uint32_t d[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) d[i] = tile[(32 * qr + i) * kWPitch + pcol];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint32_t sel = c ? 0x07060302u : 0x05040100u;
      uint32_t pr[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) pr[j] = __builtin_amdgcn_perm(d[2 * j + 1], d[2 * j], sel);
      *reinterpret_cast<uint4*>(ccodes + (2 * pcol + c) * kWCodePitch + qr * 16) =
          make_uint4(rtn8_bf16(pr[0], pr[1], pr[2], pr[3], sc), rtn8_bf16(pr[4], pr[5], pr[6], pr[7], sc),
                     rtn8_bf16(pr[8], pr[9], pr[10], pr[11], sc), rtn8_bf16(pr[12], pr[13], pr[14], pr[15], sc));
    }
  }
  __syncthreads();
  // column codes out: piece p = (column p/4, tile-row p%4), four lanes per column
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int p = tid + 256 * k, kc = p >> 2, qr = p & 3;
    if (k0 + kc < K && n0 + 32 * qr < N) {
      *reinterpret_cast<uint4*>(col_codes + (k0 + kc) * (N >> 1) + (n0 >> 1) + qr * 16) =
          *reinterpret_cast<const uint4*>(ccodes + kc * kWCodePitch + qr * 16);
      col_scales[(k0 + kc) * (N >> 5) + (n0 >> 5) + qr] = (uint8_t)(tile_e[qr][kc >> 5] + 127);
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kThreads) void quant_w2d32_kernel(
    const uint16_t* __restrict__ w, int64_t N, int64_t K, int64_t ldw,
    uint8_t* __restrict__ row_codes, uint8_t* __restrict__ row_scales,
    uint8_t* __restrict__ col_codes, uint8_t* __restrict__ col_scales, float finer_ratio, int per) {
  __shared__ __attribute__((aligned(16))) uint32_t tile[128 * kWPitch];
  __shared__ __attribute__((aligned(16))) uint8_t ccodes[128 * kWCodePitch];
  __shared__ int tile_e[4][4];
  // neighbouring 128-row strips write the two halves of each column-code
  // line: keep them on one XCD
  uint32_t bx, by;
  xcd_block(1, bx, by);
  const int64_t n0 = (int64_t)by * 128;
  const int64_t gk = (K + 127) / 128;
  int64_t kt = (int64_t)bx * per;
  const int64_t kt_end = min(gk, kt + per);
  if (kt >= kt_end) return;                              // uniform over the workgroup
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(w + n0 * ldw, (std::min<int64_t>(128, N - n0) - 1) * ldw * 2 + K * 2);
  // ping-pong register buffers (a copy between them would wait for the loads)
  uint32_t v0[32], v1[32];
  w2d32_load(rs, N, K, ldw, n0, kt * 128, v0);
  for (;;) {
    // next macro tile of this run; on the last pass the current one again
    // (a cached re-read keeps the loads unconditional)
    int64_t kn = kt + 1 < kt_end ? kt + 1 : kt;
    w2d32_load(rs, N, K, ldw, n0, kn * 128, v1);
    w2d32_tile(v0, N, K, n0, kt * 128, row_codes, row_scales, col_codes, col_scales, finer_ratio, tile, ccodes, tile_e);
    if (++kt >= kt_end) break;
    kn = kt + 1 < kt_end ? kt + 1 : kt;
    w2d32_load(rs, N, K, ldw, n0, kn * 128, v0);
    w2d32_tile(v1, N, K, n0, kt * 128, row_codes, row_scales, col_codes, col_scales, finer_ratio, tile, ccodes, tile_e);
    if (++kt >= kt_end) break;
  }
}

}  // namespace mx

using namespace mx;

extern "C" {

fp4_status fp4_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                             uint8_t* codes, uint8_t* scales, fp4_round mode, uint64_t seed,
                             uint64_t offset, hipStream_t stream) {
  if (mode != FP4_RTN && mode != FP4_SR) return FP4_EINVAL;
  if (rows < 0 || !mult32z(cols) || ldx < cols) return FP4_ESHAPE;
  if (rows == 0 || cols == 0) return FP4_OK;             // empty: nothing to write
  if (!x || !codes || !scales) return FP4_EINVAL;
  if (!aligned16(x) || !aligned16(codes) || (ldx % 8) != 0) return FP4_EALIGN;
  const int64_t cpr = cols >> 3;
  const int64_t gx = (cpr + kThreads - 1) / kThreads;
  if (gx > kMaxGridX) return FP4_ESHAPE;
  // about kTargetBlocks workgroups, each taking whole passes of kRowsPerPass rows
  int64_t gy = std::max<int64_t>(1, kTargetBlocks / gx);
  gy = std::min<int64_t>(gy, (rows + kRowsPerPass - 1) / kRowsPerPass);
  gy = std::min<int64_t>(gy, kMaxGridY);
  dim3 grid((unsigned)gx, (unsigned)gy);
  hipStream_t s = as_stream(stream);
  if (mode == FP4_SR && rows <= (int64_t(1) << 34) / cols)   // counters below 2^32
    hipLaunchKernelGGL((quant_rows_kernel<true, true>), grid, dim3(kThreads), 0, s, x, rows, cols, ldx, codes,
                       scales, seed, offset);
  else if (mode == FP4_SR)
    hipLaunchKernelGGL(quant_rows_kernel<true>, grid, dim3(kThreads), 0, s, x, rows, cols, ldx, codes,
                       scales, seed, offset);
  else
    hipLaunchKernelGGL(quant_rows_kernel<false>, grid, dim3(kThreads), 0, s, x, rows, cols, ldx, codes,
                       scales, seed, offset);
  return launch_status();
}

fp4_status fp4_quantize_cols(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                             uint8_t* codes_t, uint8_t* scales_t, int hadamard,
                             uint32_t sign_mask16, hipStream_t stream) {
  if (hadamard != 0 && hadamard != 32) return FP4_EINVAL;
  if (!mult32z(rows) || !mult32z(cols) || ldx < cols) return FP4_ESHAPE;
  if (rows == 0 || cols == 0) return FP4_OK;
  if (!x || !codes_t || !scales_t) return FP4_EINVAL;
  if (!aligned16(x) || !aligned16(codes_t) || (ldx % 8) != 0) return FP4_EALIGN;
  const int64_t gx = (cols + kColW - 1) / kColW, gy = (rows + kColTok - 1) / kColTok;
  if (gy > kMaxGridY || gx > kMaxGridX) return FP4_ESHAPE;
  dim3 grid((unsigned)gx, (unsigned)gy);
  hipStream_t s = as_stream(stream);
  if (hadamard == 32)
    hipLaunchKernelGGL(quant_cols_kernel<true>, grid, dim3(kThreads), 0, s, x, rows, cols, ldx, codes_t,
                       scales_t, sign_mask16 & 0xFFFFu);
  else
    hipLaunchKernelGGL(quant_cols_kernel<false>, grid, dim3(kThreads), 0, s, x, rows, cols, ldx, codes_t,
                       scales_t, 0u);
  return launch_status();
}

fp4_status fp4_quantize_dual(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                             uint8_t* row_codes, uint8_t* row_scales, fp4_round mode, uint64_t seed, uint64_t offset,
                             uint8_t* codes_t, uint8_t* scales_t, int hadamard, uint32_t sign_mask16,
                             hipStream_t stream) {
  if (mode != FP4_RTN && mode != FP4_SR) return FP4_EINVAL;
  if (hadamard != 0 && hadamard != 32) return FP4_EINVAL;
  if (!mult32z(rows) || !mult32z(cols) || ldx < cols) return FP4_ESHAPE;
  if (rows == 0 || cols == 0) return FP4_OK;
  if (!x || !row_codes || !row_scales || !codes_t || !scales_t) return FP4_EINVAL;
  if (!aligned16(x) || !aligned16(row_codes) || !aligned16(codes_t) || (ldx % 8) != 0) return FP4_EALIGN;
  const int64_t gx = (cols + kDualW - 1) / kDualW, gy = (rows + kDualTok - 1) / kDualTok;
  if (gy > kMaxGridY || gx > kMaxGridX) return FP4_ESHAPE;
  dim3 grid((unsigned)gx, (unsigned)gy);
  hipStream_t s = as_stream(stream);
  const uint32_t m16 = hadamard == 32 ? (sign_mask16 & 0xFFFFu) : 0u;
  const bool idx32 = rows <= (int64_t(1) << 34) / cols;  // counters below 2^32
  if (mode == FP4_SR && hadamard == 32 && idx32)
    hipLaunchKernelGGL((quant_dual_kernel<true, true, true>), grid, dim3(kDualThreads), 0, s, x, rows, cols, ldx,
                       row_codes, row_scales, seed, offset, codes_t, scales_t, m16);
  else if (mode == FP4_SR && hadamard == 32)
    hipLaunchKernelGGL((quant_dual_kernel<true, true>), grid, dim3(kDualThreads), 0, s, x, rows, cols, ldx, row_codes,
                       row_scales, seed, offset, codes_t, scales_t, m16);
  else if (mode == FP4_SR && idx32)
    hipLaunchKernelGGL((quant_dual_kernel<true, false, true>), grid, dim3(kDualThreads), 0, s, x, rows, cols, ldx,
                       row_codes, row_scales, seed, offset, codes_t, scales_t, m16);
  else if (mode == FP4_SR)
    hipLaunchKernelGGL((quant_dual_kernel<true, false>), grid, dim3(kDualThreads), 0, s, x, rows, cols, ldx, row_codes,
                       row_scales, seed, offset, codes_t, scales_t, m16);
  else if (hadamard == 32)
    hipLaunchKernelGGL((quant_dual_kernel<false, true>), grid, dim3(kDualThreads), 0, s, x, rows, cols, ldx, row_codes,
                       row_scales, seed, offset, codes_t, scales_t, m16);
  else
    hipLaunchKernelGGL((quant_dual_kernel<false, false>), grid, dim3(kDualThreads), 0, s, x, rows, cols, ldx, row_codes,
                       row_scales, seed, offset, codes_t, scales_t, m16);
  return launch_status();
}

fp4_status fp4_quantize_w2d32(const uint16_t* w, int64_t n, int64_t k, int64_t ldw,
                              uint8_t* row_codes, uint8_t* row_scales, uint8_t* col_codes,
                              uint8_t* col_scales, float finer_ratio, hipStream_t stream) {
  if (!(finer_ratio >= 0.0f && finer_ratio <= 1.0f)) return FP4_EINVAL;
  if (!mult32z(n) || !mult32z(k) || ldw < k) return FP4_ESHAPE;
  if (n == 0 || k == 0) return FP4_OK;
  if (!w || !row_codes || !row_scales || !col_codes || !col_scales) return FP4_EINVAL;
  if (!aligned16(w) || !aligned16(row_codes) || !aligned16(col_codes) || (ldw % 8) != 0)
    return FP4_EALIGN;
  const int64_t gk = (k + 127) / 128, gy = (n + 127) / 128;
  if (gy > kMaxGridY || ldw >= ((int64_t)1 << 22)) return FP4_ESHAPE;   // 128-row strips stay < 2 GiB
  // about 512 workgroups (2 per CU, each long-running), each walking a run of
  // consecutive macro tiles along K (three per CU, with the registers held to
  // 168 per lane, measured 10-15% slower on 8192-14336 x 4096)
  const int64_t want_x = std::max<int64_t>(1, 512 / gy);
  const int per = (int)((gk + want_x - 1) / want_x);
  const int64_t gx = (gk + per - 1) / per;
  hipLaunchKernelGGL(quant_w2d32_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0,
                     as_stream(stream), w, n, k, ldw, row_codes, row_scales, col_codes, col_scales,
                     finer_ratio, per);
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

int fp4_abi_version(void) { return (1 << 16) | 4; }

}  // extern "C"
