// Elementwise SwiGLU backward (gated FFN of "Format-Aware Fusion for Fast FP4
// Pretraining", §3.2): from the fp32 W2 data gradient dH and the saved bf16
// gate/up outputs a, b,
//   sig = 1/(1+exp(-a)), s = a*sig
//   dA = bf16(((dH*b)*sig) * (1 + a*(1 - sig))),  dB = bf16(dH*s)
// with single fp32 roundings in this order and no FMA.  HBM-bound: 12 bytes
// per element (4 read dH, 2+2 read a/b, 2+2 written dA/dB).
#include <hip/hip_runtime.h>

#include "abi_common.h"
#include "mx_device.h"

namespace mx {

constexpr int kBwdThreads = 256;
constexpr int kMaxGridY = 65535;

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
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float af = bf16_bits_to_f32((aw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
      const float bf = bf16_bits_to_f32((bw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
      float sig, s;
      sigmoid_silu(af, sig, s);
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

}  // namespace mx

using namespace mx;

extern "C" fp4_status fp4_swiglu_backward(int64_t t, int64_t f, const float* dh, int64_t lddh,
                                          const uint16_t* a_bf16, const uint16_t* b_bf16, uint16_t* da_bf16,
                                          uint16_t* db_bf16, void* stream) {
  if (!dh || !a_bf16 || !b_bf16 || !da_bf16 || !db_bf16) return FP4_EINVAL;
  if (!mult32(t) || !mult32(f) || lddh < f) return FP4_ESHAPE;
  if (!aligned16(dh) || !aligned16(a_bf16) || !aligned16(b_bf16) || !aligned16(da_bf16) || !aligned16(db_bf16) ||
      (lddh % 4) != 0)
    return FP4_EALIGN;
  const int64_t cpr = f >> 3;
  dim3 grid((unsigned)((cpr + kBwdThreads - 1) / kBwdThreads), (unsigned)(t < kMaxGridY ? t : kMaxGridY));
  hipLaunchKernelGGL(swiglu_bwd_kernel, grid, dim3(kBwdThreads), 0, as_stream(stream), t, f, dh, lddh, a_bf16,
                     b_bf16, da_bf16, db_bf16);
  return launch_status();
}
