// Streaming reference for the producers' bandwidth (measurement only, not
// part of the library's ABI): reads a bf16 tensor once with 16-byte loads and
// writes the traffic of a one-orientation MXFP4 producer -- half a byte per
// value (here the top nibble of each bf16 pattern, eight per 32-bit store, so
// a wave's store covers two whole 128-byte lines) and one byte per 32 values
// -- with the same grid-stride shape and loads in flight as the row
// producer, but no rounding work.  Its time is what a plain streaming kernel
// with 2.53125 bytes per value reaches at a given size.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace {

constexpr int kThreads = 256;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t nibbles8(u32x4 a) {
  return ((a.x >> 12) & 0xFu) | ((a.x >> 24) & 0xF0u) | (((a.y >> 12) & 0xFu) << 8) | (((a.y >> 28) & 0xFu) << 12) |
         (((a.z >> 12) & 0xFu) << 16) | (((a.z >> 28) & 0xFu) << 20) | (((a.w >> 12) & 0xFu) << 24) |
         ((a.w >> 28) << 28);
}

__global__ __launch_bounds__(kThreads) void stream_ref_kernel(const u32x4* __restrict__ x, int64_t chunks,
                                                            uint32_t* __restrict__ out, uint8_t* __restrict__ side) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + stride < chunks; i += 2 * stride) {
    const u32x4 a = __builtin_nontemporal_load(x + i), b = __builtin_nontemporal_load(x + i + stride);
    out[i] = nibbles8(a);
    out[i + stride] = nibbles8(b);
    if ((i & 3) == 0) side[i >> 2] = (uint8_t)(a.x >> 8);
    if (((i + stride) & 3) == 0) side[(i + stride) >> 2] = (uint8_t)(b.x >> 8);
  }
  for (; i < chunks; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(x + i);
    out[i] = nibbles8(a);
    if ((i & 3) == 0) side[i >> 2] = (uint8_t)(a.x >> 8);
  }
}

}  // namespace

// x: n bf16 values (n a multiple of 32, 16-byte aligned); out: n/2 bytes;
// side: n/32 bytes.  Returns the hipError_t of the launch.
extern "C" int mxfp4_stream_reference(const void* x, int64_t n, void* out, void* side, void* stream) {
  if (n <= 0 || (n % 32) != 0 || !x || !out || !side) return -1;
  const int64_t chunks = n / 8;
  const int64_t blocks = std::min<int64_t>((chunks + kThreads - 1) / kThreads, 8192);
  hipLaunchKernelGGL(stream_ref_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const u32x4*>(x), chunks,
                     reinterpret_cast<uint32_t*>(out), reinterpret_cast<uint8_t*>(side));
  return (int)hipGetLastError();
}
