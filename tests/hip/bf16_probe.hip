// Test-only kernel (not part of libmxfp4): packs caller-chosen fp32 values
// with mx::bf16_pack2_rne, the rounding the SwiGLU producer and the backward
// producers apply to their fp32 results, so that a test can run it on every
// quiet NaN pattern and on chosen finite values and compare with the CPU
// oracle.  Lane i packs x[2i] (low half) and x[2i+1]; lanes past n do nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../precision_mxfp4_producers_amd/csrc/mx_device.h"

__global__ __launch_bounds__(256) void bf16_pack_probe_kernel(const float* __restrict__ x, uint32_t* __restrict__ out,
                                                              int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = mx::bf16_pack2_rne(x[2 * i], x[2 * i + 1]);
}

// x: 2n fp32 values, out: n words.  Returns the hipError_t of the launch.
extern "C" int bf16_pack_probe(const float* x, uint32_t* out, int64_t n, void* stream) {
  if (n <= 0 || !x || !out) return -1;
  const int64_t blocks = (n + 255) / 256;
  if (blocks > 0x7FFFFFFF) return -1;
  hipLaunchKernelGGL(bf16_pack_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     x, out, n);
  return (int)hipGetLastError();
}
