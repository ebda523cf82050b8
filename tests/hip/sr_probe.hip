// Test-only kernel (not part of libmxfp4): runs the producers' stochastic-
// rounding encoder, mx::sr_encode from the library's device header, on
// caller-chosen bf16 values, block exponents and 32-bit draws, so that a test
// can put each draw exactly at or next to its rounding threshold and compare
// the nibbles with the CPU oracle.  The producers draw their words from
// Philox, which no test can steer onto a threshold.
//
// Lane i encodes eight values (w[4i..4i+3], two bf16 per word) under block
// exponent e[i] with draws u[8i..8i+7]; out[i] gets the eight nibbles and
// exact[i] whether its wave took the exact form.  Lanes past n encode zeros.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../precision_mxfp4_producers_amd/csrc/mx_device.h"

__global__ __launch_bounds__(256) void sr_probe_kernel(const uint32_t* __restrict__ w, const int32_t* __restrict__ e,
                                                       const uint32_t* __restrict__ u, uint32_t* __restrict__ out,
                                                       uint32_t* __restrict__ exact, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool ok = i < n;
  uint32_t wv[4] = {0u, 0u, 0u, 0u};
  int ev = 0;
  if (ok) {
#pragma unroll
    for (int j = 0; j < 4; ++j) wv[j] = w[4 * i + j];
    ev = e[i];
  }
  uint32_t packed = 0;
  mx::sr_encode<4>(wv, ev, [&](int, uint32_t* uu) {
#pragma unroll
    for (int k = 0; k < 8; ++k) uu[k] = ok ? u[8 * i + k] : 0u;
  }, &packed);
  const bool took_exact = __builtin_amdgcn_ballot_w64(mx::sr_needs_exact<4>(wv, ev)) != 0;
  if (ok) {
    out[i] = packed;
    exact[i] = took_exact ? 1u : 0u;
  }
}

extern "C" int sr_probe(const uint32_t* w, const int32_t* e, const uint32_t* u, uint32_t* out, uint32_t* exact,
                        int64_t n, void* stream) {
  if (n <= 0) return 0;
  if (!w || !e || !u || !out || !exact || n > ((int64_t)1 << 30)) return -1;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(sr_probe_kernel, dim3(blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), w, e, u,
                     out, exact, n);
  return (int)hipGetLastError();
}

// The adjacent-bin rule alone on caller-chosen fp32 magnitudes y in [0, 6]
// (any fp32, as the CTA-local NVFP4 producers form them) and draws u:
// code[i] = mx::e2m1_sr(y[i], u[i], 0).
__global__ __launch_bounds__(256) void sr_y_probe_kernel(const float* __restrict__ y, const uint32_t* __restrict__ u,
                                                         uint32_t* __restrict__ code, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) code[i] = mx::e2m1_sr(y[i], u[i], 0u);
}

extern "C" int sr_y_probe(const float* y, const uint32_t* u, uint32_t* code, int64_t n, void* stream) {
  if (n <= 0) return 0;
  if (!y || !u || !code || n > ((int64_t)1 << 30)) return -1;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(sr_y_probe_kernel, dim3(blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), y, u, code,
                     n);
  return (int)hipGetLastError();
}
