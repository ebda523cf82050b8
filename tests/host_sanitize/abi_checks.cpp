// Host-side argument checks of every entry point, built together with the
// library sources under AddressSanitizer and UndefinedBehaviorSanitizer (host
// code only; no kernel is launched, no GPU is needed).  Each call below must
// return its documented status from the host checks alone: invalid
// arguments, empty calls and the launch-shape limits.  Exit status 0 when all
// match; the sanitizers abort on any out-of-bounds access, signed overflow or
// other undefined behaviour in the checks.
#include <stdint.h>
#include <stdio.h>

#include "../../include/mxfp4.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
  if (got != want) {
    fprintf(stderr, "%s: got %d want %d\n", what, got, want);
    ++failures;
  }
}

int main() {
  void* p = reinterpret_cast<void*>(4096);               // never dereferenced
  void* odd = reinterpret_cast<void*>(4098);
  uint16_t* x = static_cast<uint16_t*>(p);
  uint8_t* b = static_cast<uint8_t*>(p);
  float* c = static_cast<float*>(p);
  const int64_t big = (int64_t)1 << 40, huge_rows = (int64_t)65536 * 128;

  expect("rows null", fp4_quantize_rows(nullptr, 32, 32, 32, nullptr, nullptr, static_cast<fp4_round>(0), 0, 0, nullptr), FP4_EINVAL);
  expect("rows shape", fp4_quantize_rows(x, 32, 33, 40, b, b, static_cast<fp4_round>(0), 0, 0, nullptr), FP4_ESHAPE);
  expect("rows align", fp4_quantize_rows(static_cast<uint16_t*>(odd), 32, 32, 32, b, b, static_cast<fp4_round>(0), 0, 0, nullptr), FP4_EALIGN);
  expect("rows mode", fp4_quantize_rows(x, 32, 32, 32, b, b, static_cast<fp4_round>(7), 0, 0, nullptr), FP4_EINVAL);
  expect("rows negative", fp4_quantize_rows(nullptr, -1, 64, 64, nullptr, nullptr, static_cast<fp4_round>(0), 0, 0, nullptr), FP4_ESHAPE);
  expect("rows empty", fp4_quantize_rows(nullptr, 0, 64, 64, nullptr, nullptr, static_cast<fp4_round>(1), 0, 0, nullptr), FP4_OK);
  expect("rows huge cols", fp4_quantize_rows(x, 32, big * 32, big * 32, b, b, static_cast<fp4_round>(0), 0, 0, nullptr), FP4_ESHAPE);
  expect("cols shape", fp4_quantize_cols(x, 48, 32, 32, b, b, 0, 0, nullptr), FP4_ESHAPE);
  expect("cols hadamard", fp4_quantize_cols(x, 32, 32, 32, b, b, 16, 0, nullptr), FP4_EINVAL);
  expect("cols limit", fp4_quantize_cols(x, huge_rows, 32, 32, b, b, 32, 0, nullptr), FP4_ESHAPE);
  expect("cols huge cols", fp4_quantize_cols(x, 32, big * 512, big * 512, b, b, 32, 0, nullptr), FP4_ESHAPE);
  expect("cols empty", fp4_quantize_cols(nullptr, 64, 0, 0, nullptr, nullptr, 0, 0, nullptr), FP4_OK);
  expect("dual shape", fp4_quantize_dual(x, 48, 32, 32, b, b, static_cast<fp4_round>(1), 0, 0, b, b, 32, 0, nullptr), FP4_ESHAPE);
  expect("dual mode", fp4_quantize_dual(x, 32, 32, 32, b, b, static_cast<fp4_round>(3), 0, 0, b, b, 32, 0, nullptr), FP4_EINVAL);
  expect("dual null", fp4_quantize_dual(x, 32, 32, 32, b, b, static_cast<fp4_round>(1), 0, 0, nullptr, b, 32, 0, nullptr), FP4_EINVAL);
  expect("dual limit", fp4_quantize_dual(x, huge_rows, 32, 32, b, b, static_cast<fp4_round>(1), 0, 0, b, b, 32, 0, nullptr), FP4_ESHAPE);
  expect("w2d32 ld", fp4_quantize_w2d32(x, 32, 32, 16, b, b, b, b, 0.87f, nullptr), FP4_ESHAPE);
  expect("w2d32 ratio", fp4_quantize_w2d32(x, 32, 32, 32, b, b, b, b, 1.5f, nullptr), FP4_EINVAL);
  expect("w2d32 pitch", fp4_quantize_w2d32(x, 32, 32, (int64_t)1 << 22, b, b, b, b, 0.87f, nullptr), FP4_ESHAPE);
  expect("w2d32 limit", fp4_quantize_w2d32(x, huge_rows, 32, 32, b, b, b, b, 0.87f, nullptr), FP4_ESHAPE);
  expect("gemm shape", fp4_gemm(32, 32, 48, b, b, b, b, c, 32, 0, nullptr), FP4_ESHAPE);
  expect("gemm acc", fp4_gemm(32, 32, 32, b, b, b, b, c, 32, 2, nullptr), FP4_EINVAL);
  expect("gemm tiles", fp4_gemm(big, big, 32, b, b, b, b, c, big, 0, nullptr), FP4_ESHAPE);
  expect("gemm k0 wide", fp4_gemm(32, big * 1024, 0, nullptr, nullptr, nullptr, nullptr, c, big * 1024, 0, nullptr),
         FP4_ESHAPE);
  expect("gemm empty", fp4_gemm(0, 64, 64, nullptr, nullptr, nullptr, nullptr, nullptr, 64, 0, nullptr), FP4_OK);
  expect("gemm negative", fp4_gemm(-32, 64, 64, nullptr, nullptr, nullptr, nullptr, nullptr, 64, 0, nullptr),
         FP4_ESHAPE);
  expect("pair shape", fp4_gemm_pair(32, 32, 48, b, b, b, b, b, b, b, b, c, 32, 0, nullptr), FP4_ESHAPE);
  expect("pair null", fp4_gemm_pair(32, 32, 32, b, b, b, b, b, b, b, nullptr, c, 32, 0, nullptr), FP4_EINVAL);
  expect("pair align", fp4_gemm_pair(32, 32, 32, b, b, b, b, b, static_cast<uint8_t*>(odd), b, b, c, 32, 0, nullptr),
         FP4_EALIGN);
  expect("pair tiles", fp4_gemm_pair(big, big, 256, b, b, b, b, b, b, b, b, c, big, 0, nullptr), FP4_ESHAPE);
  expect("pair k0 acc", fp4_gemm_pair(64, 64, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                      nullptr, c, 64, 1, nullptr), FP4_OK);
  {
    const fp4_gemm_problem ok{256, 256, 256, b, b, b, b, nullptr, nullptr, nullptr, nullptr, c, 256, 0};
    fp4_gemm_problem g[2] = {ok, ok};
    g[1].ldc = 255;
    expect("grouped ldc", fp4_gemm_grouped(g, 2, nullptr), FP4_ESHAPE);
    g[1] = ok;
    g[1].b2_codes = b;
    expect("grouped partial pair", fp4_gemm_grouped(g, 2, nullptr), FP4_EINVAL);
    expect("grouped count", fp4_gemm_grouped(g, FP4_GEMM_GROUP_MAX + 1, nullptr), FP4_EINVAL);
    expect("grouped null", fp4_gemm_grouped(nullptr, 1, nullptr), FP4_EINVAL);
    const int64_t half = (int64_t)256 * 32768;               // 2^30 tiles each, 2^31 together
    const fp4_gemm_problem wide{half, half, 256, b, b, b, b, nullptr, nullptr, nullptr, nullptr, c, half, 0};
    fp4_gemm_problem w[2] = {wide, wide};
    expect("grouped total tiles", fp4_gemm_grouped(w, 2, nullptr), FP4_ESHAPE);
    fp4_gemm_problem e[2] = {ok, ok};
    e[0].m = 0;
    e[1].k = 0;
    e[1].accumulate = 1;
    expect("grouped empty", fp4_gemm_grouped(e, 2, nullptr), FP4_OK);
  }
  uint16_t* h = static_cast<uint16_t*>(p);
  expect("swiglu ht pair", fp4_swiglu_producer(32, 32, 32, b, b, b, b, h, h, b, b, b, nullptr, 0, nullptr), FP4_EINVAL);
  expect("swiglu tiles", fp4_swiglu_producer(big, big, 32, b, b, b, b, h, h, b, b, b, b, 0, nullptr), FP4_ESHAPE);
  expect("swiglu empty", fp4_swiglu_producer(0, 64, 64, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                             nullptr, nullptr, nullptr, 0, nullptr), FP4_OK);
  expect("bwd ld", fp4_swiglu_backward(32, 32, c, 16, h, h, h, h, nullptr), FP4_ESHAPE);
  expect("bwd huge", fp4_swiglu_backward(32, big * 4096, c, big * 4096, h, h, h, h, nullptr), FP4_ESHAPE);
  expect("bwd producer shape",
         fp4_swiglu_backward_producer(32, 48, c, 48, h, h, 0, 0, 1, 0, b, b, b, b, b, b, b, b, nullptr), FP4_ESHAPE);
  expect("bwd producer null",
         fp4_swiglu_backward_producer(32, 32, c, 32, h, nullptr, 0, 0, 1, 0, b, b, b, b, b, b, b, b, nullptr),
         FP4_EINVAL);
  expect("bwd producer pitch", fp4_swiglu_backward_producer(32, 32, c, (int64_t)1 << 23, h, h, 0, 0, 1, 0, b, b, b,
                                                            b, b, b, b, b, nullptr), FP4_ESHAPE);
  expect("bwd producer empty", fp4_swiglu_backward_producer(64, 0, nullptr, 0, nullptr, nullptr, 0, 0, 1, 0, nullptr,
                                                            nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                                            nullptr, nullptr), FP4_OK);
  expect("dgrad+bwd short k", fp4_gemm_swiglu_backward_producer(32, 32, 288, b, b, b, b, h, h, 0, 0, 1, 0, b, b, b, b,
                                                               b, b, b, b, nullptr), FP4_ESHAPE);
  expect("dgrad+bwd tiles", fp4_gemm_swiglu_backward_producer(big, 1 << 21, 256, b, b, b, b, h, h, 0, 0, 1, 0, b, b,
                                                             b, b, b, b, b, b, nullptr), FP4_ESHAPE);
  expect("dgrad+bwd empty", fp4_gemm_swiglu_backward_producer(0, 64, 256, nullptr, nullptr, nullptr, nullptr, nullptr,
                                                             nullptr, 0, 0, 1, 0, nullptr, nullptr, nullptr, nullptr,
                                                             nullptr, nullptr, nullptr, nullptr, nullptr), FP4_OK);
  const int64_t i64max = INT64_MAX;
  expect("nv rows mode", fp4_nv_quantize_rows(x, 32, 32, 32, b, b, c, c, static_cast<fp4_round>(2), 0, 0, nullptr), FP4_EINVAL);
  expect("nv rows shape", fp4_nv_quantize_rows(x, 32, 48, 48, b, b, c, c, static_cast<fp4_round>(0), 0, 0, nullptr), FP4_ESHAPE);
  expect("nv rows null", fp4_nv_quantize_rows(x, 32, 32, 32, b, b, c, nullptr, static_cast<fp4_round>(0), 0, 0, nullptr), FP4_EINVAL);
  expect("nv rows limit", fp4_nv_quantize_rows(x, 65536 * 32, 32, 32, b, b, c, c, static_cast<fp4_round>(1), 0, 0, nullptr), FP4_ESHAPE);
  expect("nv rows max", fp4_nv_quantize_rows(x, i64max, 32, 32, b, b, c, c, static_cast<fp4_round>(1), 0, 0, nullptr), FP4_ESHAPE);
  expect("nv rows huge cols", fp4_nv_quantize_rows(x, 32, big * 32, big * 32, b, b, c, c, static_cast<fp4_round>(0), 0, 0, nullptr),
         FP4_ESHAPE);
  expect("nv rows align", fp4_nv_quantize_rows(x, 32, 32, 36, b, b, c, c, static_cast<fp4_round>(0), 0, 0, nullptr), FP4_EALIGN);
  expect("nv rows empty", fp4_nv_quantize_rows(nullptr, 0, 64, 64, nullptr, nullptr, nullptr, nullptr, static_cast<fp4_round>(1), 0, 0,
                                               nullptr), FP4_OK);
  expect("nv w2d16 shape", fp4_nv_quantize_w2d16(x, 48, 32, 32, b, b, b, b, c, c, nullptr), FP4_ESHAPE);
  expect("nv w2d16 null", fp4_nv_quantize_w2d16(x, 32, 32, 32, b, b, b, nullptr, c, c, nullptr), FP4_EINVAL);
  expect("nv w2d16 limit", fp4_nv_quantize_w2d16(x, 65536 * 32, 32, 32, b, b, b, b, c, c, nullptr), FP4_ESHAPE);
  expect("nv w2d16 huge k", fp4_nv_quantize_w2d16(x, 32, i64max - 31, i64max, b, b, b, b, c, c, nullptr),
         FP4_ESHAPE);
  expect("nv w2d16 align", fp4_nv_quantize_w2d16(x, 32, 32, 32, b, b, static_cast<uint8_t*>(odd), b, c, c, nullptr),
         FP4_EALIGN);
  expect("nv gemm k", fp4_nv_gemm(32, 32, 32, b, b, c, 1, b, b, c, 0, c, 32, 0, nullptr), FP4_ESHAPE);
  expect("nv gemm long k", fp4_nv_gemm(32, 32, (int64_t)1 << 24, b, b, c, 1, b, b, c, 0, c, 32, 0, nullptr),
         FP4_ESHAPE);
  expect("nv gemm huge k", fp4_nv_gemm(32, 32, i64max - 63, b, b, c, 1, b, b, c, 0, c, 32, 0, nullptr), FP4_ESHAPE);
  expect("nv gemm stride", fp4_nv_gemm(32, 32, 64, b, b, c, -1, b, b, c, 0, c, 32, 0, nullptr), FP4_EINVAL);
  expect("nv gemm acc", fp4_nv_gemm(32, 32, 64, b, b, c, 1, b, b, c, 0, c, 32, 3, nullptr), FP4_EINVAL);
  expect("nv gemm null", fp4_nv_gemm(32, 32, 64, b, b, nullptr, 1, b, b, c, 0, c, 32, 0, nullptr), FP4_EINVAL);
  expect("nv gemm tiles", fp4_nv_gemm(big, big, 64, b, b, c, 1, b, b, c, 0, c, big, 0, nullptr), FP4_ESHAPE);
  expect("nv gemm max", fp4_nv_gemm(i64max - 31, i64max - 31, 64, b, b, c, 1, b, b, c, 0, c, i64max, 0, nullptr),
         FP4_ESHAPE);
  expect("nv gemm align", fp4_nv_gemm(32, 32, 64, b, b, c, 1, b, b, c, 0, c, 34, 0, nullptr), FP4_EALIGN);
  expect("nv gemm k0 acc", fp4_nv_gemm(64, 64, 0, nullptr, nullptr, nullptr, 1, nullptr, nullptr, nullptr, 0, c, 64,
                                       1, nullptr), FP4_OK);
  expect("nv gemm empty", fp4_nv_gemm(0, 64, 64, nullptr, nullptr, nullptr, 1, nullptr, nullptr, nullptr, 0, nullptr,
                                      64, 0, nullptr), FP4_OK);
  // the host-side generator: every seed, including ones whose halves carry
  for (uint64_t s : {0ull, 1ull, 0xFFFFFFFFull, 0x100000000ull, 0xFFFFFFFFFFFFFFFFull})
    if (fp4_sign_mask_from_seed(s) > 0xFFFFu) {
      fprintf(stderr, "sign mask of seed %llu exceeds 16 bits\n", (unsigned long long)s);
      ++failures;
    }
  if (fp4_last_hip_error() != 0) ++failures;
  printf("abi_checks: %d failure(s)\n", failures);
  return failures == 0 ? 0 : 1;
}
