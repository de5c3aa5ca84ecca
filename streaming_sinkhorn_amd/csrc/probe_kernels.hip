// Throughput probes behind the roofline of the streamed log-sum-exp pass
// (declarations in include/flashot_probe.h).
//
// The pass is bounded by two units: the matrix cores that form the score
// tile, and the transcendental unit that exponentiates every score (one
// exp2 per (i, j) pair and half-step: §2.3 and App. D.3 of "FlashSinkhorn:
// IO-Aware Entropic Optimal Transport on GPU", whose own profile in
// App. H.2.1 prices the kernel the same way). These kernels measure each
// unit alone on the chip, with enough independent work per wave to hide
// latency and enough waves to fill every SIMD.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "flashot_probe.h"
#include "host_common.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kExpChains = 8;
constexpr int kMfmaChains = 4;

// Each lane runs kExpChains independent chains x <- exp2(-x). From x in
// [0, 1] every value stays in [1/2, 1]: the exponent input is an ordinary
// normal number, and the negation is a source modifier of the instruction.
__global__ __launch_bounds__(256) void probe_exp2_kernel(int64_t iters, float* __restrict__ out) {
  float x[kExpChains];
#pragma unroll
  for (int c = 0; c < kExpChains; ++c) x[c] = (float)((threadIdx.x + 37 * c) & 255) * (1.0f / 256.f);
  for (int64_t t = 0; t < iters; ++t) {
#pragma unroll
    for (int c = 0; c < kExpChains; ++c) x[c] = __builtin_amdgcn_exp2f(-x[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kExpChains; ++c) s += x[c];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Each wave runs kMfmaChains independent accumulation chains of the
// 32x32x16 fp16 matrix instruction (the one the fp32 scores use).
__global__ __launch_bounds__(256) void probe_mfma_f16_kernel(int64_t iters, float* __restrict__ out) {
  f16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (_Float16)((float)((threadIdx.x + e) & 7) * 0.125f);
    b[e] = (_Float16)((float)((threadIdx.x * 3 + e) & 7) * 0.0625f);
  }
  f32x16 acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) acc[c] = f32x16{};
  for (int64_t t = 0; t < iters; ++t) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" int ot_probe_rate(int kind, int64_t iters, int32_t blocks, float* out, double* work,
                             void* stream) {
  using namespace flashot::host;
  try {
    if (!out || !work) return fail(OT_ERR_INVALID_ARG, "out or work is NULL");
    if (iters < 1 || blocks < 1) return fail(OT_ERR_INVALID_ARG, "iters and blocks must be >= 1");
    if (kind != OT_PROBE_EXP2 && kind != OT_PROBE_MFMA_F16)
      return fail(OT_ERR_INVALID_ARG, "kind must be OT_PROBE_EXP2 or OT_PROBE_MFMA_F16");
    hipStream_t st = (hipStream_t)stream;
    const double threads = (double)blocks * 256.0;
    if (kind == OT_PROBE_EXP2) {
      probe_exp2_kernel<<<blocks, 256, 0, st>>>(iters, out);
      *work = threads * (double)iters * kExpChains;
    } else {
      probe_mfma_f16_kernel<<<blocks, 256, 0, st>>>(iters, out);
      *work = threads / 64.0 * (double)iters * kMfmaChains * (2.0 * 32 * 32 * 16);
    }
    OT_HIP(hipGetLastError());
    return OT_OK;
  } catch (...) {
    return fail(OT_ERR_HIP, "unexpected host exception");
  }
}
