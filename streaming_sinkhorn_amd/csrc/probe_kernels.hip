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

// Occupancy-limited probes: each workgroup of 256 threads (one wave per
// SIMD) reserves kLimitLds bytes of LDS, so two workgroups fit a compute
// unit and every SIMD holds two waves, as in the register-resident
// log-sum-exp pass (236 VGPRs).
constexpr int kLimitLds = 64 * 1024;

// CHAINS independent 32x32x16 fp16 accumulation chains per wave, at two
// waves per SIMD.
template <int CHAINS>
__global__ __launch_bounds__(256) void probe_mfma_chains_kernel(int64_t iters,
                                                                float* __restrict__ out) {
  f16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (_Float16)((float)((threadIdx.x + e) & 7) * 0.125f);
    b[e] = (_Float16)((float)((threadIdx.x * 3 + e) & 7) * 0.0625f);
  }
  f32x16 acc[CHAINS];
#pragma unroll
  for (int c = 0; c < CHAINS; ++c) acc[c] = f32x16{};
  for (int64_t t = 0; t < iters; ++t) {
#pragma unroll
    for (int c = 0; c < CHAINS; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CHAINS; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// The instruction mix of one pipeline stage of the d = 64 fp32 pass (two row
// tiles per wave): 26 matrix instructions in two accumulation chains, 34
// exponentials and 48 fp32 additions, interleaved one matrix instruction to
// three vector ones as that pass schedules them, at two waves per SIMD. The
// vector work does not depend on the matrix results, so the probe gives the
// rate at which the two units can share a SIMD's issue for this mix, without
// memory traffic or dependency waits. Work: the matrix flops.
constexpr int kMixMfma = 13;  // per chain and iteration
constexpr int kMixExp = 17;   // per chain and iteration
__global__ __launch_bounds__(256) void probe_mix_kernel(int64_t iters, float* __restrict__ out) {
  f16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (_Float16)((float)((threadIdx.x + e) & 7) * 0.125f);
    b[e] = (_Float16)((float)((threadIdx.x * 3 + e) & 7) * 0.0625f);
  }
  f32x16 acc[2] = {f32x16{}, f32x16{}};
  float x[2][kMixExp], y[2][kMixExp];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int k = 0; k < kMixExp; ++k) {
      x[c][k] = (float)((threadIdx.x + 5 * k + c) & 255) * (1.0f / 256.f);
      y[c][k] = 0.f;
    }
  for (int64_t t = 0; t < iters; ++t) {
#pragma unroll
    for (int k = 0; k < kMixMfma; ++k) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
        if (k < kMixExp) {
          x[c][k] = __builtin_amdgcn_exp2f(-x[c][k]);
          y[c][k] += x[c][k];
        }
        y[c][(k + 7) % kMixExp] += x[c][(k + 3) % kMixExp];
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
      }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int k = kMixMfma; k < kMixExp; ++k) {
        x[c][k] = __builtin_amdgcn_exp2f(-x[c][k]);
        y[c][k] += x[c][k];
      }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
#pragma unroll
    for (int k = 0; k < kMixExp; ++k) s += y[c][k];
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" int ot_probe_rate(int kind, int64_t iters, int32_t blocks, float* out, double* work,
                             void* stream) {
  using namespace flashot::host;
  try {
    if (!out || !work) return fail(OT_ERR_INVALID_ARG, "out or work is NULL");
    if (iters < 1 || blocks < 1) return fail(OT_ERR_INVALID_ARG, "iters and blocks must be >= 1");
    if (kind < OT_PROBE_EXP2 || kind > OT_PROBE_MIX_2W)
      return fail(OT_ERR_INVALID_ARG, "unknown probe kind");
    hipStream_t st = (hipStream_t)stream;
    const double waves = (double)blocks * 4.0;
    const double mfma_flops = 2.0 * 32 * 32 * 16;
    switch (kind) {
      case OT_PROBE_EXP2:
        probe_exp2_kernel<<<blocks, 256, 0, st>>>(iters, out);
        *work = waves * 64.0 * (double)iters * kExpChains;
        break;
      case OT_PROBE_MFMA_F16:
        probe_mfma_f16_kernel<<<blocks, 256, 0, st>>>(iters, out);
        *work = waves * (double)iters * kMfmaChains * mfma_flops;
        break;
      case OT_PROBE_MFMA_F16_1C2W:
        probe_mfma_chains_kernel<1><<<blocks, 256, kLimitLds, st>>>(iters, out);
        *work = waves * (double)iters * 1 * mfma_flops;
        break;
      case OT_PROBE_MFMA_F16_2C2W:
        probe_mfma_chains_kernel<2><<<blocks, 256, kLimitLds, st>>>(iters, out);
        *work = waves * (double)iters * 2 * mfma_flops;
        break;
      default:
        probe_mix_kernel<<<blocks, 256, kLimitLds, st>>>(iters, out);
        *work = waves * (double)iters * 2 * kMixMfma * mfma_flops;
        break;
    }
    OT_HIP(hipGetLastError());
    return OT_OK;
  } catch (...) {
    return fail(OT_ERR_HIP, "unexpected host exception");
  }
}
