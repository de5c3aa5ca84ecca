// Features of the non-Euclidean costs as affine costs
// C_ij = alpha_i + beta_j - <Q_i, K_j> ("FlashSinkhorn: IO-Aware Entropic
// Optimal Transport on GPU", §3.1 "Scope of cost structure"; §4.2 for the
// label-augmented OTDD cost). The streamed passes then run unchanged with
// OT_COST_AFFINE. Declarations and semantics in include/flashot.h.
//
// The label term W[l_i, l_j] is looked up inside the matrix product: the
// source rows carry -W[l_i, :] and the target rows the one-hot e_{l_j}, so
// the per-pair lookup costs L extra k-columns on the matrix cores instead of
// a gather per score.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "flashot.h"
#include "host_common.h"

using namespace flashot;
using namespace flashot::host;

namespace {

template <typename T>
__device__ __forceinline__ float load_f32(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_f32<float>(const float* p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float load_f32<uint16_t>(const uint16_t* p, int64_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// One wave per row: out_i = pts_i / ||pts_i|| (zero rows stay zero), half_i = 1/2.
template <typename T>
__global__ __launch_bounds__(256) void prep_cosine_kernel(const T* __restrict__ pts, int64_t rows,
                                                          int64_t d, int64_t ld,
                                                          float* __restrict__ out,
                                                          float* __restrict__ half) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= rows) return;
  float s = 0.f;
  for (int64_t k = lane; k < d; k += 64) {
    const float v = load_f32<T>(pts, i * ld + k);
    s = fmaf(v, v, s);
  }
  s = wave_sum(s);
  const float inv = s > 0.f ? 1.0f / sqrtf(s) : 0.f;
  for (int64_t k = lane; k < d; k += 64) out[i * d + k] = load_f32<T>(pts, i * ld + k) * inv;
  if (lane == 0) half[i] = 0.5f;
}

// One wave per row: source rows [2 x_i, -W[l_i, :]], target rows [y_j, e_{l_j}];
// sqn_i = ||pts_i||^2. Labels outside [0, L) get zero label features.
template <typename T>
__global__ __launch_bounds__(256) void prep_labels_kernel(const T* __restrict__ pts, int64_t rows,
                                                          int64_t d, int64_t ld,
                                                          const int32_t* __restrict__ labels,
                                                          const float* __restrict__ W, int L,
                                                          int side, float* __restrict__ out,
                                                          float* __restrict__ sqn) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= rows) return;
  const int64_t w = d + L;
  const float scale = side == 0 ? 2.f : 1.f;
  float s = 0.f;
  for (int64_t k = lane; k < d; k += 64) {
    const float v = load_f32<T>(pts, i * ld + k);
    s = fmaf(v, v, s);
    out[i * w + k] = scale * v;
  }
  const int l = labels[i];
  const bool ok = l >= 0 && l < L;
  for (int k = lane; k < L; k += 64) {
    float v = 0.f;
    if (ok) v = side == 0 ? -W[(int64_t)l * L + k] : (k == l ? 1.f : 0.f);
    out[i * w + d + k] = v;
  }
  s = wave_sum(s);
  if (lane == 0) sqn[i] = s;
}

unsigned rows4(int64_t rows) { return (unsigned)((rows + 3) / 4); }

int check_pts(const void* pts, int dtype, int64_t rows, int64_t d, int64_t ld) {
  if (!pts) return fail(OT_ERR_INVALID_ARG, "pts is NULL");
  if (rows < 1 || d < 1) return fail(OT_ERR_INVALID_ARG, "rows and d must be >= 1");
  if (ld < d) return fail(OT_ERR_INVALID_ARG, "ld must be >= d");
  if (dtype != OT_F32 && dtype != OT_BF16) return fail(OT_ERR_UNSUPPORTED, "dtype must be OT_F32 or OT_BF16");
  if (d > OT_MAX_D) return fail(OT_ERR_UNSUPPORTED, "d exceeds OT_MAX_D");
  if (rows > ((int64_t)1 << 30)) return fail(OT_ERR_UNSUPPORTED, "rows exceeds 2^30");
  if ((uintptr_t)pts % (dtype == OT_BF16 ? 2 : 4)) return fail(OT_ERR_INVALID_ARG, "pts misaligned");
  return OT_OK;
}

}  // namespace

extern "C" {

int ot_prep_cosine(const void* pts, int dtype, int64_t rows, int64_t d, int64_t ld, float* out,
                   float* half, void* stream) {
  try {
    int rc = check_pts(pts, dtype, rows, d, ld);
    if (rc) return rc;
    if (!out || !half) return fail(OT_ERR_INVALID_ARG, "out or half is NULL");
    hipStream_t st = (hipStream_t)stream;
    if (dtype == OT_BF16)
      prep_cosine_kernel<uint16_t><<<rows4(rows), 256, 0, st>>>((const uint16_t*)pts, rows, d, ld,
                                                                out, half);
    else
      prep_cosine_kernel<float><<<rows4(rows), 256, 0, st>>>((const float*)pts, rows, d, ld, out,
                                                             half);
    OT_HIP(hipGetLastError());
    return OT_OK;
  } catch (...) {
    return fail(OT_ERR_HIP, "unexpected host exception");
  }
}

int ot_prep_labels(const void* pts, int dtype, int64_t rows, int64_t d, int64_t ld,
                   const int32_t* labels, const float* W, int32_t n_labels, int32_t side,
                   float* out, float* sqn, void* stream) {
  try {
    int rc = check_pts(pts, dtype, rows, d, ld);
    if (rc) return rc;
    if (n_labels < 1) return fail(OT_ERR_INVALID_ARG, "n_labels must be >= 1");
    if (side != 0 && side != 1) return fail(OT_ERR_INVALID_ARG, "side must be 0 (source) or 1 (target)");
    if (d + n_labels > OT_MAX_D) return fail(OT_ERR_UNSUPPORTED, "d + n_labels exceeds OT_MAX_D");
    if (!labels || !W || !out || !sqn) return fail(OT_ERR_INVALID_ARG, "labels, W, out or sqn is NULL");
    hipStream_t st = (hipStream_t)stream;
    if (dtype == OT_BF16)
      prep_labels_kernel<uint16_t><<<rows4(rows), 256, 0, st>>>((const uint16_t*)pts, rows, d, ld,
                                                                labels, W, n_labels, side, out, sqn);
    else
      prep_labels_kernel<float><<<rows4(rows), 256, 0, st>>>((const float*)pts, rows, d, ld, labels,
                                                             W, n_labels, side, out, sqn);
    OT_HIP(hipGetLastError());
    return OT_OK;
  } catch (...) {
    return fail(OT_ERR_HIP, "unexpected host exception");
  }
}

}  // extern "C"
