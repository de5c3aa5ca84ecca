// Auxiliary gfx950 kernels of the streamed Sinkhorn solver: per-problem
// preparation (squared norms, operand packing, weights, bias), the merge of
// column-split partials with the half-step epilogue, deterministic
// reductions and the transport-application epilogue. None of them is on the
// O(n m) path; they are compiled with full IEEE NaN semantics so that a NaN
// in the inputs reaches the returned potentials instead of being absorbed.
//
// Method: "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU"
// (arXiv 2602.03067), App. D.1-D.3 and E.1 (see each kernel).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"

namespace flashot {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxApplySplits = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p, int64_t idx);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p, int64_t idx) {
  return p[idx];
}
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p, int64_t idx) {
  return bf16_to_f32(p[idx]);
}

// ---------------------------------------------------------------------------
// Merge of split partials + half-step epilogue (App. D.1 / D.2: write the
// potential once). Partials are (M2, S) in log2 units: the row's log-sum-exp
// over split s is ln 2 * (M2 + log2 S). For row i:
//   M = max_s M2_s, S = sum_s S_s 2^(M2_s - M),
//   shifted potential = -eps ln 2 (M + log2 S),  half-step value h_i = norm_i + shifted,
//   pot_i = h_i, or (pot_i + h_i) / 2 for the symmetric schedule (avg),
//   next bias_i = bscale * ((pot_i - norm_i)/2 + (eps/2) log w_i),
//   err_i = w_i |exp((pot_old_i - h_i)/eps) - 1|   (App. E.1 induced marginal of
//   the coupling of the previous iterate).
// bscale = 2 log2(e)/eps when the streamed kernel works in log2 units (fp32
// operands packed pre-scaled), 1 when it works in dot-product units.
// The bias is rebuilt from the stored fp32 potential, so resuming from
// returned potentials reproduces an uninterrupted run bit for bit.
__device__ __forceinline__ float block_sum_256(float v, float* sh) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
#pragma unroll
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) sh[t] += sh[t + w];
    __syncthreads();
  }
  return sh[0];
}

// Eight lanes per row: lane k merges splits k, k + 8, ... online in one pass,
// then the eight (M, S) pairs are combined by a fixed xor butterfly (every
// lane of the group ends with the same values, so the result does not depend
// on the lane). Workgroups cover 32 rows, so even 20000 rows give 625 of them.
constexpr int kMergeLanes = 8;
constexpr int kMergeRows = 256 / kMergeLanes;

__global__ __launch_bounds__(256) void lse_merge_kernel(
    const float2* __restrict__ part, int splits, int rpad, int rows, float bscale, float eps,
    const float* __restrict__ norm, const float* __restrict__ hlw, const float* __restrict__ wgt,
    float* __restrict__ pot, float* __restrict__ bias_out, float* __restrict__ err_part,
    int with_err, int write_pot, int avg) {
  __shared__ float sh[256];
  const int sub = threadIdx.x & (kMergeLanes - 1);
  const int i = blockIdx.x * kMergeRows + threadIdx.x / kMergeLanes;
  float M = -3.0e38f, S = 0.f;
  if (i < rows) {
    for (int s = sub; s < splits; s += kMergeLanes) {
      const float2 ps = part[(size_t)s * rpad + i];
      if (ps.x > M) {
        S = fmaf(S, exp2f(M - ps.x), ps.y);
        M = ps.x;
      } else {
        S = fmaf(ps.y, exp2f(ps.x - M), S);
      }
    }
  }
#pragma unroll
  for (int o = 1; o < kMergeLanes; o <<= 1) {
    const float Mo = __shfl_xor(M, o);
    const float So = __shfl_xor(S, o);
    const float Mn = fmaxf(M, Mo);
    S = S * exp2f(M - Mn) + So * exp2f(Mo - Mn);
    M = Mn;
  }
  const RowFinish fin{bscale, eps, norm, hlw, wgt, pot, bias_out, rows, rpad, with_err, write_pot, avg};
  float e = 0.f;
  if (sub == 0 && i < rows) e = finish_row(fin, i, M, S, load_row_in(fin, i));
  else if (sub == 0 && i < rpad) finish_pad_row(fin, i);
  if (with_err) {
    const float tot = block_sum_256(e, sh);
    if (threadIdx.x == 0) err_part[blockIdx.x] = tot;
  }
}

int lse_merge_blocks(int rows) { return (rows + kMergeRows - 1) / kMergeRows; }

// <w, pot> in fp64 over one workgroup in a fixed order (w = NULL: uniform 1/rows).
__device__ double dual_term(const float* __restrict__ w, const float* __restrict__ pot, int rows,
                            double* sh) {
  double s = 0.0;
  const double u = 1.0 / (double)rows;
  for (int i = threadIdx.x; i < rows; i += 256) s += (w ? (double)w[i] : u) * (double)pot[i];
  sh[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) sh[threadIdx.x] += sh[threadIdx.x + o];
    __syncthreads();
  }
  const double t = sh[0];
  __syncthreads();
  return t;
}

// out = [S, OT(mu, nu), OT(mu, mu), OT(nu, nu)] with OT = <a, f> + <b, g>.
__global__ __launch_bounds__(256) void dual_values_kernel(
    const float* __restrict__ a, const float* __restrict__ b, int n, int m,
    const float* __restrict__ f, const float* __restrict__ g, const float* __restrict__ fxx,
    const float* __restrict__ gxx, const float* __restrict__ fyy, const float* __restrict__ gyy,
    float* __restrict__ out) {
  __shared__ double sh[256];
  const double xy = dual_term(a, f, n, sh) + dual_term(b, g, m, sh);
  const double xx = dual_term(a, fxx, n, sh) + dual_term(a, gxx, n, sh);
  const double yy = dual_term(b, fyy, m, sh) + dual_term(b, gyy, m, sh);
  if (threadIdx.x == 0) {
    out[0] = (float)(xy - 0.5 * xx - 0.5 * yy);
    out[1] = (float)xy;
    out[2] = (float)xx;
    out[3] = (float)yy;
  }
}

hipError_t launch_dual_values(const float* a, const float* b, int n, int m, const float* f,
                              const float* g, const float* fxx, const float* gxx, const float* fyy,
                              const float* gyy, float* out, hipStream_t st) {
  dual_values_kernel<<<1, 256, 0, st>>>(a, b, n, m, f, g, fxx, gxx, fyy, gyy, out);
  return hipGetLastError();
}

// Deterministic single-workgroup sum of `count` partials (fixed order).
__global__ __launch_bounds__(256) void err_reduce_kernel(const float* __restrict__ part, int count,
                                                          float* __restrict__ out) {
  __shared__ float sh[256];
  float v = 0.f;
  for (int k = threadIdx.x; k < count; k += 256) v += part[k];
  const float tot = block_sum_256(v, sh);
  if (threadIdx.x == 0) out[0] = tot;
}

// Sets *out to 1.0f when f or g holds a NaN or an infinity (*out is zeroed
// first by the launcher). Grid-stride over both vectors; one flag per
// workgroup, set by an atomic OR of the bits of 1.0f (same result in any order).
__global__ __launch_bounds__(256) void nonfinite_kernel(const float* __restrict__ f, int n,
                                                         const float* __restrict__ g, int m,
                                                         float* __restrict__ out) {
  // Exponent-bit test: independent of the no-NaN compile flags of this file.
  auto bad = [](float x) { return ((__float_as_uint(x) >> 23) & 0xffu) == 0xffu; };
  int any = 0;
  const int64_t total = (int64_t)n + m;
  for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < total; k += (int64_t)gridDim.x * 256)
    any |= bad(k < n ? f[k] : g[k - n]) ? 1 : 0;
  if (__syncthreads_or(any) && threadIdx.x == 0)
    atomicOr(reinterpret_cast<unsigned int*>(out), 0x3f800000u);
}

// Merge of P V partials and epilogue. For row i of the coupling induced by
// (pot, other potential):
//   P_ij = w_i exp((pot_i - norm_i)/eps) exp((2/eps) v_ij)   (v = x.y + bias)
//   factor_i = w_i exp((pot_i - norm_i + 2 M_i)/eps),  (P V)_i = factor_i O_i,
//   r_i = factor_i S_i, barycentric = O_i / S_i, gradient = 2 (r_i x_i - (P Y)_i).
// Workgroup: 32 rows x 32 columns, transposed through LDS for coalesced stores.
template <typename T>
__global__ __launch_bounds__(256) void apply_merge_kernel(
    const float2* __restrict__ partMS, const float* __restrict__ partO, int splits, int rpad,
    int ppad, int rows, int cols, float c, float eps, const float* __restrict__ pot,
    const float* __restrict__ norm, const float* __restrict__ wgt, int mode,
    const T* __restrict__ Xsrc, int64_t ldx, const unsigned* __restrict__ vamax,
    float* __restrict__ out, float* __restrict__ marg) {
  __shared__ float scl[kMaxApplySplits][32];
  __shared__ float fac[32], rr[32], ss[32];
  __shared__ float tile[32][33];
  const int t = threadIdx.x;
  const int i0 = blockIdx.x * 32;
  const int p0 = blockIdx.y * 32;
  if (t < 32) {
    const int i = i0 + t;
    if (i < rows) {
      float M = partMS[i].x;
      for (int s = 1; s < splits; ++s) M = fmaxf(M, partMS[(size_t)s * rpad + i].x);
      const float cm = c * M;
      float S = 0.f;
      for (int s = 0; s < splits; ++s) {
        const float2 ps = partMS[(size_t)s * rpad + i];
        const float e = exp2f(fmaf(c, ps.x, -cm));
        scl[s][t] = e;
        S += ps.y * e;
      }
      const float f = wgt[i] * exp2f(fmaf(pot[i] - norm[i], kLog2e / eps, cm));
      fac[t] = f;
      ss[t] = S;
      rr[t] = f * S;
    }
  }
  __syncthreads();
  const int tx = t & 31;
  const int ty = t >> 5;
  const int i = i0 + tx;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int pl = ty + 8 * k;
    const int p = p0 + pl;
    float val = 0.f;
    if (i < rows && p < cols) {
      float O = 0.f;
      for (int s = 0; s < splits; ++s) O += partO[((size_t)s * ppad + p) * rpad + i] * scl[s][tx];
      if (vamax) O = ldexpf(O, -vcol_shift(vamax[p]));
      if (mode == kApplyBary) {
        val = O / ss[tx];
      } else if (mode == kApplyGrad) {
        const float xv = load_as_f32<T>(Xsrc, (int64_t)i * ldx + p);
        val = 2.f * (rr[tx] * xv - fac[tx] * O);
      } else {
        val = fac[tx] * O;
      }
    }
    tile[tx][pl] = val;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int rl = ty + 8 * k;
    const int ii = i0 + rl;
    const int p = p0 + tx;
    if (ii < rows && p < cols) out[(size_t)ii * cols + p] = tile[rl][tx];
  }
  if (marg && blockIdx.y == 0 && t < 32 && i0 + t < rows) marg[i0 + t] = rr[t];
}

// ---------------------------------------------------------------------------
// Small per-problem kernels.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void sqnorms_kernel(const T* __restrict__ pts, int64_t rows,
                                                       int64_t d, int64_t ld,
                                                       float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  float s = 0.f;
  for (int64_t k = lane; k < d; k += 64) {
    const float v = load_as_f32<T>(pts, row * ld + k);
    s = fmaf(v, v, s);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) out[row] = s;
}

// Packs a row-major point cloud into the MFMA operand layout of kernels.h,
// multiplying the values by `scale`. bf16 values are copied unchanged when
// scale is 1; otherwise they are scaled in fp32 and rounded back to bf16
// (exact for the power-of-two scales used).
template <typename T>
__global__ __launch_bounds__(256) void pack_points_kernel(const T* __restrict__ src, int64_t rows,
                                                           int64_t d, int64_t ld, int64_t total,
                                                           int kbp, float scale,
                                                           u32x4* __restrict__ dst) {
  constexpr int KW = 16 / sizeof(T);  // values per lane per k-block
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int lane = (int)(idx & 63);
    const int64_t tk = idx >> 6;
    const int kb = (int)(tk % kbp);
    const int64_t t = tk / kbp;
    const int64_t row = t * kTile + (lane & 31);
    const int64_t k0 = (int64_t)kb * (2 * KW) + (lane >> 5) * KW;
    T v[KW];
#pragma unroll
    for (int e = 0; e < KW; ++e)
      v[e] = (row < rows && k0 + e < d) ? src[row * ld + k0 + e] : T(0);
    if constexpr (sizeof(T) == 4) {
#pragma unroll
      for (int e = 0; e < KW; ++e) v[e] = v[e] * scale;
    } else if (scale != 1.0f) {
#pragma unroll
      for (int e = 0; e < KW; ++e)
        v[e] = (T)bf16_bits_rne(__uint_as_float((uint32_t)v[e] << 16) * scale);
    }
    dst[idx] = __builtin_bit_cast(u32x4, v);
  }
}


// Splits scale * src into hi + mid + lo, each the bf16 rounding of what the
// previous parts left (the differences are exact in fp32), and packs part p
// of k-block kb into unit 3 kb + p of the tile, in the lane layout of a bf16
// k-block: lane l holds row l % 32, values k = 16 kb + 8 (l / 32) ... + 7.
__global__ __launch_bounds__(256) void pack_split_kernel(const float* __restrict__ src,
                                                          int64_t rows, int64_t d, int64_t ld,
                                                          int64_t total, int units, float scale,
                                                          u32x4* __restrict__ dst) {
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int lane = (int)(idx & 63);
    const int64_t tu = idx >> 6;
    const int u = (int)(tu % units);
    const int64_t t = tu / units;
    const int kb = u / 3, part = u % 3;
    const int64_t row = t * kTile + (lane & 31);
    const int64_t k0 = (int64_t)kb * 16 + (lane >> 5) * 8;
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = (row < rows && k0 + e < d) ? src[row * ld + k0 + e] * scale : 0.f;
      uint32_t b = bf16_bits_rne(v);
      for (int q = 0; q < part; ++q) {
        v = v - __uint_as_float(b << 16);
        b = bf16_bits_rne(v);
      }
      h[e] = b;
    }
    u32x4 o;
    o.x = h[0] | (h[1] << 16);
    o.y = h[2] | (h[3] << 16);
    o.z = h[4] | (h[5] << 16);
    o.w = h[6] | (h[7] << 16);
    dst[idx] = o;
  }
}

// ---------------------------------------------------------------------------
// Two fp16 parts per fp32 value (half2 operand mode). A value v is written
// as hi = fp16(v) and lo = fp16(v - hi) (round to nearest even; v - hi is
// exact in fp32), so v - hi - lo is below 2^-22 |v| while v is inside the
// fp16 range. The X cloud is scaled by 2^a and the Y cloud by 2^-a, both
// exact, so every product -- and the score -- is unchanged; a balances the
// two clouds' largest magnitudes below 2^15 (fp16 holds up to 65504). When
// no a does, the plan is marked out of range and X is written as NaN, so
// the potentials come out non-finite rather than wrong.
// ---------------------------------------------------------------------------
// Largest |value| of a row-major cloud, as the bits of a non-negative float
// (a NaN coordinate compares above every finite value and infinity): block b
// scans a contiguous run of rows and writes its maximum to part[b].
__global__ __launch_bounds__(256) void absmax_kernel(const float* __restrict__ src, int64_t rows,
                                                     int64_t d, int64_t ld,
                                                     unsigned* __restrict__ part) {
  __shared__ unsigned sh[256];
  const int64_t per = (rows + gridDim.x - 1) / gridDim.x;
  const int64_t r0 = (int64_t)blockIdx.x * per;
  const int64_t r1 = r0 + per < rows ? r0 + per : rows;
  const int64_t cnt = r1 > r0 ? (r1 - r0) * d : 0;
  // element e = i d + k of the run; stepping e by 256 adds (q, rm) to (i, k)
  const int64_t q = 256 / d, rm = 256 % d;
  int64_t i = threadIdx.x / d, k = threadIdx.x % d;
  unsigned mx = 0;
  for (int64_t e = threadIdx.x; e < cnt; e += 256) {
    mx = max(mx, __float_as_uint(src[(r0 + i) * ld + k]) & 0x7fffffffu);
    i += q;
    k += rm;
    if (k >= d) {
      k -= d;
      ++i;
    }
  }
  sh[threadIdx.x] = mx;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) sh[threadIdx.x] = max(sh[threadIdx.x], sh[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = sh[0];
}

// Reduces the block maxima of X (part[0..nx)) and Y (part[kHalf2Parts..))
// and writes the plan. cx: the factor X is packed with (score scale at the
// problem's eps; a smaller eps-scaling factor only lowers |X|).
__global__ __launch_bounds__(256) void half2_plan_kernel(Half2Plan* __restrict__ p, int nx, int ny,
                                                         float cx) {
  __shared__ unsigned sh[2][256];
  unsigned ax = 0, ay = 0;
  for (int b = threadIdx.x; b < nx; b += 256) ax = max(ax, p->part[b]);
  for (int b = threadIdx.x; b < ny; b += 256) ay = max(ay, p->part[kHalf2Parts + b]);
  sh[0][threadIdx.x] = ax;
  sh[1][threadIdx.x] = ay;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) {
      sh[0][threadIdx.x] = max(sh[0][threadIdx.x], sh[0][threadIdx.x + w]);
      sh[1][threadIdx.x] = max(sh[1][threadIdx.x], sh[1][threadIdx.x + w]);
    }
    __syncthreads();
  }
  if (threadIdx.x != 0) return;
  p->amax[0] = sh[0][0];
  p->amax[1] = sh[1][0];
  const float mx = __uint_as_float(sh[0][0]) * cx;
  const float my = __uint_as_float(sh[1][0]);
  int ex = 0, ey = 0;  // m < 2^e
  if (mx > 0.f) (void)frexpf(mx, &ex);
  if (my > 0.f) (void)frexpf(my, &ey);
  int a = (ey - ex) >> 1;  // floor: X' < 2^(ex + a), Y' < 2^(ey - a)
  a = a < -100 ? -100 : (a > 100 ? 100 : a);
  p->xmul = ldexpf(1.f, a);
  p->ymul = ldexpf(1.f, -a);
  p->ok = (isfinite(mx) && isfinite(my) && ex + a <= 15 && ey - a <= 15) ? 1 : 0;
}

// Layout of pack_split with two units per k-block: units (2 kb, 2 kb + 1) of
// a tile hold hi and lo of k-block kb. side 0 packs X (times scale * xmul),
// side 1 packs Y (times scale * ymul).
__global__ __launch_bounds__(256) void pack_half2_kernel(const float* __restrict__ src,
                                                         int64_t rows, int64_t d, int64_t ld,
                                                         int64_t total, int units, float scale,
                                                         const Half2Plan* __restrict__ plan,
                                                         int side, u32x4* __restrict__ dst) {
  const float mul = scale * (side ? plan->ymul : plan->xmul);
  const bool poison = side == 0 && plan->ok == 0;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int lane = (int)(idx & 63);
    const int64_t tu = idx >> 6;
    const int u = (int)(tu % units);
    const int64_t t = tu / units;
    const int kb = u >> 1, part = u & 1;
    const int64_t row = t * kTile + (lane & 31);
    const int64_t k0 = (int64_t)kb * 16 + (lane >> 5) * 8;
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = (row < rows && k0 + e < d) ? src[row * ld + k0 + e] * mul : 0.f;
      const _Float16 hi = (_Float16)v;
      const _Float16 q = part ? (_Float16)(v - (float)hi) : hi;
      h[e] = poison ? 0x7e00u : (uint32_t)__builtin_bit_cast(uint16_t, q);
    }
    u32x4 o;
    o.x = h[0] | (h[1] << 16);
    o.y = h[2] | (h[3] << 16);
    o.z = h[4] | (h[5] << 16);
    o.w = h[6] | (h[7] << 16);
    dst[idx] = o;
  }
}

// Packs V (rows streamed x cols) as the A operand of O^T += V^T P^T: for
// column tile t, column block pb (32 values of p), quad q and lane l the four
// floats are V[32t + 8q + 4(l/32) + e][32pb + l%32], e = 0..3 -- the row order
// of the score accumulator registers 4q..4q+3.
template <typename T>
__global__ __launch_bounds__(256) void pack_values_kernel(const T* __restrict__ V, int64_t rows,
                                                           int64_t cols, int64_t ldv,
                                                           int64_t total, int pblocks,
                                                           f32x4* __restrict__ dst) {
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int lane = (int)(idx & 63);
    const int q = (int)((idx >> 6) & 3);
    const int64_t tp = idx >> 8;
    const int pb = (int)(tp % pblocks);
    const int64_t t = tp / pblocks;
    const int64_t col = (int64_t)pb * 32 + (lane & 31);
    const int64_t r0 = t * kTile + 8 * q + 4 * (lane >> 5);
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = (col < cols && r0 + e < rows) ? load_as_f32<T>(V, (r0 + e) * ldv + col) : 0.f;
    dst[idx] = v;
  }
}

// Column maxima of |V| for the fp16 value layout: thread = column, rows
// strided over blockIdx.y, one atomic max per thread (amax zeroed first).
template <typename T>
__global__ __launch_bounds__(256) void vcol_absmax_kernel(const T* __restrict__ V, int64_t rows,
                                                          int64_t cols, int64_t ldv,
                                                          unsigned* __restrict__ amax) {
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (col >= cols) return;
  unsigned mx = 0;
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y)
    mx = max(mx, __float_as_uint(load_as_f32<T>(V, r * ldv + col)) & 0x7fffffffu);
  atomicMax(&amax[col], mx);
}

// fp16 value layout (see launch_pack_values_h2): unit ((jt * pblocks + pb) * 2
// + q) * 2 + part, 64 lanes of 8 fp16 values.
template <typename T>
__global__ __launch_bounds__(256) void pack_values_h2_kernel(const T* __restrict__ V, int64_t rows,
                                                             int64_t cols, int64_t ldv,
                                                             int64_t total, int pblocks,
                                                             const unsigned* __restrict__ amax,
                                                             u32x4* __restrict__ dst) {
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int lane = (int)(idx & 63);
    const int part = (int)((idx >> 6) & 1);
    const int q = (int)((idx >> 7) & 1);
    const int64_t tp = idx >> 8;
    const int pb = (int)(tp % pblocks);
    const int64_t t = tp / pblocks;
    const int64_t col = (int64_t)pb * 32 + (lane & 31);
    const int shift = col < cols ? vcol_shift(amax[col]) : 0;
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t row = t * kTile + 8 * (2 * q + (e >> 2)) + 4 * (lane >> 5) + (e & 3);
      const float v = (col < cols && row < rows) ? ldexpf(load_as_f32<T>(V, row * ldv + col), shift)
                                                 : 0.f;
      const _Float16 hi = (_Float16)v;
      const _Float16 x = part ? (_Float16)(v - (float)hi) : hi;
      h[e] = (uint32_t)__builtin_bit_cast(uint16_t, x);
    }
    u32x4 o;
    o.x = h[0] | (h[1] << 16);
    o.y = h[2] | (h[3] << 16);
    o.z = h[4] | (h[5] << 16);
    o.w = h[6] | (h[7] << 16);
    dst[idx] = o;
  }
}

__global__ __launch_bounds__(256) void weights_kernel(const float* __restrict__ w, int rows,
                                                       int rpad, float eps,
                                                       float* __restrict__ wgt,
                                                       float* __restrict__ hlw) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= rpad) return;
  if (i < rows) {
    const float wi = w ? w[i] : 1.0f / (float)rows;
    wgt[i] = wi;
    hlw[i] = 0.5f * eps * logf(wi);
  } else {
    wgt[i] = 0.f;
    hlw[i] = 0.f;
  }
}

__global__ __launch_bounds__(256) void fill_kernel(float* __restrict__ p, float v, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * 256)
    p[i] = v;
}

__global__ __launch_bounds__(256) void bias_from_pot_kernel(const float* __restrict__ pot,
                                                             const float* __restrict__ norm,
                                                             const float* __restrict__ hlw,
                                                             int rows, int rpad, float bscale,
                                                             float* __restrict__ bias, int parts) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= rpad) return;
  const float v = (i < rows) ? bscale * (0.5f * (pot[i] - norm[i]) + hlw[i]) : kSentinel;
  bias[i] = v;
  if (parts) write_bias_parts(bias, rpad, i, v);
}


static int grid_for(int64_t total, int64_t per_block, int64_t cap = 1 << 20) {
  int64_t g = (total + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (int)g;
}

hipError_t launch_sqnorms(const void* pts, int bf16, int64_t rows, int64_t d, int64_t ld,
                          float* out, hipStream_t st) {
  const int grid = (int)((rows + 3) / 4);
  if (bf16)
    sqnorms_kernel<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)pts, rows, d, ld, out);
  else
    sqnorms_kernel<float><<<grid, 256, 0, st>>>((const float*)pts, rows, d, ld, out);
  return hipGetLastError();
}

hipError_t launch_pack_points(const void* src, int bf16, int64_t rows, int64_t d, int64_t ld,
                              int rtiles, int kbp, float scale, void* dst, hipStream_t st) {
  const int64_t total = (int64_t)rtiles * kbp * 64;
  const int grid = grid_for(total, 256, 65536);
  if (bf16)
    pack_points_kernel<uint16_t>
        <<<grid, 256, 0, st>>>((const uint16_t*)src, rows, d, ld, total, kbp, scale, (u32x4*)dst);
  else
    pack_points_kernel<float>
        <<<grid, 256, 0, st>>>((const float*)src, rows, d, ld, total, kbp, scale, (u32x4*)dst);
  return hipGetLastError();
}

hipError_t launch_pack_split(const float* src, int64_t rows, int64_t d, int64_t ld, int rtiles,
                             int units, float scale, void* dst, hipStream_t st) {
  const int64_t total = (int64_t)rtiles * units * 64;
  pack_split_kernel<<<grid_for(total, 256, 65536), 256, 0, st>>>(src, rows, d, ld, total, units,
                                                                 scale, (u32x4*)dst);
  return hipGetLastError();
}

hipError_t launch_half2_plan(const float* X, int64_t n, int64_t ldx, const float* Y, int64_t m,
                             int64_t ldy, int64_t d, float cx, Half2Plan* plan, hipStream_t st) {
  // about 4 K elements per block (enough workgroups to stream at full
  // bandwidth), at most kHalf2Parts blocks per cloud
  const int nx = grid_for(n * d, 4096, kHalf2Parts);
  const int ny = grid_for(m * d, 4096, kHalf2Parts);
  absmax_kernel<<<nx, 256, 0, st>>>(X, n, d, ldx, plan->part);
  absmax_kernel<<<ny, 256, 0, st>>>(Y, m, d, ldy, plan->part + kHalf2Parts);
  half2_plan_kernel<<<1, 256, 0, st>>>(plan, nx, ny, cx);
  return hipGetLastError();
}

hipError_t launch_pack_half2(const float* src, int64_t rows, int64_t d, int64_t ld, int rtiles,
                             int units, float scale, const Half2Plan* plan, int side, void* dst,
                             hipStream_t st) {
  const int64_t total = (int64_t)rtiles * units * 64;
  pack_half2_kernel<<<grid_for(total, 256, 65536), 256, 0, st>>>(src, rows, d, ld, total, units,
                                                                 scale, plan, side, (u32x4*)dst);
  return hipGetLastError();
}

hipError_t launch_vcol_absmax(const void* V, int bf16, int64_t rows, int64_t cols, int64_t ldv,
                              unsigned* amax, hipStream_t st) {
  fill_kernel<<<grid_for(cols, 256, 65536), 256, 0, st>>>((float*)amax, 0.f, cols);
  dim3 grid((unsigned)((cols + 255) / 256), (unsigned)(rows < 256 ? rows : 256));
  if (bf16)
    vcol_absmax_kernel<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)V, rows, cols, ldv, amax);
  else
    vcol_absmax_kernel<float><<<grid, 256, 0, st>>>((const float*)V, rows, cols, ldv, amax);
  return hipGetLastError();
}

hipError_t launch_pack_values_h2(const void* V, int bf16, int64_t rows, int64_t cols,
                                 int64_t ldv, int ctiles, int pblocks, const unsigned* amax,
                                 void* dst, hipStream_t st) {
  const int64_t total = (int64_t)ctiles * pblocks * 4 * 64;
  const int grid = grid_for(total, 256, 65536);
  if (bf16)
    pack_values_h2_kernel<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)V, rows, cols, ldv,
                                                          total, pblocks, amax, (u32x4*)dst);
  else
    pack_values_h2_kernel<float><<<grid, 256, 0, st>>>((const float*)V, rows, cols, ldv, total,
                                                       pblocks, amax, (u32x4*)dst);
  return hipGetLastError();
}

hipError_t launch_pack_values(const void* V, int bf16, int64_t rows, int64_t cols, int64_t ldv,
                              int ctiles, int pblocks, float* dst, hipStream_t st) {
  const int64_t total = (int64_t)ctiles * pblocks * 4 * 64;
  const int grid = grid_for(total, 256, 65536);
  if (bf16)
    pack_values_kernel<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)V, rows, cols, ldv, total,
                                                       pblocks, (f32x4*)dst);
  else
    pack_values_kernel<float>
        <<<grid, 256, 0, st>>>((const float*)V, rows, cols, ldv, total, pblocks, (f32x4*)dst);
  return hipGetLastError();
}

hipError_t launch_weights(const float* w, int rows, int rpad, float eps, float* wgt, float* hlw,
                          hipStream_t st) {
  weights_kernel<<<(rpad + 255) / 256, 256, 0, st>>>(w, rows, rpad, eps, wgt, hlw);
  return hipGetLastError();
}

hipError_t launch_fill(float* p, float v, int64_t count, hipStream_t st) {
  fill_kernel<<<grid_for(count, 256, 65536), 256, 0, st>>>(p, v, count);
  return hipGetLastError();
}

hipError_t launch_bias_from_pot(const float* pot, const float* norm, const float* hlw, int rows,
                                int rpad, float bscale, float* bias, int parts, hipStream_t st) {
  bias_from_pot_kernel<<<(rpad + 255) / 256, 256, 0, st>>>(pot, norm, hlw, rows, rpad, bscale,
                                                           bias, parts);
  return hipGetLastError();
}

hipError_t launch_lse_merge(const float2* part, int splits, int rpad, int rows, float bscale, float eps,
                            const float* norm, const float* hlw, const float* wgt, float* pot,
                            float* bias_out, float* err_part, int with_err, int write_pot,
                            int avg, hipStream_t st) {
  lse_merge_kernel<<<lse_merge_blocks(rpad), 256, 0, st>>>(part, splits, rpad, rows, bscale, eps, norm,
                                                       hlw, wgt, pot, bias_out, err_part,
                                                       with_err, write_pot, avg);
  return hipGetLastError();
}

hipError_t launch_err_reduce(const float* part, int count, float* out, hipStream_t st) {
  err_reduce_kernel<<<1, 256, 0, st>>>(part, count, out);
  return hipGetLastError();
}

hipError_t launch_nonfinite(const float* f, int n, const float* g, int m, float* out,
                            hipStream_t st) {
  fill_kernel<<<1, 256, 0, st>>>(out, 0.f, 1);
  nonfinite_kernel<<<grid_for((int64_t)n + m, 256, 512), 256, 0, st>>>(f, n, g, m, out);
  return hipGetLastError();
}

hipError_t launch_apply_merge(const float2* partMS, const float* partO, int splits, int rpad,
                              int ppad, int rows, int cols, float c, float eps, const float* pot,
                              const float* norm, const float* wgt, int mode, const void* Xsrc,
                              int xbf16, int64_t ldx, const unsigned* vamax, float* out,
                              float* marg, hipStream_t st) {
  if (splits > kMaxApplySplits) return hipErrorInvalidValue;
  dim3 grid((rows + 31) / 32, (cols + 31) / 32);
  if (xbf16)
    apply_merge_kernel<uint16_t><<<grid, 256, 0, st>>>(partMS, partO, splits, rpad, ppad, rows,
                                                       cols, c, eps, pot, norm, wgt, mode,
                                                       (const uint16_t*)Xsrc, ldx, vamax, out, marg);
  else
    apply_merge_kernel<float><<<grid, 256, 0, st>>>(partMS, partO, splits, rpad, ppad, rows, cols,
                                                    c, eps, pot, norm, wgt, mode,
                                                    (const float*)Xsrc, ldx, vamax, out, marg);
  return hipGetLastError();
}

}  // namespace flashot
