// Vector kernels of the streaming Hessian-vector product ("FlashSinkhorn:
// IO-Aware Entropic Optimal Transport on GPU", §3.3 Thm. 5, App. F.1-F.3,
// App. G.1 "HVP"). The transport products themselves run in the streamed
// apply kernels; these kernels do the O((n + m) d) work around them:
//   - the row terms of E A and of R A (App. F.1, F.2 step 1),
//   - the right side of the damped Schur system (F.2 step 2),
//   - conjugate gradients on S_tau = diag c - P^T diag(1/r) P + tau I with
//     device-side scalars (no host round trip per iteration),
//   - back-substitution and the final G = E A + (1/eps) R^T w (F.2 step 3).
// Rows are handled one wave per row (lanes over the dimension); every
// reduction runs in a fixed order, so results are reproducible.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"

namespace flashot {

namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Sum of 256 values of a workgroup, in a fixed order.
__device__ __forceinline__ float block_sum(float v, float* sh) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  const float t = (sh[0] + sh[1]) + (sh[2] + sh[3]);
  __syncthreads();
  return t;
}

}  // namespace

// Per row i of X (wave per row): xa_i = <x_i, a_i>,
// R1_i = 2 <a_i, r_i x_i - (P Y)_i>, and the values of the P^T pass:
// VB_i = [a_i, xa_i, R1_i / r_i] (d + 2 columns).
__global__ __launch_bounds__(256) void hvp_prep_kernel(int n, int d, const float* __restrict__ X,
                                                       int64_t ldx, const float* __restrict__ A,
                                                       int64_t lda, const float* __restrict__ PY,
                                                       const float* __restrict__ r,
                                                       float* __restrict__ xa,
                                                       float* __restrict__ ra1,
                                                       float* __restrict__ VB) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= n) return;
  const float ri = r[i];
  float sxa = 0.f, sr1 = 0.f;
  for (int k = lane; k < d; k += 64) {
    const float x = X[(int64_t)i * ldx + k];
    const float a = A[(int64_t)i * lda + k];
    const float py = PY[(int64_t)i * d + k];
    sxa = fmaf(x, a, sxa);
    sr1 = fmaf(a, fmaf(ri, x, -py), sr1);
    VB[(int64_t)i * (d + 2) + k] = a;
  }
  sxa = wave_sum(sxa);
  sr1 = 2.f * wave_sum(sr1);
  if (lane == 0) {
    xa[i] = sxa;
    ra1[i] = sr1;
    VB[(int64_t)i * (d + 2) + d] = sxa;
    VB[(int64_t)i * (d + 2) + d + 1] = sr1 / ri;
  }
}

// Per column j (wave per row of Y), from PTV_j = [(P^T A)_j, (P^T xa)_j,
// (P^T (R1/r))_j]: R2_j = 2 ((P^T xa)_j - <y_j, (P^T A)_j>) and the Schur
// right side rhs_j = R2_j - (P^T (R1/r))_j. Starts conjugate gradients from
// w2 = 0: res = p = rhs.
__global__ __launch_bounds__(256) void hvp_rhs_kernel(int m, int d, const float* __restrict__ Y,
                                                      int64_t ldy, const float* __restrict__ PTV,
                                                      float* __restrict__ rhs,
                                                      float* __restrict__ w2,
                                                      float* __restrict__ res,
                                                      float* __restrict__ pdir) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= m) return;
  float t = 0.f;
  for (int k = lane; k < d; k += 64) t = fmaf(Y[(int64_t)j * ldy + k], PTV[(int64_t)j * (d + 2) + k], t);
  t = wave_sum(t);
  if (lane == 0) {
    const float r2 = 2.f * (PTV[(int64_t)j * (d + 2) + d] - t);
    const float b = r2 - PTV[(int64_t)j * (d + 2) + d + 1];
    rhs[j] = b;
    w2[j] = 0.f;
    res[j] = b;
    pdir[j] = b;
  }
}

// ---- conjugate gradients -----------------------------------------------------
// Partial sums: one per workgroup of a fixed grid, reduced by one workgroup.
__global__ __launch_bounds__(256) void cg_dot_kernel(int len, const float* __restrict__ x,
                                                     const float* __restrict__ y,
                                                     float* __restrict__ part) {
  __shared__ float sh[4];
  float s = 0.f;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < len; i += gridDim.x * 256) s = fmaf(x[i], y[i], s);
  s = block_sum(s, sh);
  if (threadIdx.x == 0) part[blockIdx.x] = s;
}

__device__ __forceinline__ float reduce_parts(const float* __restrict__ part, int nparts,
                                              float* sh) {
  float s = 0.f;
  for (int i = threadIdx.x; i < nparts; i += 256) s += part[i];
  return block_sum(s, sh);
}

// rr = bb = ||rhs||^2; the iteration count and flags start at zero; a zero
// right side is solved by w2 = 0 at once.
__global__ __launch_bounds__(256) void cg_start_kernel(const float* __restrict__ part, int nparts,
                                                       CgState* __restrict__ cs) {
  __shared__ float sh[4];
  const float s = reduce_parts(part, nparts, sh);
  if (threadIdx.x == 0) {
    cs->rr = s;
    cs->bb = s;
    cs->alpha = 0.f;
    cs->beta = 0.f;
    cs->iters = 0;
    cs->breakdown = 0;
    cs->done = !(s > 0.f);
  }
}

// u = (P p) / r on the rows.
__global__ __launch_bounds__(256) void cg_div_kernel(int n, const float* __restrict__ Pp,
                                                     const float* __restrict__ r,
                                                     float* __restrict__ u,
                                                     const CgState* __restrict__ cs) {
  if (cs->done) return;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) u[i] = Pp[i] / r[i];
}

// q = S_tau p = c p - P^T u + tau p, and the partial sums of <p, q>.
__global__ __launch_bounds__(256) void cg_op_kernel(int m, const float* __restrict__ c,
                                                    const float* __restrict__ pdir,
                                                    const float* __restrict__ PTu, float tau,
                                                    float* __restrict__ q,
                                                    float* __restrict__ part,
                                                    const CgState* __restrict__ cs) {
  __shared__ float sh[4];
  if (cs->done) return;  // uniform over the grid
  float s = 0.f;
  for (int j = blockIdx.x * 256 + threadIdx.x; j < m; j += gridDim.x * 256) {
    const float pj = pdir[j];
    const float qj = fmaf(c[j] + tau, pj, -PTu[j]);
    q[j] = qj;
    s = fmaf(pj, qj, s);
  }
  s = block_sum(s, sh);
  if (threadIdx.x == 0) part[blockIdx.x] = s;
}

// alpha = rr / <p, q>; a curvature <p, q> that is not positive (S_tau not
// positive definite in this precision, e.g. tau = 0 at rounding level) ends
// the solve and is reported.
__global__ __launch_bounds__(256) void cg_alpha_kernel(const float* __restrict__ part, int nparts,
                                                       CgState* __restrict__ cs) {
  __shared__ float sh[4];
  if (cs->done) return;
  const float pq = reduce_parts(part, nparts, sh);
  if (threadIdx.x == 0) {
    if (!(pq > 0.f)) {
      cs->breakdown = 1;
      cs->done = 1;
    } else {
      cs->alpha = cs->rr / pq;
    }
  }
}

// w2 += alpha p, res -= alpha q, and the partial sums of ||res||^2.
__global__ __launch_bounds__(256) void cg_step_kernel(int m, const float* __restrict__ pdir,
                                                      const float* __restrict__ q,
                                                      float* __restrict__ w2,
                                                      float* __restrict__ res,
                                                      float* __restrict__ part,
                                                      const CgState* __restrict__ cs) {
  __shared__ float sh[4];
  if (cs->done) return;
  const float alpha = cs->alpha;
  float s = 0.f;
  for (int j = blockIdx.x * 256 + threadIdx.x; j < m; j += gridDim.x * 256) {
    w2[j] = fmaf(alpha, pdir[j], w2[j]);
    const float rj = fmaf(-alpha, q[j], res[j]);
    res[j] = rj;
    s = fmaf(rj, rj, s);
  }
  s = block_sum(s, sh);
  if (threadIdx.x == 0) part[blockIdx.x] = s;
}

// beta = ||res_new||^2 / ||res||^2; stop once ||res|| <= tol ||rhs||.
__global__ __launch_bounds__(256) void cg_beta_kernel(const float* __restrict__ part, int nparts,
                                                      float tol2, CgState* __restrict__ cs) {
  __shared__ float sh[4];
  if (cs->done) return;
  const float rn = reduce_parts(part, nparts, sh);
  if (threadIdx.x == 0) {
    cs->beta = rn / cs->rr;
    cs->rr = rn;
    cs->iters += 1;
    if (rn <= tol2 * cs->bb) cs->done = 1;
  }
}

// p = res + beta p.
__global__ __launch_bounds__(256) void cg_dir_kernel(int m, const float* __restrict__ res,
                                                     float* __restrict__ pdir,
                                                     const CgState* __restrict__ cs) {
  if (cs->done) return;
  const float beta = cs->beta;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j < m) pdir[j] = fmaf(beta, pdir[j], res[j]);
}

// Values of the back-substitution pass: VF_j = [w2_j y_j, w2_j] (d + 1 columns).
__global__ __launch_bounds__(256) void hvp_vf_kernel(int m, int d, const float* __restrict__ Y,
                                                     int64_t ldy, const float* __restrict__ w2,
                                                     float* __restrict__ VF) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)m * (d + 1);
  if (e >= total) return;
  const int64_t j = e / (d + 1);
  const int k = (int)(e % (d + 1));
  VF[e] = k < d ? w2[j] * Y[j * ldy + k] : w2[j];
}

// G_i = E A_i + (1/eps) (R^T w)_i, wave per row, with
//   E A_i = 2 r_i a_i - (4/eps)(r_i xa_i x_i - xa_i (PY)_i - <a_i, (PY)_i> x_i + B5_i),
//   w1_i = (R1_i - (P w2)_i) / r_i,
//   (R^T w)_i = 2 (w1_i (r_i x_i - (PY)_i) + (P w2)_i x_i - (P diag(w2) Y)_i),
// where PF_i = [(P diag(w2) Y)_i, (P w2)_i] and B5 = (P . A Y^T) Y.
__global__ __launch_bounds__(256) void hvp_final_kernel(
    int n, int d, float eps, const float* __restrict__ X, int64_t ldx, const float* __restrict__ A,
    int64_t lda, const float* __restrict__ PY, const float* __restrict__ r,
    const float* __restrict__ xa, const float* __restrict__ ra1, const float* __restrict__ PF,
    const float* __restrict__ B5, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= n) return;
  float apy = 0.f;
  for (int k = lane; k < d; k += 64)
    apy = fmaf(A[(int64_t)i * lda + k], PY[(int64_t)i * d + k], apy);
  apy = wave_sum(apy);
  const float ri = r[i], xai = xa[i];
  const float pw = PF[(int64_t)i * (d + 1) + d];
  const float w1 = (ra1[i] - pw) / ri;
  const float k4 = 4.f / eps, k2 = 2.f / eps;
  for (int k = lane; k < d; k += 64) {
    const float x = X[(int64_t)i * ldx + k];
    const float a = A[(int64_t)i * lda + k];
    const float py = PY[(int64_t)i * d + k];
    const float b5 = B5[(int64_t)i * d + k];
    const float pdy = PF[(int64_t)i * (d + 1) + k];
    const float expl = 2.f * ri * a - k4 * (ri * xai * x - xai * py - apy * x + b5);
    const float impl = k2 * (w1 * fmaf(ri, x, -py) + pw * x - pdy);
    out[(int64_t)i * d + k] = expl + impl;
  }
}

// Transport-vector merge: (P v)_i = w_i 2^((pot_i - nrm_i) log2(e)/eps + M) T
// over the split partials (M in log2 units, T rescaled to the common M), in a
// fixed order.
__global__ __launch_bounds__(256) void vec_merge_kernel(
    const float2* __restrict__ part, const float* __restrict__ partT, int splits, int rpad,
    int rows, float eps, const float* __restrict__ pot, const float* __restrict__ norm,
    const float* __restrict__ wgt, float* __restrict__ out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= rows) return;
  float M = part[i].x;
  for (int s = 1; s < splits; ++s) M = fmaxf(M, part[(size_t)s * rpad + i].x);
  float T = 0.f;
  for (int s = 0; s < splits; ++s)
    T = fmaf(partT[(size_t)s * rpad + i], exp2f(part[(size_t)s * rpad + i].x - M), T);
  const float log2e = 1.4426950408889634f;
  out[i] = wgt[i] * exp2f(fmaf(pot[i] - norm[i], log2e / eps, M)) * T;
}

// ---- launchers -------------------------------------------------------------------
hipError_t launch_vec_merge(const float2* part, const float* partT, int splits, int rpad,
                            int rows, float eps, const float* pot, const float* norm,
                            const float* wgt, float* out, hipStream_t st) {
  vec_merge_kernel<<<(rows + 255) / 256, 256, 0, st>>>(part, partT, splits, rpad, rows, eps, pot,
                                                       norm, wgt, out);
  return hipGetLastError();
}

static int rows4(int rows) { return (rows + 3) / 4; }

hipError_t launch_hvp_prep(int n, int d, const float* X, int64_t ldx, const float* A, int64_t lda,
                           const float* PY, const float* r, float* xa, float* ra1, float* VB,
                           hipStream_t st) {
  hvp_prep_kernel<<<rows4(n), 256, 0, st>>>(n, d, X, ldx, A, lda, PY, r, xa, ra1, VB);
  return hipGetLastError();
}

hipError_t launch_hvp_rhs(int m, int d, const float* Y, int64_t ldy, const float* PTV, float* rhs,
                          float* w2, float* res, float* pdir, hipStream_t st) {
  hvp_rhs_kernel<<<rows4(m), 256, 0, st>>>(m, d, Y, ldy, PTV, rhs, w2, res, pdir);
  return hipGetLastError();
}

int cg_parts(int len) {
  const int b = (len + 255) / 256;
  return b < kCgMaxParts ? b : kCgMaxParts;
}

hipError_t launch_cg_start(int m, const float* rhs, float* part, CgState* cs, hipStream_t st) {
  cg_dot_kernel<<<cg_parts(m), 256, 0, st>>>(m, rhs, rhs, part);
  cg_start_kernel<<<1, 256, 0, st>>>(part, cg_parts(m), cs);
  return hipGetLastError();
}

hipError_t launch_cg_div(int n, const float* Pp, const float* r, float* u, const CgState* cs,
                         hipStream_t st) {
  cg_div_kernel<<<(n + 255) / 256, 256, 0, st>>>(n, Pp, r, u, cs);
  return hipGetLastError();
}

hipError_t launch_cg_update(int m, const float* c, const float* PTu, float tau, float tol,
                            float* pdir, float* q, float* w2, float* res, float* part,
                            CgState* cs, hipStream_t st) {
  const int np = cg_parts(m);
  cg_op_kernel<<<np, 256, 0, st>>>(m, c, pdir, PTu, tau, q, part, cs);
  cg_alpha_kernel<<<1, 256, 0, st>>>(part, np, cs);
  cg_step_kernel<<<np, 256, 0, st>>>(m, pdir, q, w2, res, part, cs);
  cg_beta_kernel<<<1, 256, 0, st>>>(part, np, tol * tol, cs);
  cg_dir_kernel<<<(m + 255) / 256, 256, 0, st>>>(m, res, pdir, cs);
  return hipGetLastError();
}

hipError_t launch_hvp_vf(int m, int d, const float* Y, int64_t ldy, const float* w2, float* VF,
                         hipStream_t st) {
  const int64_t total = (int64_t)m * (d + 1);
  hvp_vf_kernel<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(m, d, Y, ldy, w2, VF);
  return hipGetLastError();
}

hipError_t launch_hvp_final(int n, int d, float eps, const float* X, int64_t ldx, const float* A,
                            int64_t lda, const float* PY, const float* r, const float* xa,
                            const float* ra1, const float* PF, const float* B5, float* out,
                            hipStream_t st) {
  hvp_final_kernel<<<rows4(n), 256, 0, st>>>(n, d, eps, X, ldx, A, lda, PY, r, xa, ra1, PF, B5,
                                               out);
  return hipGetLastError();
}

}  // namespace flashot
