// gfx950 kernels of the streamed log-domain Sinkhorn solver.
//
// Method: "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU"
// (arXiv 2602.03067). A Sinkhorn half-step is a row-wise log-sum-exp of the
// biased dot-product score 2 x_i.y_j/eps + bias_j (Prop. 1, App. D.1); it is
// streamed over column tiles with a running max and rescaled sum (App. D.3)
// and only the potentials are written back (App. D.2, G.1). Transport
// application P V reuses the same row softmax and accumulates V tiles
// (Prop. 3, App. E.1, Algorithm 2; G.2 row-stationary loop order).
//
// MI355X design (not the page's Triton/A100 one):
//  * the score tile is formed on the matrix cores with a 32x32 output per
//    wave, computed TRANSPOSED (columns j on the M axis, rows i on the N
//    axis). In the 32x32 accumulator layout lane l then holds 16 values of
//    ONE output row (i = l % 32), so the online LSE is lane-local: no
//    cross-lane traffic inside the column loop, one exchange with lane
//    l ^ 32 at the very end;
//  * the per-column bias enters the accumulator through one extra fp32 MFMA
//    (A = bias column, B = ones), so a score needs one FMA (scale and
//    subtract the running max) plus one exp2 and one add on the VALU;
//  * operands are pre-packed once per call into the exact register layout of
//    the MFMA (16 contiguous bytes per lane, zero-padded tiles), so every
//    load in the hot loop is a full 1 KiB coalesced wave load with no masks;
//  * the streamed axis is split over workgroups when the output axis alone
//    cannot fill 256 CUs; partial (max, sum) pairs are merged afterwards in a
//    fixed order with the exact merge of App. D.3, so results are
//    deterministic. Split indices are the fastest-varying part of the
//    workgroup index, which keeps one split's column tiles on one XCD (its
//    own L2) when the split count is a multiple of 8.
//  * P V reuses the exponentiated score registers directly as the B operand
//    of a second MFMA: O^T (p x i) += V^T (p x j) P^T (j x i). The rows of V
//    are pre-permuted into the accumulator's row order, so P never leaves
//    registers and the running rescale of O is lane-local.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include "kernels.h"

namespace flashot {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One packed k-block of the score tile: acc[j][i] += sum_k A[j][k] B[k][i].
template <bool BF16>
__device__ __forceinline__ f32x16 mfma_kblock(u32x4 a, u32x4 b, f32x16 acc) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  } else {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0,
                                               0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0,
                                               0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0,
                                               0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0,
                                               0, 0);
    return acc;
  }
}

// Operand modes of the register-resident pass.
constexpr int kModeF32 = 0;    // fp32 operands, fp32 MFMA (32x32x2)
constexpr int kModeBF16 = 1;   // bf16 operands, bf16 MFMA (32x32x16)
constexpr int kModeSplit = 2;  // fp32 operands as hi + mid + lo bf16 parts, bf16 MFMA

// One k-block of 16 fp32 values held as three bf16 parts per operand
// (v = hi + mid + lo, each part the bf16 rounding of what the previous ones
// left, so |mid| <= 2^-9 |v| and |lo| <= 2^-18 |v|). Six partial products are
// accumulated, smallest first; the three dropped ones (mid*lo, lo*mid, lo*lo)
// are below 2^-26 of |x y|, finer than fp32 rounding.
__device__ __forceinline__ f32x16 mfma_split(const u32x4* y, const u32x4* x, f32x16 acc) {
  auto m = [](u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  };
  acc = m(y[2], x[0], acc);  // lo * hi
  acc = m(y[0], x[2], acc);  // hi * lo
  acc = m(y[1], x[1], acc);  // mid * mid
  acc = m(y[1], x[0], acc);  // mid * hi
  acc = m(y[0], x[1], acc);  // hi * mid
  return m(y[0], x[0], acc); // hi * hi
}

// Adds bias_j to every accumulator entry of column j: k-slot 0 carries
// (bias_j, 1), k-slot 1 carries (0, 1).
__device__ __forceinline__ f32x16 mfma_bias(float wv, int h, f32x16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(h ? 0.0f : wv, 1.0f, acc, 0, 0, 0);
}

__device__ __forceinline__ float max16(const f32x16& v) {
  float a = fmaxf(fmaxf(v[0], v[1]), v[2]);
  float b = fmaxf(fmaxf(v[3], v[4]), v[5]);
  float d = fmaxf(fmaxf(v[6], v[7]), v[8]);
  float e = fmaxf(fmaxf(v[9], v[10]), v[11]);
  float f = fmaxf(fmaxf(v[12], v[13]), v[14]);
  return fmaxf(fmaxf(a, b), fmaxf(fmaxf(d, e), fmaxf(f, v[15])));
}

// Online LSE step of App. D.3 on 16 scores of one row, in "dot-product units":
// the natural-log score is (2/eps) * v, and c = 2 log2(e) / eps, so
// exp(score - max) = exp2(c * (v - M)).
__device__ __forceinline__ void lse_tile(const f32x16& v, float& M, float& S, float c) {
  const float Mn = fmaxf(M, max16(v));
  const float cm = c * Mn;
  const float sc = __builtin_amdgcn_exp2f(fmaf(c, M, -cm));
  float s0 = __builtin_amdgcn_exp2f(fmaf(c, v[0], -cm));
  float s1 = __builtin_amdgcn_exp2f(fmaf(c, v[1], -cm));
  float s2 = __builtin_amdgcn_exp2f(fmaf(c, v[2], -cm));
  float s3 = __builtin_amdgcn_exp2f(fmaf(c, v[3], -cm));
#pragma unroll
  for (int r = 4; r < 16; r += 4) {
    s0 += __builtin_amdgcn_exp2f(fmaf(c, v[r + 0], -cm));
    s1 += __builtin_amdgcn_exp2f(fmaf(c, v[r + 1], -cm));
    s2 += __builtin_amdgcn_exp2f(fmaf(c, v[r + 2], -cm));
    s3 += __builtin_amdgcn_exp2f(fmaf(c, v[r + 3], -cm));
  }
  S = fmaf(S, sc, (s0 + s1) + (s2 + s3));
  M = Mn;
}

// ---------------------------------------------------------------------------
// Streamed log-sum-exp partials (Algorithm 1 / 3 of the page).
//   part[s][row] = (M, S) with LSE_row over split s = (2/eps) M + ln S.
// Grid: nrowgroups * splits workgroups of 4 waves; wave w of row group g owns
// row tiles (4 g + w) * RI ... + RI - 1 and streams the column tiles of its split.
// ---------------------------------------------------------------------------
template <bool BF16, int KB, int RI, bool XRES>
__global__ __launch_bounds__(256) void lse_partial_kernel(
    const u32x4* __restrict__ Rp, const u32x4* __restrict__ Cp, const float* __restrict__ cbias,
    int rtiles, int ctiles, int kbp, int splits, int tps, float c, float2* __restrict__ part,
    int rpad) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int s = blockIdx.x % splits;
  const int rg = blockIdx.x / splits;
  const int rt0 = (rg * kWaves + wave) * RI;
  if (rt0 >= rtiles) return;
  const int jt0 = s * tps;
  const int jt1 = min(jt0 + tps, ctiles);

  int rt[RI];
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) rt[ri] = min(rt0 + ri, rtiles - 1);

  u32x4 xr[RI][KB];
  if constexpr (XRES) {
#pragma unroll
    for (int ri = 0; ri < RI; ++ri)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) xr[ri][kb] = Rp[((size_t)rt[ri] * KB + kb) * 64 + lane];
  }

  float M[RI], S[RI];
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) {
    M[ri] = -1.0e30f;
    S[ri] = 0.f;
  }

  if constexpr (XRES) {
    // Double-buffered column operand: tile jt+1 is in flight while jt is used.
    u32x4 yn[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) yn[kb] = Cp[((size_t)jt0 * KB + kb) * 64 + lane];
    float wn = cbias[jt0 * kTile + (lane & 31)];
    for (int jt = jt0; jt < jt1; ++jt) {
      u32x4 yc[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) yc[kb] = yn[kb];
      const float wv = wn;
      const int jn = min(jt + 1, jt1 - 1);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) yn[kb] = Cp[((size_t)jn * KB + kb) * 64 + lane];
      wn = cbias[jn * kTile + (lane & 31)];

      f32x16 acc[RI];
#pragma unroll
      for (int ri = 0; ri < RI; ++ri) acc[ri] = f32x16{};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int ri = 0; ri < RI; ++ri) acc[ri] = mfma_kblock<BF16>(yc[kb], xr[ri][kb], acc[ri]);
#pragma unroll
      for (int ri = 0; ri < RI; ++ri) acc[ri] = mfma_bias(wv, h, acc[ri]);
#pragma unroll
      for (int ri = 0; ri < RI; ++ri) lse_tile(acc[ri], M[ri], S[ri], c);
    }
  } else {
    for (int jt = jt0; jt < jt1; ++jt) {
      f32x16 acc[RI];
#pragma unroll
      for (int ri = 0; ri < RI; ++ri) acc[ri] = f32x16{};
      for (int kc = 0; kc < kbp; kc += KB) {
        u32x4 yc[KB];
        u32x4 xc[RI][KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) yc[kb] = Cp[((size_t)jt * kbp + kc + kb) * 64 + lane];
#pragma unroll
        for (int ri = 0; ri < RI; ++ri)
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
            xc[ri][kb] = Rp[((size_t)rt[ri] * kbp + kc + kb) * 64 + lane];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int ri = 0; ri < RI; ++ri) acc[ri] = mfma_kblock<BF16>(yc[kb], xc[ri][kb], acc[ri]);
      }
      const float wv = cbias[jt * kTile + (lane & 31)];
#pragma unroll
      for (int ri = 0; ri < RI; ++ri) acc[ri] = mfma_bias(wv, h, acc[ri]);
#pragma unroll
      for (int ri = 0; ri < RI; ++ri) lse_tile(acc[ri], M[ri], S[ri], c);
    }
  }

  // Merge the two half-waves that share a row (App. D.3 merge of partial statistics).
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) {
    const float Mp = __shfl_xor(M[ri], 32);
    const float Sp = __shfl_xor(S[ri], 32);
    const float Mt = fmaxf(M[ri], Mp);
    const float cm = c * Mt;
    const float St = S[ri] * __builtin_amdgcn_exp2f(fmaf(c, M[ri], -cm)) +
                     Sp * __builtin_amdgcn_exp2f(fmaf(c, Mp, -cm));
    if (h == 0 && rt0 + ri < rtiles)
      part[(size_t)s * rpad + (size_t)(rt0 + ri) * kTile + (lane & 31)] = make_float2(c * Mt, St);
  }
}

// ---------------------------------------------------------------------------
// Software-pipelined register-resident pass with a lazily raised stabiliser.
//
// Pipelining: each wave keeps two score tiles in flight. While the matrix
// cores form the scores of column tile t+1, the vector unit exponentiates
// tile t. The column operand alternates between two register buffers (the
// loop body is written twice with the roles swapped), so a prefetched tile is
// never copied between registers.
//
// Lazy stabiliser: the online LSE of App. D.3 is exact for any running
// stabiliser M, not only for the running maximum. The bias MFMA uses its
// second k-slot to subtract M_i from every score (A = [bias_j, 1],
// B = [1, -M_i]), so in the common case a tile costs one exp2 and one add per
// score. Only when a tile could overflow (tile sum >= 2^64), or before M has
// been set from data, does the wave take the exact path: tile maximum, raise
// M, rescale S. M is kept identical in the two lanes (l, l ^ 32) that share a
// row, because the bias MFMA reads it from lane l + 32.
//
// Units: for fp32 inputs the row operand X is packed pre-multiplied by
// c = 2 log2(e) / eps and the biases are written in the same units, so scores
// are log2 values and exp2 needs no multiply (KS = 1). bf16 operands cannot be
// rescaled without rounding, so their scores stay in dot-product units and
// are multiplied by c before exp2 (KS = c). Partials are written in log2
// units: LSE_row = ln 2 * (M2 + log2 S).
// ---------------------------------------------------------------------------
constexpr float kUnset = -1.0e30f;  // stabiliser not yet taken from data

// KB counts 1 KiB operand units per tile: one per k-block for fp32 / bf16,
// three (hi, mid, lo) per k-block in split mode.
template <int MODE, int KB, int RI>
__device__ __forceinline__ void score_tile(const u32x4 (&y)[KB], const u32x4 (&xr)[RI][KB],
                                           float wv, int h, const float (&Mf)[RI],
                                           f32x16 (&acc)[RI]) {
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) acc[ri] = f32x16{};
  if constexpr (MODE == kModeSplit) {
#pragma unroll
    for (int kb = 0; kb < KB; kb += 3)
#pragma unroll
      for (int ri = 0; ri < RI; ++ri) acc[ri] = mfma_split(&y[kb], &xr[ri][kb], acc[ri]);
  } else {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
        acc[ri] = mfma_kblock<MODE == kModeBF16>(y[kb], xr[ri][kb], acc[ri]);
  }
#pragma unroll
  for (int ri = 0; ri < RI; ++ri)
    acc[ri] = __builtin_amdgcn_mfma_f32_32x32x2f32(h ? 1.0f : wv, h ? -Mf[ri] : 1.0f, acc[ri],
                                                   0, 0, 0);
}

// Stabiliser folded into the next tile's scores: the running M once set.
__device__ __forceinline__ float fold_of(float M) { return M > 0.5f * kUnset ? M : 0.f; }

// Common-case tile: s = sum exp2(ks * a_r) relative to the folded Mf; returns
// the candidate new S and whether the exact path is needed.
template <bool SCALED>
__device__ __forceinline__ bool lse_fast(const f32x16& a, float Mf, float M, float S, float ks,
                                         float& Snew) {
  float e0 = __builtin_amdgcn_exp2f(SCALED ? a[0] : ks * a[0]);
  float e1 = __builtin_amdgcn_exp2f(SCALED ? a[1] : ks * a[1]);
  float e2 = __builtin_amdgcn_exp2f(SCALED ? a[2] : ks * a[2]);
  float e3 = __builtin_amdgcn_exp2f(SCALED ? a[3] : ks * a[3]);
#pragma unroll
  for (int r = 4; r < 16; r += 4) {
    e0 += __builtin_amdgcn_exp2f(SCALED ? a[r + 0] : ks * a[r + 0]);
    e1 += __builtin_amdgcn_exp2f(SCALED ? a[r + 1] : ks * a[r + 1]);
    e2 += __builtin_amdgcn_exp2f(SCALED ? a[r + 2] : ks * a[r + 2]);
    e3 += __builtin_amdgcn_exp2f(SCALED ? a[r + 3] : ks * a[r + 3]);
  }
  const float s = (e0 + e1) + (e2 + e3);
  Snew = fmaf(s, __builtin_amdgcn_exp2f(ks * (Mf - M)), S);
  return !(s < 0x1p64f) || !(Snew >= 0x1p-64f) || !(M > 0.5f * kUnset);
}

// Exact tile: raise M to the tile maximum (shared by the lane pair), rescale.
__device__ __forceinline__ void lse_exact(const f32x16& a, float Mf, float& M, float& S,
                                          float ks) {
  float m = max16(a) + Mf;
  m = fmaxf(m, __shfl_xor(m, 32));
  m = fmaxf(m, M);
  const float t = Mf - m;
  float e0 = 0.f, e1 = 0.f, e2 = 0.f, e3 = 0.f;
#pragma unroll
  for (int r = 0; r < 16; r += 4) {
    e0 += __builtin_amdgcn_exp2f(ks * (a[r + 0] + t));
    e1 += __builtin_amdgcn_exp2f(ks * (a[r + 1] + t));
    e2 += __builtin_amdgcn_exp2f(ks * (a[r + 2] + t));
    e3 += __builtin_amdgcn_exp2f(ks * (a[r + 3] + t));
  }
  S = fmaf(S, __builtin_amdgcn_exp2f(ks * (M - m)), (e0 + e1) + (e2 + e3));
  M = m;
}

template <int KB>
__device__ __forceinline__ void load_ctile(const u32x4* __restrict__ Cp,
                                           const float* __restrict__ cbias, int jt, int lane,
                                           u32x4 (&y)[KB], float& w) {
  w = cbias[jt * kTile + (lane & 31)];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) y[kb] = Cp[((size_t)jt * KB + kb) * 64 + lane];
}

// Orders one pipeline stage (one scheduling region): one matrix instruction
// alternating with a few vector instructions, then the loads that refill the
// column buffer the matrix instructions have just read.
template <int MODE, int KB, int RI>
__device__ __forceinline__ void stage_schedule() {
  constexpr int kPerUnit = MODE == kModeF32 ? 4 : (MODE == kModeBF16 ? 1 : 2);
  constexpr int kMfma = RI * (KB * kPerUnit + 1);
  constexpr int kValu = RI * (MODE == kModeBF16 ? 40 : 24);  // common-case LSE of RI tiles
  constexpr int kValuPer = (kValu + kMfma - 1) / kMfma;
#pragma unroll
  for (int i = 0; i < kMfma; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, kValuPer, 0);  // VALU
  }
  __builtin_amdgcn_sched_group_barrier(0x020, KB + 1, 0);      // VMEM reads
}

// One pipeline stage: scores of the next tile into accN (folding the current
// stabiliser), common-case LSE of the current tile accC, refill of the buffer
// yN just consumed; then, outside the scheduled region, the exact path for
// the waves that need it.
template <int MODE, int KB, int RI>
__device__ __forceinline__ void pipe_stage(const u32x4* __restrict__ Cp,
                                           const float* __restrict__ cbias, int jt_refill,
                                           int lane, int h, float ks, const u32x4 (&xr)[RI][KB],
                                           u32x4 (&yN)[KB], float& wN, f32x16 (&accN)[RI],
                                           float (&MfN)[RI], const f32x16 (&accC)[RI],
                                           const float (&MfC)[RI], float (&M)[RI],
                                           float (&S)[RI]) {
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) MfN[ri] = fold_of(M[ri]);
  score_tile<MODE, KB, RI>(yN, xr, wN, h, MfN, accN);
  float Sn[RI];
  bool slow = false;
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) slow |= lse_fast<MODE != kModeBF16>(accC[ri], MfC[ri], M[ri], S[ri], ks, Sn[ri]);
  load_ctile<KB>(Cp, cbias, jt_refill, lane, yN, wN);
  stage_schedule<MODE, KB, RI>();
  __builtin_amdgcn_sched_barrier(0);
  if (__builtin_amdgcn_ballot_w64(slow) != 0) {
#pragma unroll
    for (int ri = 0; ri < RI; ++ri) lse_exact(accC[ri], MfC[ri], M[ri], S[ri], ks);
  } else {
#pragma unroll
    for (int ri = 0; ri < RI; ++ri) S[ri] = Sn[ri];
  }
}

// LSE of a tile outside the pipelined loop (the last one or two of a split).
template <int MODE, int RI>
__device__ __forceinline__ void lse_tail(const f32x16 (&acc)[RI], const float (&Mf)[RI],
                                         float (&M)[RI], float (&S)[RI], float ks) {
  float Sn[RI];
  bool slow = false;
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) slow |= lse_fast<MODE != kModeBF16>(acc[ri], Mf[ri], M[ri], S[ri], ks, Sn[ri]);
  if (__builtin_amdgcn_ballot_w64(slow) != 0) {
#pragma unroll
    for (int ri = 0; ri < RI; ++ri) lse_exact(acc[ri], Mf[ri], M[ri], S[ri], ks);
  } else {
#pragma unroll
    for (int ri = 0; ri < RI; ++ri) S[ri] = Sn[ri];
  }
}

template <int MODE, int KB, int RI>
__global__ __launch_bounds__(256) void lse_pipe_kernel(
    const u32x4* __restrict__ Rp, const u32x4* __restrict__ Cp, const float* __restrict__ cbias,
    int rtiles, int ctiles, int splits, int tps, float c, float2* __restrict__ part, int rpad) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int s = blockIdx.x % splits;
  const int rg = blockIdx.x / splits;
  const int rt0 = (rg * kWaves + wave) * RI;
  if (rt0 >= rtiles) return;
  const int jt0 = s * tps;
  const int last = min(jt0 + tps, ctiles) - 1 - jt0;  // split holds tiles 0..last, last >= 0
  const float ks = MODE == kModeBF16 ? c : 1.0f;

  u32x4 xr[RI][KB];
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) {
    const int rt = min(rt0 + ri, rtiles - 1);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) xr[ri][kb] = Rp[((size_t)rt * KB + kb) * 64 + lane];
  }
  float M[RI], S[RI];
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) {
    M[ri] = kUnset;
    S[ri] = 0.f;
  }

  // Invariant at the top of the loop: accA holds the scores of tile k (with
  // MfA folded in), yB holds (or is loading) tile k+1 and yA tile k+2;
  // indices past the split's last tile are clamped to it (loaded, never
  // reduced).
  u32x4 yA[KB], yB[KB];
  float wA, wB;
  f32x16 accA[RI], accB[RI];
  float MfA[RI], MfB[RI];
  load_ctile<KB>(Cp, cbias, jt0, lane, yA, wA);
  load_ctile<KB>(Cp, cbias, jt0 + min(1, last), lane, yB, wB);
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) MfA[ri] = 0.f;
  score_tile<MODE, KB, RI>(yA, xr, wA, h, MfA, accA);
  load_ctile<KB>(Cp, cbias, jt0 + min(2, last), lane, yA, wA);
  int k = 0;
  for (; k + 2 <= last; k += 2) {
    pipe_stage<MODE, KB, RI>(Cp, cbias, jt0 + min(k + 3, last), lane, h, ks, xr, yB, wB, accB,
                             MfB, accA, MfA, M, S);
    pipe_stage<MODE, KB, RI>(Cp, cbias, jt0 + min(k + 4, last), lane, h, ks, xr, yA, wA, accA,
                             MfA, accB, MfB, M, S);
  }
  if (k + 1 <= last) {  // tiles k and k+1 remain
    lse_tail<MODE, RI>(accA, MfA, M, S, ks);
#pragma unroll
    for (int ri = 0; ri < RI; ++ri) MfB[ri] = fold_of(M[ri]);
    score_tile<MODE, KB, RI>(yB, xr, wB, h, MfB, accB);
    lse_tail<MODE, RI>(accB, MfB, M, S, ks);
  } else {  // tile k remains
    lse_tail<MODE, RI>(accA, MfA, M, S, ks);
  }

  // The lane pair shares M: the row's partial is (M in log2 units, S + S').
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) {
    const float St = S[ri] + __shfl_xor(S[ri], 32);
    if (h == 0 && rt0 + ri < rtiles)
      part[(size_t)s * rpad + (size_t)(rt0 + ri) * kTile + (lane & 31)] =
          make_float2(ks * M[ri], St);
  }
}

// ---------------------------------------------------------------------------
// LDS-shared variant of the pipelined pass. The four waves of a workgroup
// own different row tiles but stream the same column tiles, so each column
// tile is fetched from L2 once per workgroup into LDS (double-buffered, one
// barrier per stage) and every wave reads its MFMA fragments from there:
// one quarter of the L2 traffic of per-wave loads, and the register file
// holds row tiles instead of column buffers.
// ---------------------------------------------------------------------------
// Column-tile staging without branches (a branch would split the scheduled
// region): thread t moves entries t, t + 256, ... of the tile's KB * 64
// 16-byte entries; threads past the end re-read the last entry and write it
// into the padding of the LDS buffer, which holds a multiple of 256 entries.
template <int KB>
constexpr int stage_loads() { return (KB * 64 + 255) / 256; }

template <int KB>
__device__ __forceinline__ void stage_load(const u32x4* __restrict__ Cp, int jt, int tid,
                                           u32x4 (&g)[stage_loads<KB>()]) {
#pragma unroll
  for (int i = 0; i < stage_loads<KB>(); ++i)
    g[i] = Cp[(size_t)jt * KB * 64 + min(tid + 256 * i, KB * 64 - 1)];
}

template <int KB>
__device__ __forceinline__ void stage_store(u32x4* __restrict__ buf, int tid,
                                            const u32x4 (&g)[stage_loads<KB>()]) {
#pragma unroll
  for (int i = 0; i < stage_loads<KB>(); ++i) buf[tid + 256 * i] = g[i];
}

template <int MODE, int KB, int RI>
__device__ __forceinline__ void score_tile_lds(const u32x4* __restrict__ buf, int lane,
                                               const u32x4 (&xr)[RI][KB], float wv, int h,
                                               const float (&Mf)[RI], f32x16 (&acc)[RI]) {
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) acc[ri] = f32x16{};
  if constexpr (MODE == kModeSplit) {
#pragma unroll
    for (int kb = 0; kb < KB; kb += 3) {
      u32x4 y[3];
#pragma unroll
      for (int q = 0; q < 3; ++q) y[q] = buf[(kb + q) * 64 + lane];
#pragma unroll
      for (int ri = 0; ri < RI; ++ri) acc[ri] = mfma_split(y, &xr[ri][kb], acc[ri]);
    }
  } else {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const u32x4 y = buf[kb * 64 + lane];
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
        acc[ri] = mfma_kblock<MODE == kModeBF16>(y, xr[ri][kb], acc[ri]);
    }
  }
#pragma unroll
  for (int ri = 0; ri < RI; ++ri)
    acc[ri] = __builtin_amdgcn_mfma_f32_32x32x2f32(h ? 1.0f : wv, h ? -Mf[ri] : 1.0f, acc[ri],
                                                   0, 0, 0);
}

template <int MODE, int KB, int RI>
__device__ __forceinline__ void stage_schedule_lds() {
  constexpr int kPerUnit = MODE == kModeF32 ? 4 : (MODE == kModeBF16 ? 1 : 2);
  constexpr int kMfma = RI * (KB * kPerUnit + 1);
  constexpr int kValu = RI * (MODE == kModeBF16 ? 40 : 24);
  constexpr int kValuPer = (kValu + kMfma - 1) / kMfma;
  constexpr int kLoads = stage_loads<KB>();
  __builtin_amdgcn_sched_group_barrier(0x020, kLoads + 1, 0);  // next tile + bias from L2
#pragma unroll
  for (int i = 0; i < kMfma; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);         // LDS read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, kValuPer, 0);  // VALU
  }
  __builtin_amdgcn_sched_group_barrier(0x200, kLoads, 0);      // LDS write of the next tile
}

template <int MODE, int KB, int RI>
__global__ __launch_bounds__(256) void lse_lds_kernel(
    const u32x4* __restrict__ Rp, const u32x4* __restrict__ Cp, const float* __restrict__ cbias,
    int rtiles, int ctiles, int splits, int tps, float c, float2* __restrict__ part, int rpad) {
  constexpr int kLoads = stage_loads<KB>();
  __shared__ u32x4 lds[2][kLoads * 256];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int s = blockIdx.x % splits;
  const int rg = blockIdx.x / splits;
  const int rt0 = (rg * kWaves + wave) * RI;  // may be past the last row tile: the wave still
                                              // takes part in loads and barriers
  const int jt0 = s * tps;
  const int last = min(jt0 + tps, ctiles) - 1 - jt0;
  const float ks = MODE == kModeBF16 ? c : 1.0f;

  u32x4 xr[RI][KB];
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) {
    const int rt = min(rt0 + ri, rtiles - 1);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) xr[ri][kb] = Rp[((size_t)rt * KB + kb) * 64 + lane];
  }
  float M[RI], S[RI];
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) {
    M[ri] = kUnset;
    S[ri] = 0.f;
  }

  u32x4 g[kLoads];
  stage_load<KB>(Cp, jt0, tid, g);
  stage_store<KB>(lds[0], tid, g);
  stage_load<KB>(Cp, jt0 + min(1, last), tid, g);
  stage_store<KB>(lds[1], tid, g);
  float wA = cbias[jt0 * kTile + (lane & 31)];
  float wB = cbias[(jt0 + min(1, last)) * kTile + (lane & 31)];
  __syncthreads();

  // Invariant at stage k: accA / accB alternate holding the scores of tile k;
  // LDS buffer (k + 1) & 1 holds tile k+1; buffer k & 1 is free once every
  // wave has passed the stage barrier.
  f32x16 accA[RI], accB[RI];
  float MfA[RI], MfB[RI];
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) MfA[ri] = 0.f;
  score_tile_lds<MODE, KB, RI>(lds[0], lane, xr, wA, h, MfA, accA);

  auto stage = [&](int k, f32x16(&accN)[RI], float(&MfN)[RI], float& wN, const f32x16(&accC)[RI],
                   const float(&MfC)[RI], float& wC) {
    __syncthreads();  // tile k+1 is in LDS; every wave is done reading tile k's buffer
    const int jt2 = jt0 + min(k + 2, last);
    stage_load<KB>(Cp, jt2, tid, g);
    const float w2 = cbias[jt2 * kTile + (lane & 31)];
#pragma unroll
    for (int ri = 0; ri < RI; ++ri) MfN[ri] = fold_of(M[ri]);
    score_tile_lds<MODE, KB, RI>(lds[(k + 1) & 1], lane, xr, wN, h, MfN, accN);
    float Sn[RI];
    bool slow = false;
#pragma unroll
    for (int ri = 0; ri < RI; ++ri)
      slow |= lse_fast<MODE != kModeBF16>(accC[ri], MfC[ri], M[ri], S[ri], ks, Sn[ri]);
    stage_store<KB>(lds[k & 1], tid, g);
    wC = w2;  // the buffer of tile k now receives tile k+2
    stage_schedule_lds<MODE, KB, RI>();
    __builtin_amdgcn_sched_barrier(0);
    if (__builtin_amdgcn_ballot_w64(slow) != 0) {
#pragma unroll
      for (int ri = 0; ri < RI; ++ri) lse_exact(accC[ri], MfC[ri], M[ri], S[ri], ks);
    } else {
#pragma unroll
      for (int ri = 0; ri < RI; ++ri) S[ri] = Sn[ri];
    }
  };

  int k = 0;
  for (; k + 2 <= last; k += 2) {
    stage(k, accB, MfB, wB, accA, MfA, wA);
    stage(k + 1, accA, MfA, wA, accB, MfB, wB);
  }
  if (k + 1 <= last) {  // tiles k and k+1 remain; tile k+1 is in buffer (k+1)&1
    __syncthreads();
#pragma unroll
    for (int ri = 0; ri < RI; ++ri) MfB[ri] = fold_of(M[ri]);
    score_tile_lds<MODE, KB, RI>(lds[(k + 1) & 1], lane, xr, wB, h, MfB, accB);
    lse_tail<MODE, RI>(accA, MfA, M, S, ks);
    lse_tail<MODE, RI>(accB, MfB, M, S, ks);
  } else {
    lse_tail<MODE, RI>(accA, MfA, M, S, ks);
  }

#pragma unroll
  for (int ri = 0; ri < RI; ++ri) {
    const float St = S[ri] + __shfl_xor(S[ri], 32);
    if (h == 0 && rt0 + ri < rtiles)
      part[(size_t)s * rpad + (size_t)(rt0 + ri) * kTile + (lane & 31)] =
          make_float2(ks * M[ri], St);
  }
}

// ---------------------------------------------------------------------------
// Streamed transport application partials (Algorithm 2 / 4 of the page).
// Per split s and row i: (M, S) as in the LSE pass, and
//   O[p] = sum_j exp2(c (v_ij - M)) V[j][p]
// accumulated as O^T (p x i) += V^T (p x j) P^T (j x i) on the matrix cores.
// Both half-waves of a row share the running max, so O needs no merge.
// Grid: (nrowgroups * splits, passes); pass y covers value blocks
// [y * PB, y * PB + PB) of 32 columns each.
// ---------------------------------------------------------------------------
template <bool BF16, int KB, bool XRES, int PB>
__global__ __launch_bounds__(256) void apply_partial_kernel(
    const u32x4* __restrict__ Rp, const u32x4* __restrict__ Cp, const float* __restrict__ cbias,
    const f32x4* __restrict__ Vp, int rtiles, int ctiles, int kbp, int splits, int tps, float c,
    int pblocks, float2* __restrict__ partMS, float* __restrict__ partO, int rpad, int ppad) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int s = blockIdx.x % splits;
  const int rg = blockIdx.x / splits;
  const int rt = rg * kWaves + wave;
  if (rt >= rtiles) return;
  const int pb0 = blockIdx.y * PB;
  const int jt0 = s * tps;
  const int jt1 = min(jt0 + tps, ctiles);

  u32x4 xr[KB];
  if constexpr (XRES) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) xr[kb] = Rp[((size_t)rt * KB + kb) * 64 + lane];
  }
  float M = -1.0e30f, S = 0.f;
  f32x16 O[PB];
#pragma unroll
  for (int pb = 0; pb < PB; ++pb) O[pb] = f32x16{};

  for (int jt = jt0; jt < jt1; ++jt) {
    f32x16 acc = f32x16{};
    if constexpr (XRES) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        acc = mfma_kblock<BF16>(Cp[((size_t)jt * KB + kb) * 64 + lane], xr[kb], acc);
    } else {
      for (int kc = 0; kc < kbp; kc += KB) {
        u32x4 yc[KB], xc[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          yc[kb] = Cp[((size_t)jt * kbp + kc + kb) * 64 + lane];
          xc[kb] = Rp[((size_t)rt * kbp + kc + kb) * 64 + lane];
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) acc = mfma_kblock<BF16>(yc[kb], xc[kb], acc);
      }
    }
    acc = mfma_bias(cbias[jt * kTile + (lane & 31)], h, acc);

    // Running max shared by the lane pair (l, l ^ 32) that holds row i.
    float mx = max16(acc);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float Mn = fmaxf(M, mx);
    const float cm = c * Mn;
    const float sc = __builtin_amdgcn_exp2f(fmaf(c, M, -cm));
    M = Mn;
    S *= sc;
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) O[pb] *= sc;
    float p[16];
    float ssum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = __builtin_amdgcn_exp2f(fmaf(c, acc[r], -cm));
      ssum += p[r];
    }
    S += ssum;
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) {
      if (pb0 + pb < pblocks) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 vv = Vp[(((size_t)jt * pblocks + pb0 + pb) * 4 + q) * 64 + lane];
          O[pb] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv[0], p[4 * q + 0], O[pb], 0, 0, 0);
          O[pb] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv[1], p[4 * q + 1], O[pb], 0, 0, 0);
          O[pb] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv[2], p[4 * q + 2], O[pb], 0, 0, 0);
          O[pb] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv[3], p[4 * q + 3], O[pb], 0, 0, 0);
        }
      }
    }
  }

  S += __shfl_xor(S, 32);
  const size_t row = (size_t)rt * kTile + (lane & 31);
  if (blockIdx.y == 0 && h == 0) partMS[(size_t)s * rpad + row] = make_float2(M, S);
#pragma unroll
  for (int pb = 0; pb < PB; ++pb) {
    if (pb0 + pb < pblocks) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int pcol = 32 * (pb0 + pb) + 8 * (r >> 2) + 4 * h + (r & 3);
        partO[((size_t)s * ppad + pcol) * rpad + row] = O[pb][r];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------







template <bool BF16, int KB, int RI, bool XRES>
static void lse_go(const PassShape& s, const void* Rp, const void* Cp, const float* cbias,
                   float c, float2* part, hipStream_t st) {
  lse_partial_kernel<BF16, KB, RI, XRES><<<s.nrowgroups * s.splits, 256, 0, st>>>(
      (const u32x4*)Rp, (const u32x4*)Cp, cbias, s.rtiles, s.ctiles, s.kbp, s.splits, s.tps, c,
      part, s.rtiles * kTile);
}

template <int MODE, int KB, int RI>
static void lse_pipe_go(const PassShape& s, const void* Rp, const void* Cp, const float* cbias,
                        float c, float2* part, hipStream_t st) {
  lse_pipe_kernel<MODE, KB, RI><<<s.nrowgroups * s.splits, 256, 0, st>>>(
      (const u32x4*)Rp, (const u32x4*)Cp, cbias, s.rtiles, s.ctiles, s.splits, s.tps, c, part,
      s.rtiles * kTile);
}

template <int MODE, int KB, int RI>
static void lse_lds_go(const PassShape& s, const void* Rp, const void* Cp, const float* cbias,
                       float c, float2* part, hipStream_t st) {
  lse_lds_kernel<MODE, KB, RI><<<s.nrowgroups * s.splits, 256, 0, st>>>(
      (const u32x4*)Rp, (const u32x4*)Cp, cbias, s.rtiles, s.ctiles, s.splits, s.tps, c, part,
      s.rtiles * kTile);
}

template <int MODE, int KB>
static void resident_go(const PassShape& s, const void* Rp, const void* Cp, const float* cbias,
                        float c, float2* part, hipStream_t st) {
  if (s.lds) {
    if (s.ri == 2) lse_lds_go<MODE, KB, 2>(s, Rp, Cp, cbias, c, part, st);
    else lse_lds_go<MODE, KB, 1>(s, Rp, Cp, cbias, c, part, st);
  } else {
    if (s.ri == 2) lse_pipe_go<MODE, KB, 2>(s, Rp, Cp, cbias, c, part, st);
    else lse_pipe_go<MODE, KB, 1>(s, Rp, Cp, cbias, c, part, st);
  }
}

static hipError_t lse_split_dispatch(const PassShape& s, const void* Rp, const void* Cp,
                                     const float* cbias, float c, float2* part, hipStream_t st) {
  switch (s.kb) {
    case 3: resident_go<kModeSplit, 3>(s, Rp, Cp, cbias, c, part, st); break;
    case 6: resident_go<kModeSplit, 6>(s, Rp, Cp, cbias, c, part, st); break;
    case 12: resident_go<kModeSplit, 12>(s, Rp, Cp, cbias, c, part, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool BF16>
static hipError_t lse_dispatch(const PassShape& s, const void* Rp, const void* Cp,
                               const float* cbias, float c, float2* part, hipStream_t st) {
  constexpr int kMode = BF16 ? kModeBF16 : kModeF32;
  if (s.xres) {
    switch (s.kb) {
      case 1: resident_go<kMode, 1>(s, Rp, Cp, cbias, c, part, st); break;
      case 2: resident_go<kMode, 2>(s, Rp, Cp, cbias, c, part, st); break;
      case 4: resident_go<kMode, 4>(s, Rp, Cp, cbias, c, part, st); break;
      case 8: resident_go<kMode, 8>(s, Rp, Cp, cbias, c, part, st); break;
      case 16: resident_go<kMode, 16>(s, Rp, Cp, cbias, c, part, st); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (s.ri == 2)
    lse_go<BF16, 8, 2, false>(s, Rp, Cp, cbias, c, part, st);
  else
    lse_go<BF16, 8, 1, false>(s, Rp, Cp, cbias, c, part, st);
  return hipGetLastError();
}

hipError_t launch_lse_partial(const PassShape& s, int mode, const void* Rp, const void* Cp,
                              const float* cbias, float c, float2* part, hipStream_t st) {
  if (mode == kModeSplit) {
    if (!s.xres) return hipErrorInvalidValue;
    return lse_split_dispatch(s, Rp, Cp, cbias, c, part, st);
  }
  return mode == kModeBF16 ? lse_dispatch<true>(s, Rp, Cp, cbias, c, part, st)
                           : lse_dispatch<false>(s, Rp, Cp, cbias, c, part, st);
}




template <bool BF16, int KB, bool XRES, int PB>
static void apply_go(const PassShape& s, int pblocks, const void* Rp, const void* Cp,
                     const float* cbias, const float* Vp, float c, float2* partMS, float* partO,
                     int ppad, hipStream_t st) {
  dim3 grid(s.nrowgroups * s.splits, (pblocks + PB - 1) / PB);
  apply_partial_kernel<BF16, KB, XRES, PB><<<grid, 256, 0, st>>>(
      (const u32x4*)Rp, (const u32x4*)Cp, cbias, (const f32x4*)Vp, s.rtiles, s.ctiles, s.kbp,
      s.splits, s.tps, c, pblocks, partMS, partO, s.rtiles * kTile, ppad);
}

template <bool BF16, int PB>
static hipError_t apply_dispatch_kb(const PassShape& s, int pblocks, const void* Rp,
                                    const void* Cp, const float* cbias, const float* Vp, float c,
                                    float2* partMS, float* partO, int ppad, hipStream_t st) {
  if (!s.xres) {
    apply_go<BF16, 8, false, PB>(s, pblocks, Rp, Cp, cbias, Vp, c, partMS, partO, ppad, st);
    return hipGetLastError();
  }
  switch (s.kb) {
    case 1: apply_go<BF16, 1, true, PB>(s, pblocks, Rp, Cp, cbias, Vp, c, partMS, partO, ppad, st); break;
    case 2: apply_go<BF16, 2, true, PB>(s, pblocks, Rp, Cp, cbias, Vp, c, partMS, partO, ppad, st); break;
    case 4: apply_go<BF16, 4, true, PB>(s, pblocks, Rp, Cp, cbias, Vp, c, partMS, partO, ppad, st); break;
    case 8: apply_go<BF16, 8, true, PB>(s, pblocks, Rp, Cp, cbias, Vp, c, partMS, partO, ppad, st); break;
    case 16: apply_go<BF16, 16, true, PB>(s, pblocks, Rp, Cp, cbias, Vp, c, partMS, partO, ppad, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool BF16>
static hipError_t apply_dispatch(const PassShape& s, int pblocks, int pb_per_pass, const void* Rp,
                                 const void* Cp, const float* cbias, const float* Vp, float c,
                                 float2* partMS, float* partO, int ppad, hipStream_t st) {
  switch (pb_per_pass) {
    case 1: return apply_dispatch_kb<BF16, 1>(s, pblocks, Rp, Cp, cbias, Vp, c, partMS, partO, ppad, st);
    case 2: return apply_dispatch_kb<BF16, 2>(s, pblocks, Rp, Cp, cbias, Vp, c, partMS, partO, ppad, st);
    case 4: return apply_dispatch_kb<BF16, 4>(s, pblocks, Rp, Cp, cbias, Vp, c, partMS, partO, ppad, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_apply_partial(const PassShape& s, int bf16, int pblocks, int pb_per_pass,
                                const void* Rp, const void* Cp, const float* cbias,
                                const float* Vp, float c, float2* partMS, float* partO, int ppad,
                                hipStream_t st) {
  return bf16 ? apply_dispatch<true>(s, pblocks, pb_per_pass, Rp, Cp, cbias, Vp, c, partMS, partO,
                                     ppad, st)
              : apply_dispatch<false>(s, pblocks, pb_per_pass, Rp, Cp, cbias, Vp, c, partMS,
                                      partO, ppad, st);
}


}  // namespace flashot
