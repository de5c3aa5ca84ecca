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
      part[(size_t)s * rpad + (size_t)(rt0 + ri) * kTile + (lane & 31)] = make_float2(Mt, St);
  }
}

// ---------------------------------------------------------------------------
// Software-pipelined variant of the register-resident pass. Each wave keeps
// two score tiles in flight: while the matrix cores form the scores of column
// tile t+1, the vector unit runs the online LSE of tile t, so one wave keeps
// both units busy. The column operand alternates between two register
// buffers (the loop body is written twice with the roles swapped), so a
// prefetched tile is never copied between registers.
// ---------------------------------------------------------------------------
template <bool BF16, int KB, int RI>
__device__ __forceinline__ void score_tile(const u32x4 (&y)[KB], const u32x4 (&xr)[RI][KB],
                                           float wv, int h, f32x16 (&acc)[RI]) {
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) acc[ri] = f32x16{};
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int ri = 0; ri < RI; ++ri) acc[ri] = mfma_kblock<BF16>(y[kb], xr[ri][kb], acc[ri]);
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) acc[ri] = mfma_bias(wv, h, acc[ri]);
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
template <bool BF16, int KB, int RI>
__device__ __forceinline__ void stage_schedule() {
  constexpr int kMfma = RI * (KB * (BF16 ? 1 : 4) + 1);
  constexpr int kValu = RI * 62;  // online LSE of RI score tiles
  constexpr int kValuPer = (kValu + kMfma - 1) / kMfma;
#pragma unroll
  for (int i = 0; i < kMfma; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, kValuPer, 0);  // VALU
  }
  __builtin_amdgcn_sched_group_barrier(0x020, KB + 1, 0);      // VMEM reads
}

template <bool BF16, int KB, int RI>
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
    M[ri] = -1.0e30f;
    S[ri] = 0.f;
  }

  // Invariant at the top of the loop: accA holds the scores of tile k, yB
  // holds (or is loading) tile k+1 and yA tile k+2; indices past the split's
  // last tile are clamped to it (loaded, never reduced).
  u32x4 yA[KB], yB[KB];
  float wA, wB;
  f32x16 accA[RI], accB[RI];
  load_ctile<KB>(Cp, cbias, jt0, lane, yA, wA);
  load_ctile<KB>(Cp, cbias, jt0 + min(1, last), lane, yB, wB);
  score_tile<BF16, KB, RI>(yA, xr, wA, h, accA);
  load_ctile<KB>(Cp, cbias, jt0 + min(2, last), lane, yA, wA);
  int k = 0;
  for (; k + 2 <= last; k += 2) {
    score_tile<BF16, KB, RI>(yB, xr, wB, h, accB);
#pragma unroll
    for (int ri = 0; ri < RI; ++ri) lse_tile(accA[ri], M[ri], S[ri], c);
    load_ctile<KB>(Cp, cbias, jt0 + min(k + 3, last), lane, yB, wB);
    stage_schedule<BF16, KB, RI>();
    __builtin_amdgcn_sched_barrier(0);
    score_tile<BF16, KB, RI>(yA, xr, wA, h, accA);
#pragma unroll
    for (int ri = 0; ri < RI; ++ri) lse_tile(accB[ri], M[ri], S[ri], c);
    load_ctile<KB>(Cp, cbias, jt0 + min(k + 4, last), lane, yA, wA);
    stage_schedule<BF16, KB, RI>();
    __builtin_amdgcn_sched_barrier(0);
  }
  if (k + 1 <= last) {  // tiles k and k+1 remain
    score_tile<BF16, KB, RI>(yB, xr, wB, h, accB);
#pragma unroll
    for (int ri = 0; ri < RI; ++ri) lse_tile(accA[ri], M[ri], S[ri], c);
#pragma unroll
    for (int ri = 0; ri < RI; ++ri) lse_tile(accB[ri], M[ri], S[ri], c);
  } else {  // tile k remains
#pragma unroll
    for (int ri = 0; ri < RI; ++ri) lse_tile(accA[ri], M[ri], S[ri], c);
  }

#pragma unroll
  for (int ri = 0; ri < RI; ++ri) {
    const float Mp = __shfl_xor(M[ri], 32);
    const float Sp = __shfl_xor(S[ri], 32);
    const float Mt = fmaxf(M[ri], Mp);
    const float cm = c * Mt;
    const float St = S[ri] * __builtin_amdgcn_exp2f(fmaf(c, M[ri], -cm)) +
                     Sp * __builtin_amdgcn_exp2f(fmaf(c, Mp, -cm));
    if (h == 0 && rt0 + ri < rtiles)
      part[(size_t)s * rpad + (size_t)(rt0 + ri) * kTile + (lane & 31)] = make_float2(Mt, St);
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

template <bool BF16, int KB, int RI>
static void lse_pipe_go(const PassShape& s, const void* Rp, const void* Cp, const float* cbias,
                        float c, float2* part, hipStream_t st) {
  lse_pipe_kernel<BF16, KB, RI><<<s.nrowgroups * s.splits, 256, 0, st>>>(
      (const u32x4*)Rp, (const u32x4*)Cp, cbias, s.rtiles, s.ctiles, s.splits, s.tps, c, part,
      s.rtiles * kTile);
}

static int lse_variant() {
  static int v = [] {
    const char* e = getenv("FLASHOT_LSE_V");
    return (e && *e) ? atoi(e) : 2;
  }();
  return v;
}

template <bool BF16>
static hipError_t lse_dispatch(const PassShape& s, const void* Rp, const void* Cp,
                               const float* cbias, float c, float2* part, hipStream_t st) {
  if (s.xres && lse_variant() == 2) {
#define FLASHOT_PIPE_CASE(KBV)                                      \
  case KBV:                                                         \
    if (s.ri == 2)                                                  \
      lse_pipe_go<BF16, KBV, 2>(s, Rp, Cp, cbias, c, part, st);     \
    else                                                            \
      lse_pipe_go<BF16, KBV, 1>(s, Rp, Cp, cbias, c, part, st);     \
    break;
    switch (s.kb) {
      FLASHOT_PIPE_CASE(1)
      FLASHOT_PIPE_CASE(2)
      FLASHOT_PIPE_CASE(4)
      FLASHOT_PIPE_CASE(8)
      FLASHOT_PIPE_CASE(16)
      default:
        return hipErrorInvalidValue;
    }
#undef FLASHOT_PIPE_CASE
    return hipGetLastError();
  }
  if (!s.xres) {
    if (s.ri == 2)
      lse_go<BF16, 8, 2, false>(s, Rp, Cp, cbias, c, part, st);
    else
      lse_go<BF16, 8, 1, false>(s, Rp, Cp, cbias, c, part, st);
    return hipGetLastError();
  }
#define FLASHOT_LSE_CASE(KBV)                                  \
  case KBV:                                                    \
    if (s.ri == 2)                                             \
      lse_go<BF16, KBV, 2, true>(s, Rp, Cp, cbias, c, part, st); \
    else                                                       \
      lse_go<BF16, KBV, 1, true>(s, Rp, Cp, cbias, c, part, st); \
    break;
  switch (s.kb) {
    FLASHOT_LSE_CASE(1)
    FLASHOT_LSE_CASE(2)
    FLASHOT_LSE_CASE(4)
    FLASHOT_LSE_CASE(8)
    FLASHOT_LSE_CASE(16)
    default:
      return hipErrorInvalidValue;
  }
#undef FLASHOT_LSE_CASE
  return hipGetLastError();
}

hipError_t launch_lse_partial(const PassShape& s, int bf16, const void* Rp, const void* Cp,
                              const float* cbias, float c, float2* part, hipStream_t st) {
  return bf16 ? lse_dispatch<true>(s, Rp, Cp, cbias, c, part, st)
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
