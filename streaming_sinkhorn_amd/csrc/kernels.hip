// Register-resident streamed log-sum-exp passes of the Sinkhorn solver
// (the hot kernels for d up to 128 fp32 / 256 bf16).
//
// Method: "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU"
// (arXiv 2602.03067). A Sinkhorn half-step is a row-wise log-sum-exp of the
// biased dot-product score 2 x_i.y_j/eps + bias_j (Prop. 1, App. D.1); it is
// streamed over column tiles with a running stabiliser and rescaled sum
// (App. D.3) and only the potentials are written back (App. D.2, G.1); the row
// block stays on chip for the whole sweep (App. G.2 row-stationary order).
//
// MI355X design (not the page's Triton/A100 one):
//  * the score tile is formed on the matrix cores with a 32x32 output per
//    wave, computed TRANSPOSED (columns j on the M axis, rows i on the N
//    axis). In the 32x32 accumulator layout lane l then holds 16 values of
//    ONE output row (i = l % 32), so the online LSE is lane-local: no
//    cross-lane traffic inside the column loop, one exchange with lane
//    l ^ 32 at the very end;
//  * one extra bf16 MFMA adds the per-column bias and subtracts the row's
//    running stabiliser, both as three exact bf16 parts (the column side's
//    parts are written next to the biases; the row side's are rebuilt only
//    when the stabiliser moves), so the common-case score costs one exp2
//    and one add on the vector unit;
//  * fp32 points are formed on the fp16 matrix cores from two fp16 parts per
//    value (device_common.h), on request on the bf16 matrix cores from three
//    bf16 parts or with fp32 MFMA; bf16 points directly;
//  * operands are pre-packed once per call into the exact register layout of
//    the MFMA (16 contiguous bytes per lane, zero-padded tiles), so every
//    load in the hot loop is a full 1 KiB coalesced wave load with no masks;
//  * each wave keeps two score tiles in flight (matrix work of tile t+1
//    interleaved with the exponentials of tile t); wide fp32 tiles are shared
//    by the workgroup's waves through LDS;
//  * the streamed axis is split over workgroups when the output axis alone
//    cannot fill 256 CUs; partial (stabiliser, sum) pairs are merged
//    afterwards in a fixed order with the exact merge of App. D.3, so results
//    are deterministic. In the per-wave pass, when the split count is a
//    multiple of 4, the workgroups' (split, row group) pairs are laid over
//    the 8 XCDs as a 2 x 4 grid (pipe_block below), so each XCD's L2 serves
//    half of the rows and a quarter of the columns; the LDS-shared pass keeps
//    the split index fastest in the workgroup index.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device_common.h"

namespace flashot {

template <int MODE, int KB>
__device__ __forceinline__ void load_ctile(const u32x4* __restrict__ Cp,
                                           const float* __restrict__ cbias,
                                           const uint2* __restrict__ cb3, int jt, int lane,
                                           u32x4 (&y)[KB], BiasOp<MODE>& ab) {
  ab = load_bias<MODE>(cbias, cb3, jt, lane);
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) y[kb] = Cp[((size_t)jt * KB + kb) * 64 + lane];
}

// Orders one pipeline stage (one scheduling region): one matrix instruction
// alternating with a few vector instructions, then the loads that refill the
// column buffer the matrix instructions have just read.
template <int MODE, int KB, int RI>
__device__ __forceinline__ void stage_schedule() {
  constexpr int kMfma = RI * (tile_mfmas<MODE, KB>() + 1);
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
// VEC (transport-vector pass): vN receives the values of the tile scored in
// this stage (jt_vals), vC holds those of the tile reduced now, and T
// carries sum exp2(score - M) v next to S.
template <int MODE, int KB, int RI, bool VEC>
__device__ __forceinline__ void pipe_stage(const u32x4* __restrict__ Cp,
                                           const float* __restrict__ cbias,
                                           const uint2* __restrict__ cb3,
                                           const float* __restrict__ vcol, int jt_refill,
                                           int jt_vals, int lane, int h, float ks,
                                           const u32x4 (&xr)[RI][KB], u32x4 (&yN)[KB],
                                           BiasOp<MODE>& aN,
                                           f32x16 (&accN)[RI], float (&MfN)[RI],
                                           const f32x16 (&accC)[RI], const float (&MfC)[RI],
                                           f32x16& vN, const f32x16& vC, float (&M)[RI],
                                           float (&S)[RI], float (&T)[RI], float (&Mfc)[RI],
                                           BiasOp<MODE> (&Bst)[RI]) {
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) MfN[ri] = Mfc[ri];
  score_tile<MODE, KB, RI>(yN, xr, aN, Bst, h, accN);
  // The fast-path sums are taken unconditionally (the rare exact path restores
  // the old ones): no row's work becomes conditional on another's, so the
  // stage stays one scheduling region in which the exponentials of tile k
  // interleave with the matrix work of tile k+1.
  float So[RI], To[RI];
  int slow = 0;
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) {
    So[ri] = S[ri];
    if constexpr (VEC) {
      To[ri] = T[ri];
      slow |= lse_fast_v<MODE != kModeBF16, lazy_lse<MODE, KB>()>(accC[ri], vC, MfC[ri], M[ri], So[ri], To[ri], ks,
                                            S[ri], T[ri]);
    } else {
      slow |= lse_fast<MODE != kModeBF16, lazy_lse<MODE, KB>()>(accC[ri], MfC[ri], M[ri], So[ri], ks, S[ri]);
    }
  }
  load_ctile<MODE, KB>(Cp, cbias, cb3, jt_refill, lane, yN, aN);
  if constexpr (VEC) vN = load_tile_values(vcol, jt_vals, h);
  stage_schedule<MODE, KB, RI>();
  __builtin_amdgcn_sched_barrier(0);
  if (__builtin_amdgcn_ballot_w64(slow) != 0) {
#pragma unroll
    for (int ri = 0; ri < RI; ++ri) {
      S[ri] = So[ri];
      if constexpr (VEC) {
        T[ri] = To[ri];
        lse_exact_v<lazy_lse<MODE, KB>()>(accC[ri], vC, MfC[ri], M[ri], S[ri], T[ri], ks);
      } else {
        lse_exact<lazy_lse<MODE, KB>()>(accC[ri], MfC[ri], M[ri], S[ri], ks);
      }
    }
    refold<MODE, RI>(M, h, Mfc, Bst);
  }
}

// Tail LSE of RI tiles (plain or transport-vector).
template <int MODE, int KB, int RI, bool VEC>
__device__ __forceinline__ void tail_any(const f32x16 (&acc)[RI], const f32x16& v,
                                         const float (&Mf)[RI], float (&M)[RI], float (&S)[RI],
                                         float (&T)[RI], float ks) {
  if constexpr (VEC) lse_tail_v<MODE, RI, lazy_lse<MODE, KB>()>(acc, v, Mf, M, S, T, ks);
  else lse_tail<MODE, RI, lazy_lse<MODE, KB>()>(acc, Mf, M, S, ks);
}

// Partials of a row: (M in log2 units, S + S'), and T + T' for VEC.
template <int RI, bool VEC>
__device__ __forceinline__ void write_partials(const float (&M)[RI], const float (&S)[RI],
                                               const float (&T)[RI], int h, int lane, int rt0,
                                               int rtiles, int s, int rpad, float ks,
                                               float2* __restrict__ part,
                                               float* __restrict__ partT) {
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) {
    const float St = S[ri] + __shfl_xor(S[ri], 32);
    float Tt = 0.f;
    if constexpr (VEC) Tt = T[ri] + __shfl_xor(T[ri], 32);
    if (h == 0 && rt0 + ri < rtiles) {
      const size_t at = (size_t)s * rpad + (size_t)(rt0 + ri) * kTile + (lane & 31);
      part[at] = make_float2(ks * M[ri], St);
      if constexpr (VEC) partT[at] = Tt;
    }
  }
}

// One wave's sweep over column tiles jt0 .. jt0 + last (last >= 0) for its
// RI row tiles from rt0 (indices past the operand are clamped; their rows
// are never written): running (M, S[, T]) per lane, the lane pair l, l ^ 32
// sharing M and holding halves of the row's sums.
template <int MODE, int KB, int RI, bool VEC>
__device__ __forceinline__ void pipe_sweep(const u32x4* __restrict__ Rp, const u32x4* __restrict__ Cp,
                                           const float* __restrict__ cbias,
                                           const float* __restrict__ vcol, int rt0, int rtiles,
                                           int ctiles, int jt0, int last, int lane, float ks,
                                           float (&M)[RI], float (&S)[RI], float (&T)[RI]) {
  const int h = lane >> 5;
  const uint2* __restrict__ cb3 = bias_parts(cbias, ctiles * kTile);
  u32x4 xr[RI][KB];
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) {
    const int rt = min(rt0 + ri, rtiles - 1);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) xr[ri][kb] = Rp[((size_t)rt * KB + kb) * 64 + lane];
  }
  float Mfc[RI];
  BiasOp<MODE> Bst[RI];
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) {
    M[ri] = kUnset;
    S[ri] = 0.f;
    T[ri] = 0.f;
  }
  refold<MODE, RI>(M, h, Mfc, Bst);

  // Invariant at the top of the loop: accA holds the scores of tile k (with
  // MfA folded in), yB holds (or is loading) tile k+1 and yA tile k+2;
  // indices past the split's last tile are clamped to it (loaded, never
  // reduced).
  u32x4 yA[KB], yB[KB];
  BiasOp<MODE> aA, aB;
  f32x16 accA[RI], accB[RI], vA{}, vB{};
  float MfA[RI], MfB[RI];
  load_ctile<MODE, KB>(Cp, cbias, cb3, jt0, lane, yA, aA);
  load_ctile<MODE, KB>(Cp, cbias, cb3, jt0 + min(1, last), lane, yB, aB);
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) MfA[ri] = Mfc[ri];
  score_tile<MODE, KB, RI>(yA, xr, aA, Bst, h, accA);
  if constexpr (VEC) vA = load_tile_values(vcol, jt0, h);
  load_ctile<MODE, KB>(Cp, cbias, cb3, jt0 + min(2, last), lane, yA, aA);
  int k = 0;
  for (; k + 2 <= last; k += 2) {
    pipe_stage<MODE, KB, RI, VEC>(Cp, cbias, cb3, vcol, jt0 + min(k + 3, last), jt0 + k + 1, lane, h,
                                  ks, xr, yB, aB, accB, MfB, accA, MfA, vB, vA, M, S, T, Mfc, Bst);
    pipe_stage<MODE, KB, RI, VEC>(Cp, cbias, cb3, vcol, jt0 + min(k + 4, last), jt0 + k + 2, lane, h,
                                  ks, xr, yA, aA, accA, MfA, accB, MfB, vA, vB, M, S, T, Mfc, Bst);
  }
  if (k + 1 <= last) {  // tiles k and k+1 remain
    tail_any<MODE, KB, RI, VEC>(accA, vA, MfA, M, S, T, ks);
    refold<MODE, RI>(M, h, Mfc, Bst);
#pragma unroll
    for (int ri = 0; ri < RI; ++ri) MfB[ri] = Mfc[ri];
    score_tile<MODE, KB, RI>(yB, xr, aB, Bst, h, accB);
    if constexpr (VEC) vB = load_tile_values(vcol, jt0 + k + 1, h);
    tail_any<MODE, KB, RI, VEC>(accB, vB, MfB, M, S, T, ks);
  } else {  // tile k remains
    tail_any<MODE, KB, RI, VEC>(accA, vA, MfA, M, S, T, ks);
  }
}

// Workgroup -> (column split, row group) of the per-wave resident pass
// (lse_pipe_kernel; the LDS-shared pass measured 1 % slower with it and keeps
// the split index fastest). Workgroups
// go to the 8 XCDs round robin (workgroup w on XCD w % 8), each XCD with its
// own L2. When the split count is a multiple of 4 the XCDs form a 2 x 4
// grid: XCD x takes the row
// groups of half x / 4 and the splits of quarter x % 4, so it reads half of
// the row operand and a quarter of the column operand from memory, not all
// rows and a split's share of the columns (about two thirds of the HBM / MALL
// fetch at a square problem). The grid then holds an even number of row
// groups (the padding one exits at once). Other split counts keep the split
// index fastest.
__host__ __device__ inline int pipe_rowgroups(int nrowgroups, int splits) {
  return splits % 4 == 0 ? (nrowgroups + 1) / 2 * 2 : nrowgroups;
}
__device__ __forceinline__ void pipe_block(int bid, int splits, int nrgp, int& s, int& rg) {
  if (splits % 4 == 0) {
    const int xcd = bid & 7, li = bid >> 3;
    const int sq = splits >> 2;
    s = (xcd & 3) * sq + li % sq;
    rg = (xcd >> 2) * (nrgp >> 1) + li / sq;
  } else {
    s = bid % splits;
    rg = bid / splits;
  }
}

template <int MODE, int KB, int RI, bool VEC>
__global__ __launch_bounds__(256) void lse_pipe_kernel(
    const u32x4* __restrict__ Rp, const u32x4* __restrict__ Cp, const float* __restrict__ cbias,
    const float* __restrict__ vcol, int rtiles, int ctiles, int splits, int tps, float c,
    float2* __restrict__ part, float* __restrict__ partT, int rpad) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int s, rg;
  pipe_block(blockIdx.x, splits, gridDim.x / splits, s, rg);
  const int rt0 = (rg * kWaves + wave) * RI;
  if (rt0 >= rtiles) return;
  const int jt0 = s * tps;
  const int last = min(jt0 + tps, ctiles) - 1 - jt0;  // split holds tiles 0..last, last >= 0
  const float ks = MODE == kModeBF16 ? c : 1.0f;
  float M[RI], S[RI], T[RI];
  pipe_sweep<MODE, KB, RI, VEC>(Rp, Cp, cbias, vcol, rt0, rtiles, ctiles, jt0, last, lane, ks, M, S, T);
  // The lane pair shares M: the row's partial is (M in log2 units, S + S').
  write_partials<RI, VEC>(M, S, T, lane >> 5, lane, rt0, rtiles, s, rpad, ks, part, partT);
}

// Single-launch half-step of a small problem. A workgroup of W waves owns
// one 32-row tile; wave w sweeps column tiles [w tpw, (w + 1) tpw) and leaves
// the rows' (M in log2 units, S) in LDS; wave 0 merges the W pairs of each
// row in wave order with the exact merge (App. D.3) and ends the half-step
// (potential, next bias, marginal-error term) in the same launch, with the
// row's inputs loaded before the sweep. A problem too small to fill the chip
// is bound by launches and the latency of their dependent steps: this removes
// the separate merge launch and its global partials, with no
// cross-workgroup synchronisation.
template <int MODE, int KB, int W>
__global__ __launch_bounds__(W * 64) void lse_solo_kernel(
    const u32x4* __restrict__ Rp, const u32x4* __restrict__ Cp, const float* __restrict__ cbias,
    int rtiles, int ctiles, int tpw, float c, RowFinish fin, float* __restrict__ err_part) {
  __shared__ float2 ms[W][kTile];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rt = blockIdx.x;
  const int i = rt * kTile + lane;
  const bool owner = wave == 0 && lane < kTile && i < fin.rows;
  RowIn in{};
  if (owner) in = load_row_in(fin, i);
  const int jt0 = wave * tpw;
  const float ks = MODE == kModeBF16 ? c : 1.0f;
  float M[1] = {kUnset}, S[1] = {0.f}, T[1] = {0.f};
  if (jt0 < ctiles)  // waves past the last column tile contribute (M unset, S = 0)
    pipe_sweep<MODE, KB, 1, false>(Rp, Cp, cbias, nullptr, rt, rtiles, ctiles, jt0,
                                   min(jt0 + tpw, ctiles) - 1 - jt0, lane, ks, M, S, T);
  const float St = S[0] + __shfl_xor(S[0], 32);
  if (lane < kTile) ms[wave][lane] = make_float2(ks * M[0], St);
  __syncthreads();
  if (wave != 0) return;
  float Mm = -3.0e38f, Sm = 0.f;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const float2 ps = ms[w][lane & 31];
    if (ps.x > Mm) {
      Sm = fmaf(Sm, exp2f(Mm - ps.x), ps.y);
      Mm = ps.x;
    } else {
      Sm = fmaf(ps.y, exp2f(ps.x - Mm), Sm);
    }
  }
  float e = 0.f;
  if (owner) e = finish_row(fin, i, Mm, Sm, in);
  else if (lane < kTile) finish_pad_row(fin, i);
  if (fin.with_err) {
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) e += __shfl_xor(e, o);
    if (lane == 0) err_part[rt] = e;
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
                                               const u32x4 (&xr)[RI][KB], BiasOp<MODE> ab,
                                               const BiasOp<MODE> (&Bst)[RI], int h,
                                               f32x16 (&acc)[RI]) {
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) acc[ri] = bias_start<MODE>(ab, Bst[ri]);
  if constexpr (MODE == kModeSplit) {
#pragma unroll
    for (int kb = 0; kb < KB; kb += 3) {
      u32x4 y[3];
#pragma unroll
      for (int q = 0; q < 3; ++q) y[q] = buf[(kb + q) * 64 + lane];
#pragma unroll
      for (int ri = 0; ri < RI; ++ri) acc[ri] = mfma_split(y, &xr[ri][kb], acc[ri]);
    }
  } else if constexpr (MODE == kModeHalf2) {
#pragma unroll
    for (int kb = 0; kb < KB; kb += 2) {
      u32x4 y[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) y[q] = buf[(kb + q) * 64 + lane];
#pragma unroll
      for (int ri = 0; ri < RI; ++ri) acc[ri] = mfma_half2(y, &xr[ri][kb], acc[ri]);
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
  for (int ri = 0; ri < RI; ++ri) acc[ri] = bias_finish<MODE>(ab, Bst[ri], h, acc[ri]);
}

template <int MODE, int KB, int RI>
__device__ __forceinline__ void stage_schedule_lds() {
  constexpr int kMfma = RI * (tile_mfmas<MODE, KB>() + 1);
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

template <int MODE, int KB, int RI, bool VEC>
__global__ __launch_bounds__(256) void lse_lds_kernel(
    const u32x4* __restrict__ Rp, const u32x4* __restrict__ Cp, const float* __restrict__ cbias,
    const float* __restrict__ vcol, int rtiles, int ctiles, int splits, int tps, float c,
    float2* __restrict__ part, float* __restrict__ partT, int rpad) {
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
  const uint2* __restrict__ cb3 = bias_parts(cbias, ctiles * kTile);

  u32x4 xr[RI][KB];
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) {
    const int rt = min(rt0 + ri, rtiles - 1);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) xr[ri][kb] = Rp[((size_t)rt * KB + kb) * 64 + lane];
  }
  float M[RI], S[RI], T[RI], Mfc[RI];
  BiasOp<MODE> Bst[RI];
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) {
    M[ri] = kUnset;
    S[ri] = 0.f;
    T[ri] = 0.f;
  }
  refold<MODE, RI>(M, h, Mfc, Bst);

  u32x4 g[kLoads];
  stage_load<KB>(Cp, jt0, tid, g);
  stage_store<KB>(lds[0], tid, g);
  stage_load<KB>(Cp, jt0 + min(1, last), tid, g);
  stage_store<KB>(lds[1], tid, g);
  BiasOp<MODE> aA = load_bias<MODE>(cbias, cb3, jt0, lane);
  BiasOp<MODE> aB = load_bias<MODE>(cbias, cb3, jt0 + min(1, last), lane);
  __syncthreads();

  // Invariant at stage k: accA / accB alternate holding the scores of tile k;
  // LDS buffer (k + 1) & 1 holds tile k+1; buffer k & 1 is free once every
  // wave has passed the stage barrier.
  f32x16 accA[RI], accB[RI], vA{}, vB{};
  float MfA[RI], MfB[RI];
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) MfA[ri] = Mfc[ri];
  score_tile_lds<MODE, KB, RI>(lds[0], lane, xr, aA, Bst, h, accA);
  if constexpr (VEC) vA = load_tile_values(vcol, jt0, h);

  auto stage = [&](int k, f32x16(&accN)[RI], float(&MfN)[RI], BiasOp<MODE>& aN,
                   const f32x16(&accC)[RI], const float(&MfC)[RI], BiasOp<MODE>& aC, f32x16& vN,
                   const f32x16& vC) {
    __syncthreads();  // tile k+1 is in LDS; every wave is done reading tile k's buffer
    const int jt2 = jt0 + min(k + 2, last);
    stage_load<KB>(Cp, jt2, tid, g);
    const BiasOp<MODE> a2 = load_bias<MODE>(cbias, cb3, jt2, lane);
#pragma unroll
    for (int ri = 0; ri < RI; ++ri) MfN[ri] = Mfc[ri];
    score_tile_lds<MODE, KB, RI>(lds[(k + 1) & 1], lane, xr, aN, Bst, h, accN);
    // fast-path sums taken unconditionally (see pipe_stage)
    float So[RI], To[RI];
    int slow = 0;
#pragma unroll
    for (int ri = 0; ri < RI; ++ri) {
      So[ri] = S[ri];
      if constexpr (VEC) {
        To[ri] = T[ri];
        slow |= lse_fast_v<MODE != kModeBF16, lazy_lse<MODE, KB>()>(accC[ri], vC, MfC[ri], M[ri], So[ri], To[ri], ks,
                                              S[ri], T[ri]);
      } else {
        slow |= lse_fast<MODE != kModeBF16, lazy_lse<MODE, KB>()>(accC[ri], MfC[ri], M[ri], So[ri], ks, S[ri]);
      }
    }
    if constexpr (VEC) vN = load_tile_values(vcol, jt0 + k + 1, h);
    stage_store<KB>(lds[k & 1], tid, g);
    aC = a2;  // the buffer of tile k now receives tile k+2
    stage_schedule_lds<MODE, KB, RI>();
    __builtin_amdgcn_sched_barrier(0);
    if (__builtin_amdgcn_ballot_w64(slow) != 0) {
#pragma unroll
      for (int ri = 0; ri < RI; ++ri) {
        S[ri] = So[ri];
        if constexpr (VEC) {
          T[ri] = To[ri];
          lse_exact_v<lazy_lse<MODE, KB>()>(accC[ri], vC, MfC[ri], M[ri], S[ri], T[ri], ks);
        } else {
          lse_exact<lazy_lse<MODE, KB>()>(accC[ri], MfC[ri], M[ri], S[ri], ks);
        }
      }
      refold<MODE, RI>(M, h, Mfc, Bst);
    }
  };

  int k = 0;
  for (; k + 2 <= last; k += 2) {
    stage(k, accB, MfB, aB, accA, MfA, aA, vB, vA);
    stage(k + 1, accA, MfA, aA, accB, MfB, aB, vA, vB);
  }
  if (k + 1 <= last) {  // tiles k and k+1 remain; tile k+1 is in buffer (k+1)&1
    __syncthreads();
#pragma unroll
    for (int ri = 0; ri < RI; ++ri) MfB[ri] = Mfc[ri];  // M has not moved since the last refold
    score_tile_lds<MODE, KB, RI>(lds[(k + 1) & 1], lane, xr, aB, Bst, h, accB);
    if constexpr (VEC) vB = load_tile_values(vcol, jt0 + k + 1, h);
    tail_any<MODE, KB, RI, VEC>(accA, vA, MfA, M, S, T, ks);
    tail_any<MODE, KB, RI, VEC>(accB, vB, MfB, M, S, T, ks);
  } else {
    tail_any<MODE, KB, RI, VEC>(accA, vA, MfA, M, S, T, ks);
  }

  write_partials<RI, VEC>(M, S, T, h, lane, rt0, rtiles, s, rpad, ks, part, partT);
}

// ---------------------------------------------------------------------------
// Launchers of the register-resident passes.
// ---------------------------------------------------------------------------
// Arguments shared by every resident launch; vcol / partT are used by the
// transport-vector instantiations only.
struct ResArgs {
  const void* Rp;
  const void* Cp;
  const float* cbias;
  const float* vcol;
  float c;
  float2* part;
  float* partT;
  const LaunchTimer* timer;  // null: plain launch
};

template <int MODE, int KB, int RI, bool VEC>
static void lse_pipe_go(const PassShape& s, const ResArgs& a, hipStream_t st) {
  launch_timed(lse_pipe_kernel<MODE, KB, RI, VEC>,
               dim3(pipe_rowgroups(s.nrowgroups, s.splits) * s.splits), dim3(256), st, a.timer,
               (const u32x4*)a.Rp, (const u32x4*)a.Cp, a.cbias, a.vcol, s.rtiles, s.ctiles,
               s.splits, s.tps, a.c, a.part, a.partT, s.rtiles * kTile);
}

template <int MODE, int KB, int RI, bool VEC>
static void lse_lds_go(const PassShape& s, const ResArgs& a, hipStream_t st) {
  launch_timed(lse_lds_kernel<MODE, KB, RI, VEC>, dim3(s.nrowgroups * s.splits), dim3(256), st,
               a.timer, (const u32x4*)a.Rp, (const u32x4*)a.Cp, a.cbias, a.vcol, s.rtiles,
               s.ctiles, s.splits, s.tps, a.c, a.part, a.partT, s.rtiles * kTile);
}

template <int MODE, int KB, bool VEC>
static void resident_go(const PassShape& s, const ResArgs& a, hipStream_t st) {
  if (s.lds) {
    if (s.ri == 2) lse_lds_go<MODE, KB, 2, VEC>(s, a, st);
    else lse_lds_go<MODE, KB, 1, VEC>(s, a, st);
  } else {
    if (s.ri == 2) lse_pipe_go<MODE, KB, 2, VEC>(s, a, st);
    else lse_pipe_go<MODE, KB, 1, VEC>(s, a, st);
  }
}

template <bool VEC>
static hipError_t lse_split_dispatch(const PassShape& s, const ResArgs& a, hipStream_t st) {
  switch (s.kb) {
    case 3: resident_go<kModeSplit, 3, VEC>(s, a, st); break;
    case 6: resident_go<kModeSplit, 6, VEC>(s, a, st); break;
    case 12: resident_go<kModeSplit, 12, VEC>(s, a, st); break;
    case 24:  // 64 < d <= 128: one resident row tile per wave, columns through LDS
      if (!s.lds || s.ri != 1) return hipErrorInvalidValue;
      lse_lds_go<kModeSplit, 24, 1, VEC>(s, a, st);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Two fp16 parts per k-block: 2, 4, 8 units for d <= 64, 16 for
// 64 < d <= 128 (columns through LDS; 32 KiB of row operand per wave).
template <bool VEC>
static hipError_t lse_half2_dispatch(const PassShape& s, const ResArgs& a, hipStream_t st) {
  switch (s.kb) {
    case 2: resident_go<kModeHalf2, 2, VEC>(s, a, st); break;
    case 4: resident_go<kModeHalf2, 4, VEC>(s, a, st); break;
    case 8: resident_go<kModeHalf2, 8, VEC>(s, a, st); break;
    case 16:
      if (!s.lds) return hipErrorInvalidValue;
      if (s.ri == 2) lse_lds_go<kModeHalf2, 16, 2, VEC>(s, a, st);
      else lse_lds_go<kModeHalf2, 16, 1, VEC>(s, a, st);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int MODE, bool VEC>
static hipError_t lse_resident_dispatch(const PassShape& s, const ResArgs& a, hipStream_t st) {
  switch (s.kb) {
    case 1: resident_go<MODE, 1, VEC>(s, a, st); break;
    case 2: resident_go<MODE, 2, VEC>(s, a, st); break;
    case 4: resident_go<MODE, 4, VEC>(s, a, st); break;
    case 8: resident_go<MODE, 8, VEC>(s, a, st); break;
    case 16: resident_go<MODE, 16, VEC>(s, a, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int MODE, int KB>
static void lse_solo_go(const PassShape& s, const void* Rp, const void* Cp, const float* cbias,
                        float c, const RowFinish& fin, float* err_part, hipStream_t st,
                        const LaunchTimer* t) {
  constexpr int W = kSoloWaves;
  const int tpw = (s.ctiles + W - 1) / W;
  launch_timed(lse_solo_kernel<MODE, KB, W>, dim3(s.rtiles), dim3(W * 64), st, t,
               (const u32x4*)Rp, (const u32x4*)Cp, cbias, s.rtiles, s.ctiles, tpw, c, fin,
               err_part);
}

bool lse_solo_supported(const PassShape& s, int mode) {
  if (!s.xres || s.lds) return false;
  if (mode == kModeHalf2) return s.kb == 2 || s.kb == 4 || s.kb == 8;
  if (mode == kModeBF16) return s.kb == 1 || s.kb == 2 || s.kb == 4 || s.kb == 8 || s.kb == 16;
  return false;
}

hipError_t launch_lse_solo(const PassShape& s, int mode, const void* Rp, const void* Cp,
                           const float* cbias, float c, const RowFinish& fin, float* err_part,
                           hipStream_t st, const LaunchTimer* t) {
  if (!lse_solo_supported(s, mode) || fin.avg || fin.rpad != s.rtiles * kTile)
    return hipErrorInvalidValue;
  if (mode == kModeHalf2) {
    switch (s.kb) {
      case 2: lse_solo_go<kModeHalf2, 2>(s, Rp, Cp, cbias, c, fin, err_part, st, t); break;
      case 4: lse_solo_go<kModeHalf2, 4>(s, Rp, Cp, cbias, c, fin, err_part, st, t); break;
      default: lse_solo_go<kModeHalf2, 8>(s, Rp, Cp, cbias, c, fin, err_part, st, t); break;
    }
  } else {
    switch (s.kb) {
      case 1: lse_solo_go<kModeBF16, 1>(s, Rp, Cp, cbias, c, fin, err_part, st, t); break;
      case 2: lse_solo_go<kModeBF16, 2>(s, Rp, Cp, cbias, c, fin, err_part, st, t); break;
      case 4: lse_solo_go<kModeBF16, 4>(s, Rp, Cp, cbias, c, fin, err_part, st, t); break;
      case 8: lse_solo_go<kModeBF16, 8>(s, Rp, Cp, cbias, c, fin, err_part, st, t); break;
      default: lse_solo_go<kModeBF16, 16>(s, Rp, Cp, cbias, c, fin, err_part, st, t); break;
    }
  }
  return hipGetLastError();
}

template <bool VEC>
static hipError_t resident_dispatch(const PassShape& s, int mode, const ResArgs& a,
                                    hipStream_t st) {
  if (!s.xres) return hipErrorInvalidValue;
  if (mode == kModeSplit) return lse_split_dispatch<VEC>(s, a, st);
  if (mode == kModeHalf2) return lse_half2_dispatch<VEC>(s, a, st);
  if (mode == kModeBF16) return lse_resident_dispatch<kModeBF16, VEC>(s, a, st);
  return lse_resident_dispatch<kModeF32, VEC>(s, a, st);
}

hipError_t launch_lse_resident(const PassShape& s, int mode, const void* Rp, const void* Cp,
                               const float* cbias, float c, float2* part, hipStream_t st,
                               const LaunchTimer* t) {
  return resident_dispatch<false>(s, mode,
                                  ResArgs{Rp, Cp, cbias, nullptr, c, part, nullptr, t}, st);
}

hipError_t launch_vec_resident(const PassShape& s, int mode, const void* Rp, const void* Cp,
                               const float* cbias, const float* vcol, float c, float2* part,
                               float* partT, hipStream_t st) {
  return resident_dispatch<true>(s, mode, ResArgs{Rp, Cp, cbias, vcol, c, part, partT, nullptr},
                                 st);
}

}  // namespace flashot
