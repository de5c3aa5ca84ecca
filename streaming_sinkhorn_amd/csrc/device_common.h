// Device helpers shared by the streamed kernels of the Sinkhorn solver
// (score tiles on the matrix cores, online log-sum-exp steps). Internal.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.h"

namespace flashot {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// Launches `kernel` on `st`; with a timer the dispatch itself records the
// start and end events (no event commands of their own between launches).
template <typename... F, typename... A>
static void launch_timed(void (*kernel)(F...), dim3 grid, dim3 block, hipStream_t st,
                         const LaunchTimer* timer, A... args) {
  if (timer)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, timer->start, timer->stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
}

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

// 1 KiB operand units per k-block, and matrix instructions per tile of KB units.
template <int MODE>
constexpr int units_per_kblock() { return MODE == kModeSplit ? 3 : (MODE == kModeHalf2 ? 2 : 1); }
template <int MODE, int KB>
constexpr int tile_mfmas() {
  return MODE == kModeF32 ? 4 * KB
                          : (MODE == kModeSplit ? 2 * KB : (MODE == kModeHalf2 ? 3 * KB / 2 : KB));
}

// The lazy online LSE (lse_fast) for passes whose tiles carry little matrix
// work (at most three score MFMAs: d <= 16 in the fp16 split, d <= 48 in
// bf16), where the vector work bounds the pass.
template <int MODE, int KB>
constexpr bool lazy_lse() { return tile_mfmas<MODE, KB>() <= 3; }

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

// One k-block of 16 fp32 values held as two fp16 parts per operand (v = hi +
// lo, lo the fp16 rounding of v - hi, so v - hi - lo is below 2^-22 |v|;
// the values are pre-scaled by powers of two into the fp16 range). Three
// partial products are accumulated, smallest first; the dropped lo * lo and
// the two residuals are each below 2^-22 of |x y|.
__device__ __forceinline__ f32x16 mfma_half2(const u32x4* y, const u32x4* x, f32x16 acc) {
  auto m = [](u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  };
  acc = m(y[1], x[0], acc);  // lo * hi
  acc = m(y[0], x[1], acc);  // hi * lo
  return m(y[0], x[0], acc); // hi * hi
}

// Adds bias_j - Mf_i to accumulator entry (j, i) on the bf16 matrix cores
// (32x32x8, the same 8 passes as the wider bf16 shape, and half the cycles of
// the fp32 32x32x2 instruction). Each lane supplies four bf16 k-values:
// a (column side, lane l): lanes < 32 the three bf16 parts of bias_j (j = l)
// and 0, lanes >= 32 three bf16 ones and 0; b (row side): lanes < 32 three
// ones and 0, lanes >= 32 the parts of -Mf_i (i = l - 32) and 0. So k-slots
// 0..2 carry (parts of bias_j, 1) and k-slots 4..6 carry (1, parts of
// -Mf_i). The parts sum to the fp32 values exactly and the products are exact.
// Measured on gfx950, this instruction's rounding is biased when it adds onto
// a nonzero accumulator (mean error about -0.2 ulp at score magnitudes) and
// unbiased from a zero one, so the passes form bias - stabiliser first and
// accumulate the score products onto it.
__device__ __forceinline__ f32x16 mfma_bias_stab(uint2 a, uint2 b, f32x16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(__builtin_bit_cast(s16x4, a),
                                                  __builtin_bit_cast(s16x4, b), acc, 0, 0, 0);
}

// Row-side operand of mfma_bias_stab for the folded stabiliser Mf.
__device__ __forceinline__ uint2 stab_operand(float Mf, int h) {
  return h ? bf16x3_parts(-Mf) : make_uint2(kBf16OnesLo, kBf16OnesHi);
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
// stabiliser M, not only for the running maximum. The bias MFMA
// (mfma_bias_stab) also subtracts M_i from every score, so in the common
// case a tile costs one exp2 and one add per score (plus one rescale per
// tile in the eager variant, none in the lazy one; see lse_fast). Only when
// a tile could overflow (tile sum >= 2^64), before M has been set from data,
// or (lazy variant) for the tile already scored when M moved, does the wave
// take the exact path: tile maximum, raise M, rescale S. M is kept identical
// in the two lanes (l, l ^ 32) that share a row, because the bias MFMA reads
// it from lane l + 32.
//
// Units: for fp32 inputs the row operand X is packed pre-multiplied by
// c = 2 log2(e) / eps and the biases are written in the same units, so scores
// are log2 values and exp2 needs no multiply (KS = 1). In half2 mode X is
// further multiplied by 2^a and Y by 2^-a (exact), which leaves the product
// unchanged. bf16 operands cannot be
// rescaled without rounding, so their scores stay in dot-product units and
// are multiplied by c before exp2 (KS = c). Partials are written in log2
// units: LSE_row = ln 2 * (M2 + log2 S).
// ---------------------------------------------------------------------------
constexpr float kUnset = -1.0e30f;  // stabiliser not yet taken from data

// How a pass adds bias_j - Mf_i, per operand mode. The fp32-precision modes
// (three-part bf16 split, fp32 MFMA) keep the fp32 32x32x2 instruction after
// the score products, which adds in round-to-nearest without disturbing
// their smallest-first product order. The default fp16 split and bf16 points
// start each tile from mfma_bias_stab (bf16 parts, half the cycles).
template <int MODE>
constexpr bool f32_bias() { return MODE == kModeSplit || MODE == kModeF32; }
// Column-side operand: the fp32 bias, or the lane's entry of the parts layout.
template <int MODE>
using BiasOp = typename std::conditional<f32_bias<MODE>(), float, uint2>::type;

template <int MODE>
__device__ __forceinline__ BiasOp<MODE> load_bias(const float* __restrict__ cbias,
                                                  const uint2* __restrict__ cb3, size_t jt,
                                                  int lane) {
  if constexpr (f32_bias<MODE>()) return cbias[jt * kTile + (lane & 31)];
  else return cb3[jt * 64 + lane];
}
// Column-side operand of tiles past the end of the columns: the sentinel bias.
template <int MODE>
__device__ __forceinline__ BiasOp<MODE> sentinel_bias(int h) {
  if constexpr (f32_bias<MODE>()) return kSentinel;
  else return h ? make_uint2(kBf16OnesLo, kBf16OnesHi) : bf16x3_parts(kSentinel);
}
// Row-side operand for the folded stabiliser Mf.
template <int MODE>
__device__ __forceinline__ BiasOp<MODE> stab_of(float Mf, int h) {
  if constexpr (f32_bias<MODE>()) return h ? -Mf : 1.0f;
  else return stab_operand(Mf, h);
}
// Accumulator a tile's score products start from.
template <int MODE>
__device__ __forceinline__ f32x16 bias_start(BiasOp<MODE> a, BiasOp<MODE> b) {
  if constexpr (f32_bias<MODE>()) return f32x16{};
  else return mfma_bias_stab(a, b, f32x16{});
}
// After the products: the fp32 modes add bias_j - Mf_i here (k-slot 0 carries
// (bias_j, 1), k-slot 1 carries (1, -Mf_i)).
template <int MODE>
__device__ __forceinline__ f32x16 bias_finish(BiasOp<MODE> a, BiasOp<MODE> b, int h, f32x16 acc) {
  if constexpr (f32_bias<MODE>()) return __builtin_amdgcn_mfma_f32_32x32x2f32(h ? 1.0f : a, b, acc, 0, 0, 0);
  else return acc;
}

// KB counts 1 KiB operand units per tile: one per k-block for fp32 / bf16,
// three (hi, mid, lo) per k-block in split mode, two (hi, lo) in half2 mode.
template <int MODE, int KB, int RI>
__device__ __forceinline__ void score_tile(const u32x4 (&y)[KB], const u32x4 (&xr)[RI][KB],
                                           BiasOp<MODE> ab, const BiasOp<MODE> (&Bst)[RI], int h,
                                           f32x16 (&acc)[RI]) {
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) acc[ri] = bias_start<MODE>(ab, Bst[ri]);
  if constexpr (MODE == kModeSplit) {
#pragma unroll
    for (int kb = 0; kb < KB; kb += 3)
#pragma unroll
      for (int ri = 0; ri < RI; ++ri) acc[ri] = mfma_split(&y[kb], &xr[ri][kb], acc[ri]);
  } else if constexpr (MODE == kModeHalf2) {
#pragma unroll
    for (int kb = 0; kb < KB; kb += 2)
#pragma unroll
      for (int ri = 0; ri < RI; ++ri) acc[ri] = mfma_half2(&y[kb], &xr[ri][kb], acc[ri]);
  } else {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
        acc[ri] = mfma_kblock<MODE == kModeBF16>(y[kb], xr[ri][kb], acc[ri]);
  }
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) acc[ri] = bias_finish<MODE>(ab, Bst[ri], h, acc[ri]);
}

// Stabiliser folded into the next tile's scores: the running M once set.
__device__ __forceinline__ float fold_of(float M) { return M > 0.5f * kUnset ? M : 0.f; }

// After M may have moved (the exact path): the folded stabiliser of the next
// tiles and its row-side bias operand.
template <int MODE, int RI>
__device__ __forceinline__ void refold(const float (&M)[RI], int h, float (&Mfc)[RI],
                                       BiasOp<MODE> (&Bst)[RI]) {
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) {
    Mfc[ri] = fold_of(M[ri]);
    Bst[ri] = stab_of<MODE>(Mfc[ri], h);
  }
}

// Common-case tile: s = sum exp2(ks * a_r) relative to the folded Mf; returns
// the candidate new S and whether the exact path is needed. Two variants:
//  * eager (LAZY = false): the tile is rescaled by 2^(Mf - M) into the
//    current stabiliser, and the exact path raises M to every new maximum;
//  * lazy (LAZY = true): no rescale; the tile must have been scored with the
//    current stabiliser (Mf == M), and the exact path raises M only when a
//    tile could reach 2^32, so a raise sends just the one tile already scored
//    with the old value down the exact path. One exponential and three
//    vector instructions fewer per tile: measured 3-6 % faster where the
//    vector work bounds the pass (d = 16), but 2 % slower at d = 64, where
//    the matrix work does.
template <bool SCALED, bool LAZY>
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
  if constexpr (LAZY) {
    Snew = S + s;
    // Exact path when the tile could overflow (or is NaN), or was scored with
    // another stabiliser than the current one (also when M is not set: Mf = 0).
    return !(s < 0x1p64f) | (Mf != M);
  } else {
    Snew = fmaf(s, __builtin_amdgcn_exp2f(ks * (Mf - M)), S);
    // Exact path when: the tile could overflow; the stabiliser is not set; or
    // the tile was folded before it was set (Mf = 0 above a lower M), where
    // the rescale factor itself could overflow.
    return !(s < 0x1p64f) | !(Snew >= 0x1p-64f) | !(M > 0.5f * kUnset) | !(Mf <= M);
  }
}

// Exact tile: raise M to the tile maximum (shared by the lane pair), rescale.
// The maximum is taken over the scores u = a + Mf as rounded, and every
// exponent is u - m of those same values: it is <= 0, and exactly 0 at the
// maximum, however large |u| is (writing it as a + (Mf - m) instead lets
// rounding push the maximum's exponent far from 0 once |scores| reach fp32's
// integer range). A NaN score still reaches S.
// In the lazy variant M is kept while the tile's maximum stays within 2^32 of
// it (exponents <= 32, a tile sum below 2^36), so a raise of any row does not
// force its next tiles onto this path.
template <bool LAZY>
__device__ __forceinline__ float stab_after(float m, float M, float ks) {
  if constexpr (LAZY) return (M > 0.5f * kUnset && ks * (m - M) <= 32.f) ? M : fmaxf(m, M);
  else return fmaxf(m, M);
}

template <bool LAZY>
__device__ __forceinline__ void lse_exact(const f32x16& a, float Mf, float& M, float& S,
                                          float ks) {
  float m = a[0] + Mf;
#pragma unroll
  for (int r = 1; r < 16; ++r) m = fmaxf(m, a[r] + Mf);
  m = fmaxf(m, __shfl_xor(m, 32));
  m = stab_after<LAZY>(m, M, ks);
  float e0 = 0.f, e1 = 0.f, e2 = 0.f, e3 = 0.f;
#pragma unroll
  for (int r = 0; r < 16; r += 4) {
    e0 += __builtin_amdgcn_exp2f(ks * ((a[r + 0] + Mf) - m));
    e1 += __builtin_amdgcn_exp2f(ks * ((a[r + 1] + Mf) - m));
    e2 += __builtin_amdgcn_exp2f(ks * ((a[r + 2] + Mf) - m));
    e3 += __builtin_amdgcn_exp2f(ks * ((a[r + 3] + Mf) - m));
  }
  S = fmaf(S, __builtin_amdgcn_exp2f(ks * (M - m)), (e0 + e1) + (e2 + e3));
  M = m;
}

// Online LSE of RI score tiles (one per row tile) outside a scheduled
// pipeline stage: common case, or the exact path for the whole wave.
template <int MODE, int RI, bool LAZY>
__device__ __forceinline__ void lse_tail(const f32x16 (&acc)[RI], const float (&Mf)[RI],
                                         float (&M)[RI], float (&S)[RI], float ks) {
  float So[RI];
  int slow = 0;
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) {
    So[ri] = S[ri];
    slow |= lse_fast<MODE != kModeBF16, LAZY>(acc[ri], Mf[ri], M[ri], So[ri], ks, S[ri]);
  }
  if (__builtin_amdgcn_ballot_w64(slow) != 0) {
#pragma unroll
    for (int ri = 0; ri < RI; ++ri) {
      S[ri] = So[ri];
      lse_exact<LAZY>(acc[ri], Mf[ri], M[ri], S[ri], ks);
    }
  }
}

// ---------------------------------------------------------------------------
// Transport-vector variant (P v with one value column): next to S, the same
// online recurrence carries T = sum_j exp2(score_ij - M) v_j, rescaled with S
// whenever M moves, so (P v)_i = a_i 2^((f_i - alpha_i) log2(e)/eps + M) T.
// ---------------------------------------------------------------------------
// Values v_j of the 16 accumulator rows a lane holds in tile jt: row r of
// the 32x32 accumulator is column j = 8 (r / 4) + 4 h + r % 4 of the tile.
__device__ __forceinline__ f32x16 load_tile_values(const float* __restrict__ v, int jt, int h) {
  const float4* p = reinterpret_cast<const float4*>(v + (size_t)jt * kTile + 4 * h);
  f32x16 out;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float4 q = p[2 * k];
    out[4 * k + 0] = q.x;
    out[4 * k + 1] = q.y;
    out[4 * k + 2] = q.z;
    out[4 * k + 3] = q.w;
  }
  return out;
}

template <bool SCALED, bool LAZY>
__device__ __forceinline__ bool lse_fast_v(const f32x16& a, const f32x16& v, float Mf, float M,
                                           float S, float T, float ks, float& Snew,
                                           float& Tnew) {
  float e0 = 0.f, e1 = 0.f, t0 = 0.f, t1 = 0.f;
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    const float x0 = __builtin_amdgcn_exp2f(SCALED ? a[r] : ks * a[r]);
    const float x1 = __builtin_amdgcn_exp2f(SCALED ? a[r + 1] : ks * a[r + 1]);
    e0 += x0;
    e1 += x1;
    t0 = fmaf(x0, v[r], t0);
    t1 = fmaf(x1, v[r + 1], t1);
  }
  const float s = e0 + e1;
  if constexpr (LAZY) {  // as lse_fast
    Snew = S + s;
    Tnew = T + (t0 + t1);
    return !(s < 0x1p64f) | (Mf != M);
  } else {
    const float f = __builtin_amdgcn_exp2f(ks * (Mf - M));
    Snew = fmaf(s, f, S);
    Tnew = fmaf(t0 + t1, f, T);
    return !(s < 0x1p64f) | !(Snew >= 0x1p-64f) | !(M > 0.5f * kUnset) | !(Mf <= M);
  }
}

template <bool LAZY>
__device__ __forceinline__ void lse_exact_v(const f32x16& a, const f32x16& v, float Mf, float& M,
                                            float& S, float& T, float ks) {
  // the same exponents and stabiliser as lse_exact
  float m = a[0] + Mf;
#pragma unroll
  for (int r = 1; r < 16; ++r) m = fmaxf(m, a[r] + Mf);
  m = fmaxf(m, __shfl_xor(m, 32));
  m = stab_after<LAZY>(m, M, ks);
  float e = 0.f, tv = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float x = __builtin_amdgcn_exp2f(ks * ((a[r] + Mf) - m));
    e += x;
    tv = fmaf(x, v[r], tv);
  }
  const float sc = __builtin_amdgcn_exp2f(ks * (M - m));
  S = fmaf(S, sc, e);
  T = fmaf(T, sc, tv);
  M = m;
}

template <int MODE, int RI, bool LAZY>
__device__ __forceinline__ void lse_tail_v(const f32x16 (&acc)[RI], const f32x16& v,
                                           const float (&Mf)[RI], float (&M)[RI], float (&S)[RI],
                                           float (&T)[RI], float ks) {
  float So[RI], To[RI];
  int slow = 0;
#pragma unroll
  for (int ri = 0; ri < RI; ++ri) {
    So[ri] = S[ri];
    To[ri] = T[ri];
    slow |= lse_fast_v<MODE != kModeBF16, LAZY>(acc[ri], v, Mf[ri], M[ri], So[ri], To[ri], ks, S[ri],
                                          T[ri]);
  }
  if (__builtin_amdgcn_ballot_w64(slow) != 0) {
#pragma unroll
    for (int ri = 0; ri < RI; ++ri) {
      S[ri] = So[ri];
      T[ri] = To[ri];
      lse_exact_v<LAZY>(acc[ri], v, Mf[ri], M[ri], S[ri], T[ri], ks);
    }
  }
}

}  // namespace flashot
