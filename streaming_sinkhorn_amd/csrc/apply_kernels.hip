// Streamed transport application (Algorithms 2 / 4 of "FlashSinkhorn:
// IO-Aware Entropic Optimal Transport on GPU", Prop. 3, App. E.1): the same
// score tile and row softmax as the log-sum-exp pass, with the exponentiated
// scores reused directly as the B operand of a second MFMA that accumulates
// O^T += V^T P^T. The rows of V are pre-permuted into the accumulator's row
// order, so P never leaves registers and the running rescale of O is
// lane-local (App. G.2 row-stationary loop order).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device_common.h"

namespace flashot {

static inline int ceil_div_dev(int a, int b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// Streamed transport application partials (Algorithm 2 / 4 of the page).
// Per split s and row i: (M, S) as in the LSE pass, and
//   O[p] = sum_j exp2(c (v_ij - M)) V[j][p]
// accumulated as O^T (p x i) += V^T (p x j) P^T (j x i) on the matrix cores.
// Both half-waves of a row share the running max, so O needs no merge.
// HAD (Algorithm 5, Hadamard-weighted transport (P . A Y^T) V): a second
// score tile W_ij = a_i . y_j is formed from the packed rows of A on the
// same column operand, and each exponentiated score is multiplied by it
// before the value product; S keeps the unweighted sum. With XRES the rows
// of X and of A stay in registers for the whole sweep (d <= 64 in fp32);
// wider rows are streamed per k-chunk.
// Grid: (nrowgroups * splits, passes); pass y covers value blocks
// [y * PB, y * PB + PB) of 32 columns each.
// ---------------------------------------------------------------------------
template <bool BF16, int KB, bool XRES, int PB, bool HAD>
__global__ __launch_bounds__(256) void apply_partial_kernel(
    const u32x4* __restrict__ Rp, const u32x4* __restrict__ Cp, const u32x4* __restrict__ Ap,
    const float* __restrict__ cbias, const f32x4* __restrict__ Vp, int rtiles, int ctiles,
    int kbp, int splits, int tps, float c, int pblocks, float2* __restrict__ partMS,
    float* __restrict__ partO, int rpad, int ppad) {
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

  u32x4 xr[KB], ar[HAD && XRES ? KB : 1];
  if constexpr (XRES) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      xr[kb] = Rp[((size_t)rt * KB + kb) * 64 + lane];
      if constexpr (HAD) ar[kb] = Ap[((size_t)rt * KB + kb) * 64 + lane];
    }
  }
  float M = -1.0e30f, S = 0.f;
  f32x16 O[PB];
#pragma unroll
  for (int pb = 0; pb < PB; ++pb) O[pb] = f32x16{};

  for (int jt = jt0; jt < jt1; ++jt) {
    f32x16 acc = f32x16{};
    f32x16 accw = f32x16{};
    if constexpr (XRES) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const u32x4 y = Cp[((size_t)jt * KB + kb) * 64 + lane];
        acc = mfma_kblock<BF16>(y, xr[kb], acc);
        if constexpr (HAD) accw = mfma_kblock<BF16>(y, ar[kb], accw);
      }
    } else {
      for (int kc = 0; kc < kbp; kc += KB) {
        u32x4 yc[KB], xc[KB], ac[HAD ? KB : 1];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          yc[kb] = Cp[((size_t)jt * kbp + kc + kb) * 64 + lane];
          xc[kb] = Rp[((size_t)rt * kbp + kc + kb) * 64 + lane];
          if constexpr (HAD) ac[kb] = Ap[((size_t)rt * kbp + kc + kb) * 64 + lane];
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          acc = mfma_kblock<BF16>(yc[kb], xc[kb], acc);
          if constexpr (HAD) accw = mfma_kblock<BF16>(yc[kb], ac[kb], accw);
        }
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
    if constexpr (HAD) {
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] *= accw[r];
    }
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
// The same pass with the value product on the fp16 matrix cores. Each
// exponentiated score p (in (0, 1] after the running max) is split into
// fp16 parts ph = fp16(p), pl = fp16(p - ph); V arrives as hi, lo fp16 parts
// of V 2^b (per-column exact scale, undone in the merge), so a product
// costs three 32x32x16 fp16 MFMAs per 16 streamed rows (ph vh, ph vl, pl vh;
// each below 2^-22 relative error per term) where fp32 operands took eight
// 32x32x2 ones. A lane's accumulator entries 8q .. 8q + 7 are its B operand
// for k-chunk q as they stand: the value layout follows that k order.
// SMODE: kModeHalf2 scores (fp32 points as two fp16 parts, log2 units,
// c = 1), kModeBF16 or kModeF32 scores (dot-product units, multiplied by c).
// KB: operand units per tile (XRES) or per k-chunk.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pack_f16x2(_Float16 a, _Float16 b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

template <int SMODE, int KB, bool XRES, int PB>
__global__ __launch_bounds__(256) void apply_h2_kernel(
    const u32x4* __restrict__ Rp, const u32x4* __restrict__ Cp, const float* __restrict__ cbias,
    const u32x4* __restrict__ Vh, int rtiles, int ctiles, int kbp, int splits, int tps, float c,
    int pblocks, float2* __restrict__ partMS, float* __restrict__ partO, int rpad, int ppad) {
  constexpr int KU = units_per_kblock<SMODE>();
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

  u32x4 xr[XRES ? KB : 1];
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
    for (int kc = 0; kc < (XRES ? KB : kbp); kc += KB) {
      u32x4 yc[KB], xc[XRES ? 1 : KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        yc[kb] = Cp[((size_t)jt * kbp + kc + kb) * 64 + lane];
        if constexpr (!XRES) xc[kb] = Rp[((size_t)rt * kbp + kc + kb) * 64 + lane];
      }
#pragma unroll
      for (int kb = 0; kb < KB; kb += KU) {
        const u32x4* xo = XRES ? &xr[kb] : &xc[kb];
        if constexpr (SMODE == kModeHalf2) acc = mfma_half2(&yc[kb], xo, acc);
        else acc = mfma_kblock<SMODE == kModeBF16>(yc[kb], xo[0], acc);
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
    u32x4 ph[2], pl[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const _Float16 a = (_Float16)p[8 * q + e], b = (_Float16)p[8 * q + e + 1];
        hw[e / 2] = pack_f16x2(a, b);
        lw[e / 2] = pack_f16x2((_Float16)(p[8 * q + e] - (float)a),
                               (_Float16)(p[8 * q + e + 1] - (float)b));
      }
      ph[q] = u32x4{hw[0], hw[1], hw[2], hw[3]};
      pl[q] = u32x4{lw[0], lw[1], lw[2], lw[3]};
    }
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) {
      if (pb0 + pb < pblocks) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const u32x4* vb = Vh + ((((size_t)jt * pblocks + pb0 + pb) * 2 + q) * 2) * 64 + lane;
          const f16x8 vh = __builtin_bit_cast(f16x8, vb[0]);
          const f16x8 vl = __builtin_bit_cast(f16x8, vb[64]);
          O[pb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vl, __builtin_bit_cast(f16x8, ph[q]),
                                                         O[pb], 0, 0, 0);
          O[pb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vh, __builtin_bit_cast(f16x8, pl[q]),
                                                         O[pb], 0, 0, 0);
          O[pb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vh, __builtin_bit_cast(f16x8, ph[q]),
                                                         O[pb], 0, 0, 0);
        }
      }
    }
  }

  S += __shfl_xor(S, 32);
  const size_t row = (size_t)rt * kTile + (lane & 31);
  if (blockIdx.y == 0 && h == 0) partMS[(size_t)s * rpad + row] = make_float2(c * M, S);
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
// Pipelined transport application for register-resident row tiles: the
// log-sum-exp pass's machinery (device_common.h) with the value product
// added. Per wave one row tile (32 rows) in registers; the four waves of a
// workgroup share each column tile -- its score operand and its PB blocks of
// fp16 value parts -- through a four-slot LDS ring. Stage k
//  * scores tile k+1 on the matrix cores (two score tiles in flight),
//  * multiplies the values of tile k-1 into O (its p parts were formed in
//    stage k-1), so that stage's matrix work does not wait for its own
//    exponentials,
//  * exponentiates tile k and splits p into fp16 parts on the vector unit,
//  * and stages tile k+2 into the slot of tile k-2 (one barrier per stage).
// The stabiliser is raised lazily: p = exp2(score - M) is used as computed
// while the tile sum stays below 2^15 (so every p fits the fp16 parts), and
// only a tile past that (or, with M folded into the bias MFMA, scored with
// an older M) takes the exact path that raises M to the tile maximum and
// rescales S and O.
// Partials per split and row: (M in log2 units, S) and O, as the merge
// (apply_merge_kernel, c = 1) expects.
// ---------------------------------------------------------------------------
constexpr float kApplyTileSumLimit = 0x1p15f;

// Two ways the stabiliser M enters a tile, chosen by the operand mode:
//  * FOLD (two-part fp16 scores, already in log2 units): M is folded into the
//    bias MFMA like in the log-sum-exp pass, so a tile's exponent is the
//    accumulator itself; a tile scored with an older M takes the exact path;
//  * not FOLD (fp32 or bf16 scores in dot-product units, multiplied by c):
//    the accumulator holds score + bias and p = exp2(fma(c, a, -c M)) with
//    the current M, one rounding at the exponent's magnitude, as in the
//    fp32-value application pass.
// Common-case tile: p and their sum s. Returns whether the exact path is
// needed: the sum (hence some p) could leave the fp16 range, is NaN, M is not
// yet set from data, or (FOLD) the tile was scored with an older M.
template <bool FOLD>
__device__ __forceinline__ bool apply_fast(const f32x16& a, float Mf, float M, float ks, f32x16& p,
                                           float& s) {
  float e[4];
  const float kM = -ks * M;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    p[r] = __builtin_amdgcn_exp2f(FOLD ? a[r] : fmaf(ks, a[r], kM));
    e[r & 3] = r < 4 ? p[r] : e[r & 3] + p[r];
  }
  s = (e[0] + e[1]) + (e[2] + e[3]);
  if constexpr (FOLD) return !(s < kApplyTileSumLimit) | (Mf != M);
  else return !(s < kApplyTileSumLimit) | !(M > 0.5f * kUnset);
}

// Exact path: p recomputed against a stabiliser M that bounds every p of
// the tile by 2^8. M stays while the tile maximum (shared by the lane pair
// that holds the row) is within 8 of it in log2 units, else it is raised to
// that maximum and S and O are rescaled. Raising only past that margin
// keeps the raises, and the exact path of the tile already scored with the
// old M that each raise costs, rare once a row's first tiles are in; a tile
// that took the path for its sum (>= 2^15, so some p >= 2^11) always raises.
// FOLD: exponents from the scores u = a + Mf as rounded, as in lse_exact.
constexpr float kApplyRaiseMargin = 8.0f;

template <bool FOLD, int PB>
__device__ __forceinline__ void apply_exact(const f32x16& a, float Mf, float& M, float& S,
                                            f32x16 (&O)[PB], float ks, f32x16& p) {
  float m = FOLD ? a[0] + Mf : a[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) m = fmaxf(m, FOLD ? a[r] + Mf : a[r]);
  m = fmaxf(m, __shfl_xor(m, 32));
  // M not set (kUnset): the tile maximum
  const float Mn = (M > 0.5f * kUnset && ks * (m - M) <= kApplyRaiseMargin) ? M : fmaxf(m, M);
  const float sc = __builtin_amdgcn_exp2f(ks * (M - Mn));  // 0 when M was not set
  const float kM = -ks * Mn;
  float e[4];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    p[r] = __builtin_amdgcn_exp2f(FOLD ? ks * ((a[r] + Mf) - Mn) : fmaf(ks, a[r], kM));
    e[r & 3] = r < 4 ? p[r] : e[r & 3] + p[r];
  }
  S = fmaf(S, sc, (e[0] + e[1]) + (e[2] + e[3]));
#pragma unroll
  for (int pb = 0; pb < PB; ++pb) O[pb] *= sc;
  M = Mn;
}

// -1.0f that the compiler cannot see through: p - hi written as
// fma(hi, -1, p) with it is selected as one mixed-precision fma that reads hi
// straight from its fp16 half (a literal -1 folds back into a conversion and
// a subtraction). The product is exact and p - hi is exact in fp32, so the
// value is the difference itself.
__device__ __forceinline__ float opaque_minus_one() {
  float r;
  asm("s_mov_b32 %0, -1.0" : "=s"(r));
  return r;
}

// p (accumulator entries 8q .. 8q+7 are the B operand of k-chunk q) as fp16
// parts: hi = fp16(p) and lo = fp16(p - hi), both rounded to nearest.
__device__ __forceinline__ void split_p(const f32x16& p, u32x4 (&ph)[2], u32x4 (&pl)[2]) {
  typedef _Float16 h2v __attribute__((ext_vector_type(2)));
  typedef float f2v __attribute__((ext_vector_type(2)));
  const float m1 = opaque_minus_one();
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const f2v v = {p[8 * q + 2 * w], p[8 * q + 2 * w + 1]};
      const h2v hi = __builtin_convertvector(v, h2v);
      const f2v d = {__builtin_fmaf((float)hi[0], m1, v[0]), __builtin_fmaf((float)hi[1], m1, v[1])};
      const h2v lo = __builtin_convertvector(d, h2v);
      ph[q][w] = __builtin_bit_cast(uint32_t, hi);
      pl[q][w] = __builtin_bit_cast(uint32_t, lo);
    }
}

// Value product of one tile for one 32-column value block: O^T += V^T P^T,
// smallest products first. VP = 2: V's hi / lo parts at units vb[0..3] =
// (chunk 0 hi, chunk 0 lo, chunk 1 hi, chunk 1 lo), three products per
// chunk. VP = 1 (bf16 values): hi parts alone at vb[0..1] = (chunk 0 hi,
// chunk 1 hi), two products per chunk: a bf16 value's lo part is zero. Its
// 8 significant bits fit fp16 wherever the scaled value is at least 2^-17,
// and below that the hi part is the nearest multiple of 2^-24, which leaves
// at most 2^-25, and that rounds to zero in fp16 (ties to even).
template <int VP = 2>
__device__ __forceinline__ f32x16 value_block(const u32x4* __restrict__ vb, int lane,
                                              const u32x4 (&ph)[2], const u32x4 (&pl)[2],
                                              f32x16 o) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const f16x8 vh = __builtin_bit_cast(f16x8, vb[(VP * q) * 64 + lane]);
    if constexpr (VP == 2) {
      const f16x8 vl = __builtin_bit_cast(f16x8, vb[(2 * q + 1) * 64 + lane]);
      o = __builtin_amdgcn_mfma_f32_32x32x16_f16(vl, __builtin_bit_cast(f16x8, ph[q]), o, 0, 0, 0);
    }
    o = __builtin_amdgcn_mfma_f32_32x32x16_f16(vh, __builtin_bit_cast(f16x8, pl[q]), o, 0, 0, 0);
    o = __builtin_amdgcn_mfma_f32_32x32x16_f16(vh, __builtin_bit_cast(f16x8, ph[q]), o, 0, 0, 0);
  }
  return o;
}

// value_block on fragments already in registers: v[0 .. 2 VP) are this
// lane's entries of the units in the staging order above.
template <int VP>
__device__ __forceinline__ f32x16 value_block_frag(const u32x4* v, const u32x4 (&ph)[2],
                                                   const u32x4 (&pl)[2], f32x16 o) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const f16x8 vh = __builtin_bit_cast(f16x8, v[VP * q]);
    if constexpr (VP == 2) {
      const f16x8 vl = __builtin_bit_cast(f16x8, v[2 * q + 1]);
      o = __builtin_amdgcn_mfma_f32_32x32x16_f16(vl, __builtin_bit_cast(f16x8, ph[q]), o, 0, 0, 0);
    }
    o = __builtin_amdgcn_mfma_f32_32x32x16_f16(vh, __builtin_bit_cast(f16x8, pl[q]), o, 0, 0, 0);
    o = __builtin_amdgcn_mfma_f32_32x32x16_f16(vh, __builtin_bit_cast(f16x8, ph[q]), o, 0, 0, 0);
  }
  return o;
}

// Source unit, within a pass's PB value blocks of 4 units each, of staged
// value unit vi (2 VP units per block); blocks past npb repeat the last one.
template <int VP>
__device__ __forceinline__ int value_src_unit(int vi, int npb) {
  if constexpr (VP == 2) return min(vi, 4 * npb - 1);
  else return min(vi >> 1, npb - 1) * 4 + 2 * (vi & 1);
}

template <int SMODE, int KB, int PB, int VP>
__global__ __launch_bounds__(256) void apply_res_kernel(
    const u32x4* __restrict__ Rp, const u32x4* __restrict__ Cp, const float* __restrict__ cbias,
    const u32x4* __restrict__ Vh, int rtiles, int ctiles, int splits, int tps, float c,
    int pblocks, float2* __restrict__ partMS, float* __restrict__ partO, int rpad, int ppad) {
  constexpr int TU = KB + 2 * VP * PB;        // staged 1 KiB units per column tile
  constexpr int NL = (TU * 64 + 255) / 256;   // staging loads per thread
  constexpr bool FOLD = SMODE == kModeHalf2;  // scores in log2 units, M folded into the bias MFMA
  __shared__ u32x4 lds[4][NL * 256];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int s = blockIdx.x % splits;
  const int rg = blockIdx.x / splits;
  // may be past the last row tile: the wave still takes part in loads and barriers
  const int rt = rg * kWaves + wave;
  const int pb0 = blockIdx.y * PB;
  const int npb = min(PB, pblocks - pb0);     // value blocks of this pass, >= 1
  const int jt0 = s * tps;
  const int last = min(jt0 + tps, ctiles) - 1 - jt0;  // split holds tiles 0..last
  const float ks = FOLD ? 1.0f : c;
  const uint2* __restrict__ cb3 = bias_parts(cbias, ctiles * kTile);

  // Staging slots of this thread: unit u of the staged tile (score operand
  // units first, then the pass's value units), lane le of the unit. A wave's
  // 64 threads take one unit, so the source choice is wave-uniform; threads
  // past the end re-read the last unit into the padding.
  const u32x4* src[NL];
  size_t stride[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int e = min(tid + 256 * i, TU * 64 - 1);
    const int u = e >> 6, le = e & 63;
    if (u < KB) {
      src[i] = Cp + (size_t)u * 64 + le;
      stride[i] = (size_t)KB * 64;
    } else {
      src[i] = Vh + ((size_t)pb0 * 4 + value_src_unit<VP>(u - KB, npb)) * 64 + le;
      stride[i] = (size_t)pblocks * 4 * 64;
    }
  }
  auto gload = [&](int jt, u32x4 (&g)[NL]) {
#pragma unroll
    for (int i = 0; i < NL; ++i) g[i] = src[i][(size_t)jt * stride[i]];
  };
  auto sstore = [&](int slot, const u32x4 (&g)[NL]) {
#pragma unroll
    for (int i = 0; i < NL; ++i) lds[slot][tid + 256 * i] = g[i];
  };

  u32x4 xr[1][KB];
  {
    const int rtc = min(rt, rtiles - 1);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) xr[0][kb] = Rp[((size_t)rtc * KB + kb) * 64 + lane];
  }
  float M[1] = {kUnset}, S = 0.f, Mfc[1];
  BiasOp<SMODE> Bst[1];
  refold<SMODE, 1>(M, h, Mfc, Bst);
  f32x16 O[PB];
#pragma unroll
  for (int pb = 0; pb < PB; ++pb) O[pb] = f32x16{};

  auto score = [&](int slot, BiasOp<SMODE> ab, f32x16& acc) {
    u32x4 y[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) y[kb] = lds[slot][kb * 64 + lane];
    f32x16 a1[1];
    score_tile<SMODE, KB, 1>(y, xr, ab, Bst, h, a1);
    acc = a1[0];
  };
  // Every block of the pass is multiplied (a pass's last blocks past npb
  // repeat the last staged unit and are never written): no branch inside
  // the scheduled stage.
  auto values = [&](int slot, const u32x4 (&ph)[2], const u32x4 (&pl)[2]) {
    const u32x4* vb = &lds[slot][KB * 64];
#pragma unroll
    for (int pb = 0; pb < PB; ++pb)
      O[pb] = value_block<VP>(vb + pb * 2 * VP * 64, lane, ph, pl, O[pb]);
  };

  // Prologue: tiles 0 and 1 staged, tile 0 scored.
  u32x4 g[NL];
  gload(jt0, g);
  sstore(0, g);
  gload(jt0 + min(1, last), g);
  sstore(1, g);
  BiasOp<SMODE> aA = load_bias<SMODE>(cbias, cb3, jt0, lane);
  BiasOp<SMODE> aB = load_bias<SMODE>(cbias, cb3, jt0 + min(1, last), lane);
  __syncthreads();
  f32x16 accA, accB;
  float MfA = Mfc[0], MfB = 0.f;
  score(0, aA, accA);
  u32x4 phA[2], plA[2], phB[2], plB[2];

  // Stage k: tile k (accC, scored with MfC) is exponentiated and split into
  // phC / plC; with PREV the values of tile k-1 (parts phP / plP) enter O;
  // with NEXT tile k+1 is scored into accN and tile k+2 is staged.
  auto stage = [&](int k, auto next, auto prev, f32x16& accN, float& MfN, BiasOp<SMODE>& aN,
                   const f32x16& accC, float MfC, BiasOp<SMODE>& aC, const u32x4 (&phP)[2],
                   const u32x4 (&plP)[2], u32x4 (&phC)[2], u32x4 (&plC)[2]) {
    constexpr bool NEXT = decltype(next)::value;
    constexpr bool PREV = decltype(prev)::value;
    __syncthreads();  // tile k+1 is in its slot; every wave is done with stage k-1
    BiasOp<SMODE> a2{};
    if constexpr (NEXT) {
      const int jt2 = jt0 + min(k + 2, last);
      gload(jt2, g);
      a2 = load_bias<SMODE>(cbias, cb3, jt2, lane);
      MfN = Mfc[0];
      score((k + 1) & 3, aN, accN);
    }
    if constexpr (PREV) values((k - 1) & 3, phP, plP);
    f32x16 p;
    float ts;
    const bool slow = apply_fast<FOLD>(accC, MfC, M[0], ks, p, ts);
    split_p(p, phC, plC);
    if constexpr (NEXT || PREV) {
      constexpr int kMfma = (NEXT ? tile_mfmas<SMODE, KB>() + 1 : 0) + (PREV ? 2 * (VP + 1) * PB : 0);
      constexpr int kValu = 16 + 16 + 48 + 8;  // exponentials, sums, split, checks
      constexpr int kValuPer = (kValu + kMfma - 1) / kMfma;
      if constexpr (NEXT) __builtin_amdgcn_sched_group_barrier(0x020, NL + 1, 0);  // global loads
#pragma unroll
      for (int i = 0; i < kMfma; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);         // LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, kValuPer, 0);  // VALU
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (__builtin_amdgcn_ballot_w64(slow) != 0) {
      apply_exact<FOLD, PB>(accC, MfC, M[0], S, O, ks, p);
      split_p(p, phC, plC);
      if constexpr (FOLD) refold<SMODE, 1>(M, h, Mfc, Bst);
    } else {
      S += ts;
    }
    if constexpr (NEXT) {
      sstore((k + 2) & 3, g);
      aC = a2;  // tile k's operand slot now belongs to tile k+2
    }
  };

  using Yes = std::integral_constant<bool, true>;
  using No = std::integral_constant<bool, false>;
  if (last == 0) {
    stage(0, No{}, No{}, accB, MfB, aB, accA, MfA, aA, phB, plB, phA, plA);
    values(0, phA, plA);
  } else {
    stage(0, Yes{}, No{}, accB, MfB, aB, accA, MfA, aA, phB, plB, phA, plA);
    int k = 1;  // at the top: tile k's scores in accB, tile k-1's parts in phA / plA
    for (; k + 2 <= last; k += 2) {
      stage(k, Yes{}, Yes{}, accA, MfA, aA, accB, MfB, aB, phA, plA, phB, plB);
      stage(k + 1, Yes{}, Yes{}, accB, MfB, aB, accA, MfA, aA, phB, plB, phA, plA);
    }
    if (k + 1 == last) {  // stages k and k+1 = last remain
      stage(k, Yes{}, Yes{}, accA, MfA, aA, accB, MfB, aB, phA, plA, phB, plB);
      stage(k + 1, No{}, Yes{}, accB, MfB, aB, accA, MfA, aA, phB, plB, phA, plA);
      values((k + 1) & 3, phA, plA);
    } else {              // stage k = last remains
      stage(k, No{}, Yes{}, accA, MfA, aA, accB, MfB, aB, phA, plA, phB, plB);
      values(k & 3, phB, plB);
    }
  }

  S += __shfl_xor(S, 32);
  if (rt >= rtiles) return;
  const size_t row = (size_t)rt * kTile + (lane & 31);
  if (blockIdx.y == 0 && h == 0) partMS[(size_t)s * rpad + row] = make_float2(ks * M[0], S);
#pragma unroll
  for (int pb = 0; pb < PB; ++pb) {
    if (pb < npb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int pcol = 32 * (pb0 + pb) + 8 * (r >> 2) + 4 * h + (r & 3);
        partO[((size_t)s * ppad + pcol) * rpad + row] = O[pb][r];
      }
    }
  }
}

template <int SMODE, int KB, int PB, int VP>
static void apply_res_go(const PassShape& s, int pblocks, const void* Rp, const void* Cp,
                         const float* cbias, const void* Vh, float c, float2* partMS,
                         float* partO, int ppad, hipStream_t st) {
  dim3 grid(s.nrowgroups * s.splits, (pblocks + PB - 1) / PB);
  apply_res_kernel<SMODE, KB, PB, VP><<<grid, 256, 0, st>>>(
      (const u32x4*)Rp, (const u32x4*)Cp, cbias, (const u32x4*)Vh, s.rtiles, s.ctiles, s.splits,
      s.tps, c, pblocks, partMS, partO, s.rtiles * kTile, ppad);
}

template <int SMODE, int PB, int VP>
static hipError_t apply_res_kb(const PassShape& s, int pblocks, const void* Rp, const void* Cp,
                               const float* cbias, const void* Vh, float c, float2* partMS,
                               float* partO, int ppad, hipStream_t st) {
  // Value blocks per pass: at most two (16 units of row operand: one), which
  // keeps the kernel at two waves per SIMD without register spills; wider
  // value matrices take more passes over the same scores.
#define RES_CASE(K)                                                                         \
  case K:                                                                                   \
    apply_res_go<SMODE, K, (K >= 16 ? 1 : (PB > 2 ? 2 : PB)), VP>(s, pblocks, Rp, Cp, cbias, \
                                                                 Vh, c, partMS, partO, ppad, st); \
    break;
  switch (s.kb) {
    case 1:
      if constexpr (SMODE == kModeHalf2) return hipErrorInvalidValue;
      else
        apply_res_go<SMODE, 1, (PB > 2 ? 2 : PB), VP>(s, pblocks, Rp, Cp, cbias, Vh, c, partMS,
                                                     partO, ppad, st);
      break;
    RES_CASE(2)
    RES_CASE(4)
    RES_CASE(8)
    RES_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef RES_CASE
  return hipGetLastError();
}

template <int SMODE, int KB, bool XRES, int PB>
static void apply_h2_go(const PassShape& s, int pblocks, const void* Rp, const void* Cp,
                        const float* cbias, const void* Vh, float c, float2* partMS, float* partO,
                        int ppad, hipStream_t st) {
  dim3 grid(s.nrowgroups * s.splits, (pblocks + PB - 1) / PB);
  apply_h2_kernel<SMODE, KB, XRES, PB><<<grid, 256, 0, st>>>(
      (const u32x4*)Rp, (const u32x4*)Cp, cbias, (const u32x4*)Vh, s.rtiles, s.ctiles, s.kbp,
      s.splits, s.tps, c, pblocks, partMS, partO, s.rtiles * kTile, ppad);
}

// ---------------------------------------------------------------------------
// Transport application for wide points (row operand not resident): the
// k-chunked pass of the log-sum-exp kernel for wide points (kernels_wide.hip)
// with a value epilogue per column block. A workgroup owns 4 RT row tiles (RT
// per wave) and walks its split's column blocks of CT tiles; a block's score
// tiles are accumulated over the whole dimension in stages of BK k-blocks,
// the column slice staged once in LDS for the four waves (double-buffered)
// and each wave's row slice loaded straight into registers (two sets). After
// the block's last stage the bias and the stabiliser are added (fp32
// instruction), then, tile by tile: the lazy-stabiliser softmax of the
// resident pass (apply_fast / apply_exact), the fp16 split of p, and the
// value product against the tile's value parts: with at most two value
// units per tile, read by each wave straight into registers one tile ahead,
// the next tile's exponentials formed while this tile's value products run
// (no barrier in the epilogue); wider, staged in a second, double-buffered
// LDS area while the previous tile is multiplied. The
// stabiliser a block's tiles are scored against is the one at the block's
// start, so a raise inside a block sends the block's later tiles down the
// exact path (FOLD modes). Splits hold whole blocks: the host rounds the
// tiles per split to a multiple of CT. The fp16-split (FOLD) and bf16
// scores only: fp32 scores keep the chunked kernel above.
// ---------------------------------------------------------------------------
template <int SMODE, int RT, int CT, int BK, int PB, int VP>
__global__ __launch_bounds__(256) void apply_wide_kernel(
    const u32x4* __restrict__ Rp, const u32x4* __restrict__ Cp, const float* __restrict__ cbias,
    const u32x4* __restrict__ Vh, int rtiles, int ctiles, int kbp, int splits, int tps,
    int nrowgroups, float c, int pblocks, float2* __restrict__ partMS, float* __restrict__ partO,
    int rpad, int ppad) {
  constexpr int KU = units_per_kblock<SMODE>();
  constexpr int SU = BK * KU;                     // units per tile per stage
  constexpr int NL = (CT * SU * 64 + 255) / 256;  // column staging loads per thread
  constexpr int VE = PB * 2 * VP * 64;            // value entries (16 B) per tile
  constexpr int NV = (VE + 255) / 256;            // value staging loads per thread
  constexpr bool FOLD = SMODE == kModeHalf2;
  // Value fragments of at most two units per block: read by each wave into
  // registers (RV), else staged in LDS tile by tile.
  constexpr bool RV = RT == 1 && PB * VP <= 2;
  __shared__ u32x4 lds[2][NL * 256];
  __shared__ u32x4 vlds[RV ? 1 : 2][RV ? 1 : NV * 256];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  // XCD-aware order, as in the wide log-sum-exp pass: workgroup w runs on XCD
  // w % 8, and an XCD's workgroups take row groups xcd, xcd + 8, ... with the
  // split index fastest.
  const int xcd = blockIdx.x & 7;
  const int li = blockIdx.x >> 3;
  const int s = li % splits;
  const int rg = (li / splits) * 8 + xcd;
  if (rg >= nrowgroups) return;                   // whole workgroup: no barrier is skipped
  const int rt0 = (rg * kWaves + wave) * RT;      // this wave's row tiles (may be past the last)
  const int pb0 = blockIdx.y * PB;
  const int npb = min(PB, pblocks - pb0);
  const int jtb = s * tps;                        // first column tile of the split
  const int nb = (min(jtb + tps, ctiles) - jtb + CT - 1) / CT;  // >= 1
  const int nstages = kbp / SU;                   // per column block (even)
  const int total = nb * nstages;
  const float ks = FOLD ? 1.0f : c;

  int cq[NL], uo[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int e = min(tid + 256 * i, CT * SU * 64 - 1);
    cq[i] = e / (SU * 64);
    uo[i] = ((e / 64) % SU) * 64 + (e & 63);
  }
  auto gload = [&](int step, u32x4 (&g)[NL]) {
    step = min(step, total - 1);
    const int jt = jtb + (step / nstages) * CT;
    const size_t koff = (size_t)(step % nstages) * SU * 64;
#pragma unroll
    for (int i = 0; i < NL; ++i)
      g[i] = Cp[(size_t)min(jt + cq[i], ctiles - 1) * kbp * 64 + koff + uo[i]];
  };
  auto sstore = [&](u32x4* buf, const u32x4 (&g)[NL]) {
#pragma unroll
    for (int i = 0; i < NL; ++i) buf[tid + 256 * i] = g[i];
  };
  const u32x4* xsrc[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r)
    xsrc[r] = Rp + (size_t)min(rt0 + r, rtiles - 1) * kbp * 64 + lane;
  auto rload = [&](int step, u32x4 (&x)[RT][SU]) {
    step = min(step, total - 1);
    const size_t koff = (size_t)(step % nstages) * SU * 64;
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int u = 0; u < SU; ++u) x[r][u] = xsrc[r][koff + u * 64];
  };
  // Value staging: entry e of a tile's PB * 2 VP units (the pass's blocks;
  // units past npb repeat the last one and are never written out).
  int vu[NV], vl[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = min(tid + 256 * i, VE - 1);
    vu[i] = value_src_unit<VP>(e >> 6, npb);
    vl[i] = e & 63;
  }
  auto vload = [&](int jt, u32x4 (&gv)[NV]) {
    jt = min(jt, ctiles - 1);
#pragma unroll
    for (int i = 0; i < NV; ++i)
      gv[i] = Vh[(((size_t)jt * pblocks + pb0) * 4 + vu[i]) * 64 + vl[i]];
  };
  auto vstore = [&](int buf, const u32x4 (&gv)[NV]) {
#pragma unroll
    for (int i = 0; i < NV; ++i) vlds[buf][tid + 256 * i] = gv[i];
  };

  float M[RT], S[RT];
  f32x16 O[RT][PB];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    M[r] = kUnset;
    S[r] = 0.f;
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) O[r][pb] = f32x16{};
  }

  u32x4 gA[NL], gB[NL];
  u32x4 xA[RT][SU], xB[RT][SU];
  gload(0, gA);
  rload(0, xA);
  sstore(lds[0], gA);
  gload(1, gB);
  rload(1, xB);
  __syncthreads();

  auto compute = [&](const u32x4* buf, const u32x4 (&x)[RT][SU], f32x16 (&acc)[RT][CT]) {
#pragma unroll
    for (int kb = 0; kb < BK; ++kb) {
      u32x4 yf[CT][KU];
#pragma unroll
      for (int q = 0; q < CT; ++q)
#pragma unroll
        for (int u = 0; u < KU; ++u) yf[q][u] = buf[(q * SU + kb * KU + u) * 64 + lane];
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int q = 0; q < CT; ++q) {
          if constexpr (SMODE == kModeHalf2)
            acc[r][q] = mfma_half2(yf[q], &x[r][kb * KU], acc[r][q]);
          else
            acc[r][q] = mfma_kblock<SMODE == kModeBF16>(yf[q][0], x[r][kb], acc[r][q]);
        }
    }
  };

  int step = 0;
  for (int bi = 0; bi < nb; ++bi) {
    const int jt0 = jtb + bi * CT;
    float Mf[RT];
    f32x16 acc[RT][CT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      Mf[r] = FOLD ? fold_of(M[r]) : 0.f;
#pragma unroll
      for (int q = 0; q < CT; ++q) acc[r][q] = f32x16{};
    }
    for (int st = 0; st < nstages; st += 2, step += 2) {
      gload(step + 2, gA);
      compute(lds[0], xA, acc);
      rload(step + 2, xA);
      sstore(lds[1], gB);
      __syncthreads();
      gload(step + 3, gB);
      compute(lds[1], xB, acc);
      rload(step + 3, xB);
      sstore(lds[0], gA);
      __syncthreads();
    }
    // bias_j - Mf_i after the products, on the fp32 instruction (k-slot 0:
    // (bias_j, 1), k-slot 1: (1, -Mf_i)): over a whole dimension of products
    // the partial sums then round at the products' magnitude, not at the
    // bias's, and the one addition is rounded to nearest.
#pragma unroll
    for (int q = 0; q < CT; ++q) {
      const int jt = jt0 + q;
      const float bj = jt < ctiles ? cbias[(size_t)min(jt, ctiles - 1) * kTile + (lane & 31)]
                                   : kSentinel;
#pragma unroll
      for (int r = 0; r < RT; ++r)
        acc[r][q] = __builtin_amdgcn_mfma_f32_32x32x2f32(h ? 1.0f : bj, h ? -Mf[r] : 1.0f,
                                                         acc[r][q], 0, 0, 0);
    }

    if constexpr (RV) {
      // Value epilogue with the fragments in registers, fetched one tile
      // ahead, and no barrier: the exponentials and the fp16 split of tile
      // q + 1 (after tile q's exact path, which may raise M) are formed while
      // tile q's value products run.
      constexpr int NF = PB * 2 * VP;
      auto vfetch = [&](int jt, u32x4 (&v)[NF]) {
        jt = min(jt, ctiles - 1);
#pragma unroll
        for (int i = 0; i < NF; ++i)
          v[i] = Vh[(((size_t)jt * pblocks + pb0) * 4 + value_src_unit<VP>(i, npb)) * 64 + lane];
      };
      u32x4 vA[NF], vB[NF];
      vfetch(jt0, vA);
      f32x16 pn;
      float tsn;
      bool slown = apply_fast<FOLD>(acc[0][0], Mf[0], M[0], ks, pn, tsn);
#pragma unroll
      for (int q = 0; q < CT; ++q) {
        u32x4 (&vc)[NF] = (q & 1) ? vB : vA;
        u32x4 (&vn)[NF] = (q & 1) ? vA : vB;
        if (q + 1 < CT) vfetch(jt0 + q + 1, vn);
        f32x16 p = pn;
        if (__builtin_amdgcn_ballot_w64(slown) != 0)
          apply_exact<FOLD, PB>(acc[0][q], Mf[0], M[0], S[0], O[0], ks, p);
        else
          S[0] += tsn;
        u32x4 ph[2], pl[2];
        split_p(p, ph, pl);
        if (q + 1 < CT) slown = apply_fast<FOLD>(acc[0][q + 1], Mf[0], M[0], ks, pn, tsn);
#pragma unroll
        for (int pb = 0; pb < PB; ++pb)
          O[0][pb] = value_block_frag<VP>(&vc[pb * 2 * VP], ph, pl, O[0][pb]);
      }
    } else {
      // Value epilogue with the fragments staged in LDS, tile by tile.
      u32x4 gv[NV];
      vload(jt0, gv);
      vstore(0, gv);
#pragma unroll
      for (int q = 0; q < CT; ++q) {
        __syncthreads();  // tile q's values are in vlds[q & 1]; the other slot is free
        if (q + 1 < CT) vload(jt0 + q + 1, gv);
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          // p's fp16 parts times the tile's values; written out in both
          // branches below, so that the common one keeps p and O in place
          // (one join after the exact path costs register copies per tile)
          auto values = [&](const f32x16& p) {
            u32x4 ph[2], pl[2];
            split_p(p, ph, pl);
#pragma unroll
            for (int pb = 0; pb < PB; ++pb)
              O[r][pb] = value_block<VP>(&vlds[q & 1][pb * 2 * VP * 64], lane, ph, pl, O[r][pb]);
          };
          f32x16 p;
          float ts;
          const bool slow = apply_fast<FOLD>(acc[r][q], Mf[r], M[r], ks, p, ts);
          if (__builtin_amdgcn_ballot_w64(slow) != 0) {
            apply_exact<FOLD, PB>(acc[r][q], Mf[r], M[r], S[r], O[r], ks, p);
            values(p);
          } else {
            S[r] += ts;
            values(p);
          }
        }
        if (q + 1 < CT) vstore((q + 1) & 1, gv);
      }
    }
  }

#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const float St = S[r] + __shfl_xor(S[r], 32);
    const int rt = rt0 + r;
    if (rt >= rtiles) continue;
    const size_t row = (size_t)rt * kTile + (lane & 31);
    if (blockIdx.y == 0 && h == 0) partMS[(size_t)s * rpad + row] = make_float2(ks * M[r], St);
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) {
      if (pb < npb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int pcol = 32 * (pb0 + pb) + 8 * (e >> 2) + 4 * h + (e & 3);
          partO[((size_t)s * ppad + pcol) * rpad + row] = O[r][pb][e];
        }
      }
    }
  }
}

template <int SMODE, int PB, int VP>
static hipError_t apply_wide_go(const PassShape& s, int pblocks, const void* Rp, const void* Cp,
                                const float* cbias, const void* Vh, float c, float2* partMS,
                                float* partO, int ppad, hipStream_t st) {
  // One row tile per wave: its O accumulators next to the block's score tiles
  // fit two waves per SIMD with four column tiles per block for up to two
  // value blocks, two column tiles for four (two row tiles per wave, which
  // would halve the LDS reads per matrix instruction, need more registers
  // than two waves per SIMD allow).
  constexpr int RT = 1;
  constexpr int CT = PB >= 4 ? 2 : 4;
  constexpr int BK = SMODE == kModeHalf2 ? 1 : 2;
  constexpr int SU = BK * units_per_kblock<SMODE>();
  static_assert(kApplyWideCT % CT == 0, "splits hold whole blocks");
  if (s.tps % CT || s.kbp % (2 * SU)) return hipErrorInvalidValue;
  const int nrg = ceil_div_dev(s.rtiles, kWaves * RT);
  dim3 grid((nrg + 7) / 8 * 8 * s.splits, (pblocks + PB - 1) / PB);
  apply_wide_kernel<SMODE, RT, CT, BK, PB, VP><<<grid, 256, 0, st>>>(
      (const u32x4*)Rp, (const u32x4*)Cp, cbias, (const u32x4*)Vh, s.rtiles, s.ctiles, s.kbp,
      s.splits, s.tps, nrg, c, pblocks, partMS, partO, s.rtiles * kTile, ppad);
  return hipGetLastError();
}

// Pass with the value product on fp16 parts: the pipelined resident kernel,
// or the block-tiled kernel when the row operand is not resident.
template <int SMODE, int PB, int VP>
static hipError_t apply_stream_pb(const PassShape& s, int pblocks, const void* Rp, const void* Cp,
                                  const float* cbias, const void* Vh, float c, float2* partMS,
                                  float* partO, int ppad, hipStream_t st) {
  if constexpr (SMODE == kModeF32) {
    // fp32 scores (the Hessian-vector product's transport-matrix passes, whose
    // damped Schur solve is sensitive to how their arithmetic differs from the
    // vector passes'): the pipelined resident kernel for d <= 64 (it holds two
    // waves per SIMD up to 8 resident units), else the plain per-tile kernel
    // with an eager running maximum.
    if (s.xres && s.kb <= 8)
      return apply_res_kb<SMODE, PB, 2>(s, pblocks, Rp, Cp, cbias, Vh, c, partMS, partO, ppad, st);
    switch (s.xres ? s.kb : 8) {
      case 1: apply_h2_go<SMODE, 1, true, PB>(s, pblocks, Rp, Cp, cbias, Vh, c, partMS, partO, ppad, st); break;
      case 2: apply_h2_go<SMODE, 2, true, PB>(s, pblocks, Rp, Cp, cbias, Vh, c, partMS, partO, ppad, st); break;
      case 4: apply_h2_go<SMODE, 4, true, PB>(s, pblocks, Rp, Cp, cbias, Vh, c, partMS, partO, ppad, st); break;
      case 8:
        if (s.xres) apply_h2_go<SMODE, 8, true, PB>(s, pblocks, Rp, Cp, cbias, Vh, c, partMS, partO, ppad, st);
        else apply_h2_go<SMODE, 8, false, PB>(s, pblocks, Rp, Cp, cbias, Vh, c, partMS, partO, ppad, st);
        break;
      case 16: apply_h2_go<SMODE, 16, true, PB>(s, pblocks, Rp, Cp, cbias, Vh, c, partMS, partO, ppad, st); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  } else {
    if (s.xres) return apply_res_kb<SMODE, PB, VP>(s, pblocks, Rp, Cp, cbias, Vh, c, partMS, partO, ppad, st);
    return apply_wide_go<SMODE, PB, VP>(s, pblocks, Rp, Cp, cbias, Vh, c, partMS, partO, ppad, st);
  }
}

template <int SMODE, int VP>
static hipError_t apply_stream_dispatch(const PassShape& s, int pblocks, int pb_per_pass,
                                        const void* Rp, const void* Cp, const float* cbias,
                                        const void* Vh, float c, float2* partMS, float* partO,
                                        int ppad, hipStream_t st) {
  switch (pb_per_pass) {
    case 1: return apply_stream_pb<SMODE, 1, VP>(s, pblocks, Rp, Cp, cbias, Vh, c, partMS, partO, ppad, st);
    case 2: return apply_stream_pb<SMODE, 2, VP>(s, pblocks, Rp, Cp, cbias, Vh, c, partMS, partO, ppad, st);
    case 4: return apply_stream_pb<SMODE, 4, VP>(s, pblocks, Rp, Cp, cbias, Vh, c, partMS, partO, ppad, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_apply_stream(const PassShape& s, int smode, int pblocks, int pb_per_pass,
                               int vparts, const void* Rp, const void* Cp, const float* cbias,
                               const void* Vh, float c, float2* partMS, float* partO, int ppad,
                               hipStream_t st) {
  if (vparts != 1 && vparts != 2) return hipErrorInvalidValue;
  if (smode == kModeHalf2)
    return vparts == 1
               ? apply_stream_dispatch<kModeHalf2, 1>(s, pblocks, pb_per_pass, Rp, Cp, cbias, Vh,
                                                      c, partMS, partO, ppad, st)
               : apply_stream_dispatch<kModeHalf2, 2>(s, pblocks, pb_per_pass, Rp, Cp, cbias, Vh,
                                                      c, partMS, partO, ppad, st);
  if (smode == kModeBF16)
    return vparts == 1
               ? apply_stream_dispatch<kModeBF16, 1>(s, pblocks, pb_per_pass, Rp, Cp, cbias, Vh, c,
                                                     partMS, partO, ppad, st)
               : apply_stream_dispatch<kModeBF16, 2>(s, pblocks, pb_per_pass, Rp, Cp, cbias, Vh, c,
                                                     partMS, partO, ppad, st);
  // fp32 scores (the Hessian-vector product's passes): fp32 values, both parts
  if (smode == kModeF32)
    return apply_stream_dispatch<kModeF32, 2>(s, pblocks, pb_per_pass, Rp, Cp, cbias, Vh, c, partMS,
                                              partO, ppad, st);
  return hipErrorInvalidValue;
}

template <bool BF16, int KB, bool XRES, int PB, bool HAD = false>
static void apply_go(const PassShape& s, int pblocks, const void* Rp, const void* Cp,
                     const void* Ap, const float* cbias, const float* Vp, float c,
                     float2* partMS, float* partO, int ppad, hipStream_t st) {
  dim3 grid(s.nrowgroups * s.splits, (pblocks + PB - 1) / PB);
  apply_partial_kernel<BF16, KB, XRES, PB, HAD><<<grid, 256, 0, st>>>(
      (const u32x4*)Rp, (const u32x4*)Cp, (const u32x4*)Ap, cbias, (const f32x4*)Vp, s.rtiles,
      s.ctiles, s.kbp, s.splits, s.tps, c, pblocks, partMS, partO, s.rtiles * kTile, ppad);
}

template <bool BF16, int PB>
static hipError_t apply_dispatch_kb(const PassShape& s, int pblocks, const void* Rp,
                                    const void* Cp, const float* cbias, const float* Vp, float c,
                                    float2* partMS, float* partO, int ppad, hipStream_t st) {
  if (!s.xres) {
    apply_go<BF16, 8, false, PB>(s, pblocks, Rp, Cp, nullptr, cbias, Vp, c, partMS, partO, ppad,
                                 st);
    return hipGetLastError();
  }
  switch (s.kb) {
    case 1: apply_go<BF16, 1, true, PB>(s, pblocks, Rp, Cp, nullptr, cbias, Vp, c, partMS, partO, ppad, st); break;
    case 2: apply_go<BF16, 2, true, PB>(s, pblocks, Rp, Cp, nullptr, cbias, Vp, c, partMS, partO, ppad, st); break;
    case 4: apply_go<BF16, 4, true, PB>(s, pblocks, Rp, Cp, nullptr, cbias, Vp, c, partMS, partO, ppad, st); break;
    case 8: apply_go<BF16, 8, true, PB>(s, pblocks, Rp, Cp, nullptr, cbias, Vp, c, partMS, partO, ppad, st); break;
    case 16: apply_go<BF16, 16, true, PB>(s, pblocks, Rp, Cp, nullptr, cbias, Vp, c, partMS, partO, ppad, st); break;
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

// Hadamard-weighted pass, fp32 operands only. The rows of X and A are read
// per column tile in chunks of min(kb, 8) k-blocks; every layout's unit count
// per tile is a multiple of that chunk.
template <int KB, bool XRES>
static hipError_t hadamard_pb(const PassShape& s, int pblocks, int pb_per_pass, const void* Rp,
                              const void* Cp, const void* Ap, const float* cbias,
                              const float* Vp, float c, float2* partMS, float* partO, int ppad,
                              hipStream_t st) {
  switch (pb_per_pass) {
    case 1: apply_go<false, KB, XRES, 1, true>(s, pblocks, Rp, Cp, Ap, cbias, Vp, c, partMS, partO, ppad, st); break;
    case 2: apply_go<false, KB, XRES, 2, true>(s, pblocks, Rp, Cp, Ap, cbias, Vp, c, partMS, partO, ppad, st); break;
    case 4: apply_go<false, KB, XRES, 4, true>(s, pblocks, Rp, Cp, Ap, cbias, Vp, c, partMS, partO, ppad, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_apply_hadamard(const PassShape& s, int pblocks, int pb_per_pass, const void* Rp,
                                 const void* Cp, const void* Ap, const float* cbias,
                                 const float* Vp, float c, float2* partMS, float* partO, int ppad,
                                 hipStream_t st) {
  const int chunk = s.kbp < 8 ? s.kbp : 8;
  if (s.kbp % chunk) return hipErrorInvalidValue;
  if (s.xres) {  // d <= 64 fp32: rows of X and A resident in registers (kbp = 1, 2, 4, 8)
    switch (s.kbp) {
      case 1: return hadamard_pb<1, true>(s, pblocks, pb_per_pass, Rp, Cp, Ap, cbias, Vp, c, partMS, partO, ppad, st);
      case 2: return hadamard_pb<2, true>(s, pblocks, pb_per_pass, Rp, Cp, Ap, cbias, Vp, c, partMS, partO, ppad, st);
      case 4: return hadamard_pb<4, true>(s, pblocks, pb_per_pass, Rp, Cp, Ap, cbias, Vp, c, partMS, partO, ppad, st);
      case 8: return hadamard_pb<8, true>(s, pblocks, pb_per_pass, Rp, Cp, Ap, cbias, Vp, c, partMS, partO, ppad, st);
      default: break;  // wider resident layouts stream per chunk below
    }
  }
  switch (chunk) {
    case 1: return hadamard_pb<1, false>(s, pblocks, pb_per_pass, Rp, Cp, Ap, cbias, Vp, c, partMS, partO, ppad, st);
    case 2: return hadamard_pb<2, false>(s, pblocks, pb_per_pass, Rp, Cp, Ap, cbias, Vp, c, partMS, partO, ppad, st);
    case 4: return hadamard_pb<4, false>(s, pblocks, pb_per_pass, Rp, Cp, Ap, cbias, Vp, c, partMS, partO, ppad, st);
    case 8: return hadamard_pb<8, false>(s, pblocks, pb_per_pass, Rp, Cp, Ap, cbias, Vp, c, partMS, partO, ppad, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace flashot
