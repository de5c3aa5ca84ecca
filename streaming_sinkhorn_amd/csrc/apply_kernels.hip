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

// ---------------------------------------------------------------------------
// Streamed transport application partials (Algorithm 2 / 4 of the page).
// Per split s and row i: (M, S) as in the LSE pass, and
//   O[p] = sum_j exp2(c (v_ij - M)) V[j][p]
// accumulated as O^T (p x i) += V^T (p x j) P^T (j x i) on the matrix cores.
// Both half-waves of a row share the running max, so O needs no merge.
// HAD (Algorithm 5, Hadamard-weighted transport (P . A Y^T) V): a second
// score tile W_ij = a_i . y_j is formed from the packed rows of A on the
// same column operand, and each exponentiated score is multiplied by it
// before the value product; S keeps the unweighted sum.
// Grid: (nrowgroups * splits, passes); pass y covers value blocks
// [y * PB, y * PB + PB) of 32 columns each.
// ---------------------------------------------------------------------------
template <bool BF16, int KB, bool XRES, int PB, bool HAD>
__global__ __launch_bounds__(256) void apply_partial_kernel(
    const u32x4* __restrict__ Rp, const u32x4* __restrict__ Cp, const u32x4* __restrict__ Ap,
    const float* __restrict__ cbias, const f32x4* __restrict__ Vp, int rtiles, int ctiles,
    int kbp, int splits, int tps, float c, int pblocks, float2* __restrict__ partMS,
    float* __restrict__ partO, int rpad, int ppad) {
  static_assert(!(HAD && XRES), "the weighted pass streams its row operands per chunk");
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
    f32x16 accw = f32x16{};
    if constexpr (XRES) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        acc = mfma_kblock<BF16>(Cp[((size_t)jt * KB + kb) * 64 + lane], xr[kb], acc);
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

template <int SMODE, int KB, bool XRES, int PB>
static void apply_h2_go(const PassShape& s, int pblocks, const void* Rp, const void* Cp,
                        const float* cbias, const void* Vh, float c, float2* partMS, float* partO,
                        int ppad, hipStream_t st) {
  dim3 grid(s.nrowgroups * s.splits, (pblocks + PB - 1) / PB);
  apply_h2_kernel<SMODE, KB, XRES, PB><<<grid, 256, 0, st>>>(
      (const u32x4*)Rp, (const u32x4*)Cp, cbias, (const u32x4*)Vh, s.rtiles, s.ctiles, s.kbp,
      s.splits, s.tps, c, pblocks, partMS, partO, s.rtiles * kTile, ppad);
}

template <int SMODE, int PB>
static hipError_t apply_h2_kb(const PassShape& s, int pblocks, const void* Rp, const void* Cp,
                              const float* cbias, const void* Vh, float c, float2* partMS,
                              float* partO, int ppad, hipStream_t st) {
  if (!s.xres) {
    apply_h2_go<SMODE, 8, false, PB>(s, pblocks, Rp, Cp, cbias, Vh, c, partMS, partO, ppad, st);
    return hipGetLastError();
  }
  switch (s.kb) {
    case 1: if constexpr (SMODE != kModeHalf2) { apply_h2_go<SMODE, 1, true, PB>(s, pblocks, Rp, Cp, cbias, Vh, c, partMS, partO, ppad, st); break; } else { return hipErrorInvalidValue; }
    case 2: apply_h2_go<SMODE, 2, true, PB>(s, pblocks, Rp, Cp, cbias, Vh, c, partMS, partO, ppad, st); break;
    case 4: apply_h2_go<SMODE, 4, true, PB>(s, pblocks, Rp, Cp, cbias, Vh, c, partMS, partO, ppad, st); break;
    case 8: apply_h2_go<SMODE, 8, true, PB>(s, pblocks, Rp, Cp, cbias, Vh, c, partMS, partO, ppad, st); break;
    case 16: apply_h2_go<SMODE, 16, true, PB>(s, pblocks, Rp, Cp, cbias, Vh, c, partMS, partO, ppad, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int SMODE>
static hipError_t apply_h2_dispatch(const PassShape& s, int pblocks, int pb_per_pass,
                                    const void* Rp, const void* Cp, const float* cbias,
                                    const void* Vh, float c, float2* partMS, float* partO,
                                    int ppad, hipStream_t st) {
  switch (pb_per_pass) {
    case 1: return apply_h2_kb<SMODE, 1>(s, pblocks, Rp, Cp, cbias, Vh, c, partMS, partO, ppad, st);
    case 2: return apply_h2_kb<SMODE, 2>(s, pblocks, Rp, Cp, cbias, Vh, c, partMS, partO, ppad, st);
    case 4: return apply_h2_kb<SMODE, 4>(s, pblocks, Rp, Cp, cbias, Vh, c, partMS, partO, ppad, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_apply_h2(const PassShape& s, int smode, int pblocks, int pb_per_pass,
                           const void* Rp, const void* Cp, const float* cbias, const void* Vh,
                           float c, float2* partMS, float* partO, int ppad, hipStream_t st) {
  if (smode == kModeHalf2)
    return apply_h2_dispatch<kModeHalf2>(s, pblocks, pb_per_pass, Rp, Cp, cbias, Vh, c, partMS,
                                         partO, ppad, st);
  if (smode == kModeBF16)
    return apply_h2_dispatch<kModeBF16>(s, pblocks, pb_per_pass, Rp, Cp, cbias, Vh, c, partMS,
                                        partO, ppad, st);
  if (smode == kModeF32)
    return apply_h2_dispatch<kModeF32>(s, pblocks, pb_per_pass, Rp, Cp, cbias, Vh, c, partMS,
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
template <int KB>
static hipError_t hadamard_pb(const PassShape& s, int pblocks, int pb_per_pass, const void* Rp,
                              const void* Cp, const void* Ap, const float* cbias,
                              const float* Vp, float c, float2* partMS, float* partO, int ppad,
                              hipStream_t st) {
  switch (pb_per_pass) {
    case 1: apply_go<false, KB, false, 1, true>(s, pblocks, Rp, Cp, Ap, cbias, Vp, c, partMS, partO, ppad, st); break;
    case 2: apply_go<false, KB, false, 2, true>(s, pblocks, Rp, Cp, Ap, cbias, Vp, c, partMS, partO, ppad, st); break;
    case 4: apply_go<false, KB, false, 4, true>(s, pblocks, Rp, Cp, Ap, cbias, Vp, c, partMS, partO, ppad, st); break;
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
  switch (chunk) {
    case 1: return hadamard_pb<1>(s, pblocks, pb_per_pass, Rp, Cp, Ap, cbias, Vp, c, partMS, partO, ppad, st);
    case 2: return hadamard_pb<2>(s, pblocks, pb_per_pass, Rp, Cp, Ap, cbias, Vp, c, partMS, partO, ppad, st);
    case 4: return hadamard_pb<4>(s, pblocks, pb_per_pass, Rp, Cp, Ap, cbias, Vp, c, partMS, partO, ppad, st);
    case 8: return hadamard_pb<8>(s, pblocks, pb_per_pass, Rp, Cp, Ap, cbias, Vp, c, partMS, partO, ppad, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace flashot
