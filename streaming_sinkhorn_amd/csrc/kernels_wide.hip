// Streamed log-sum-exp pass for wide points (the row operand does not fit in
// registers): both operands are streamed per column tile in k-chunks.
//
// Method: "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU"
// (arXiv 2602.03067), Algorithms 1 / 3, App. D.2 (the row block cannot stay
// on chip when d is large, so operand chunks are re-read per column tile),
// App. D.3 (online log-sum-exp).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device_common.h"

namespace flashot {

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

template <bool BF16, int KB, int RI, bool XRES>
static void lse_go(const PassShape& s, const void* Rp, const void* Cp, const float* cbias,
                   float c, float2* part, hipStream_t st) {
  lse_partial_kernel<BF16, KB, RI, XRES><<<s.nrowgroups * s.splits, 256, 0, st>>>(
      (const u32x4*)Rp, (const u32x4*)Cp, cbias, s.rtiles, s.ctiles, s.kbp, s.splits, s.tps, c,
      part, s.rtiles * kTile);
}


template <bool BF16>
static hipError_t lse_wide_dispatch(const PassShape& s, const void* Rp, const void* Cp,
                                    const float* cbias, float c, float2* part, hipStream_t st) {
  if (s.ri == 2)
    lse_go<BF16, 8, 2, false>(s, Rp, Cp, cbias, c, part, st);
  else
    lse_go<BF16, 8, 1, false>(s, Rp, Cp, cbias, c, part, st);
  return hipGetLastError();
}

hipError_t launch_lse_wide(const PassShape& s, int mode, const void* Rp, const void* Cp,
                           const float* cbias, float c, float2* part, hipStream_t st) {
  if (s.xres || mode == kModeSplit) return hipErrorInvalidValue;
  return mode == kModeBF16 ? lse_wide_dispatch<true>(s, Rp, Cp, cbias, c, part, st)
                           : lse_wide_dispatch<false>(s, Rp, Cp, cbias, c, part, st);
}

}  // namespace flashot
