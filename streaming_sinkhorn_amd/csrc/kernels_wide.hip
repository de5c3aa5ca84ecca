// Streamed log-sum-exp pass for wide points (the row operand does not fit in
// registers): a workgroup-tiled pass that stages k-slices of its row block and
// of one column block at a time in LDS.
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
// Tiled pass for wide points. A workgroup owns 4 RT row tiles (each wave RT
// of them) and walks its split's column blocks of CT tiles; for each block
// the score tiles are accumulated over the whole dimension in stages of BK
// k-blocks. The stage's slice of the column block, which all four waves
// use, is staged once in LDS with one barrier per stage (three buffers and
// the next stage's first k-block read ahead for one-unit k-blocks, a double
// buffer for the split modes); each wave loads the slice of its own row
// tiles straight into registers (two
// register sets, each refilled right after the stage that read it), so LDS
// carries only the shared operand. A wave's RT + CT fragments feed RT * CT
// MFMA tiles. bias_j - M_i enters by one MFMA per tile: at the block's start
// (bf16 parts) or, in the fp32-precision modes, after its last stage (fp32).
// Then the online LSE (device_common.h) consumes the RT x CT tiles.
// Units: 1 KiB operand units of the packed layout; KU units per k-block
// (3 in split mode, 2 in half2 mode), kbp units per tile, padded to whole
// stages.
// ---------------------------------------------------------------------------
template <int MODE>
constexpr int wide_ku() { return units_per_kblock<MODE>(); }

template <int MODE, int CT, int BK>
constexpr int wide_stage_elems() { return CT * BK * wide_ku<MODE>() * 64; }

template <int MODE, int CT, int BK>
constexpr int wide_loads() { return (wide_stage_elems<MODE, CT, BK>() + 255) / 256; }

template <int MODE, int RT, int CT, int BK>
__global__ __launch_bounds__(256) void lse_wide_kernel(
    const u32x4* __restrict__ Rp, const u32x4* __restrict__ Cp, const float* __restrict__ cbias,
    int rtiles, int ctiles, int kbp, int splits, int bps, int nrowgroups, float c,
    float2* __restrict__ part, int rpad) {
  constexpr int KU = wide_ku<MODE>();
  constexpr int SU = BK * KU;               // units per tile per stage
  constexpr int NX = 4 * RT;                // row tiles of the workgroup
  constexpr int NL = wide_loads<MODE, CT, BK>();
  __shared__ u32x4 lds[KU == 1 ? 3 : 2][NL * 256];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  // Workgroups are dispatched round-robin over the 8 XCDs. Workgroup w runs
  // on XCD w % 8; the XCD's workgroups are ordered split-fastest over row
  // groups xcd, xcd + 8, ..., so the few row blocks in flight on an XCD (each
  // re-read once per column block) stay in its L2.
  const int xcd = blockIdx.x & 7;
  const int li = blockIdx.x >> 3;
  const int s = li % splits;
  const int rg = (li / splits) * 8 + xcd;
  if (rg >= nrowgroups) return;             // whole workgroup: no barrier is skipped
  const int rt0 = rg * NX;                  // first row tile of the workgroup
  const int nblocks = (ctiles + CT - 1) / CT;
  const int b0 = s * bps;
  const int nb = min(b0 + bps, nblocks) - b0;  // >= 1 by construction of the split
  const int nstages = kbp / SU;             // per column block
  const int total = nb * nstages;
  const float ks = MODE == kModeBF16 ? c : 1.0f;
  const uint2* __restrict__ cb3 = bias_parts(cbias, ctiles * kTile);
  const BiasOp<MODE> sent = sentinel_bias<MODE>(h);

  // Column staging slots of this thread: column tile cq of the current block,
  // unit offset uo within the stage.
  int cq[NL], uo[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int e = min(tid + 256 * i, wide_stage_elems<MODE, CT, BK>() - 1);
    cq[i] = e / (SU * 64);
    uo[i] = ((e / 64) % SU) * 64 + (e & 63);
  }
  // Loads column stage `step` (clamped to the last one) into registers: branch-free.
  auto gload = [&](int step, u32x4 (&g)[NL]) {
    step = min(step, total - 1);
    const int blk = b0 + step / nstages;
    const size_t koff = (size_t)(step % nstages) * SU * 64;
#pragma unroll
    for (int i = 0; i < NL; ++i)
      g[i] = Cp[(size_t)min(blk * CT + cq[i], ctiles - 1) * kbp * 64 + koff + uo[i]];
  };
  auto sstore = [&](u32x4* buf, const u32x4 (&g)[NL]) {
#pragma unroll
    for (int i = 0; i < NL; ++i) buf[tid + 256 * i] = g[i];
  };
  // This wave's row tiles (clamped; rows past the last tile are computed and
  // never written) and their stage slices, loaded straight into registers.
  const u32x4* xsrc[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r)
    xsrc[r] = Rp + (size_t)min(rt0 + wave * RT + r, rtiles - 1) * kbp * 64 + lane;
  auto rload = [&](int step, u32x4 (&x)[RT][SU]) {
    step = min(step, total - 1);
    const size_t koff = (size_t)(step % nstages) * SU * 64;
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int u = 0; u < SU; ++u) x[r][u] = xsrc[r][koff + u * 64];
  };

  float M[RT], S[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    M[r] = kUnset;
    S[r] = 0.f;
  }
  u32x4 gA[NL], gB[NL];
  u32x4 xA[RT][SU], xB[RT][SU];

  // Products of one k-block: fragments f of the CT column tiles.
  auto kblock = [&](const u32x4 (&f)[CT][KU], const u32x4 (&x)[RT][SU], int kb,
                    f32x16 (&acc)[RT][CT]) {
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int q = 0; q < CT; ++q) {
        if constexpr (MODE == kModeSplit)
          acc[r][q] = mfma_split(f[q], &x[r][kb * KU], acc[r][q]);
        else if constexpr (MODE == kModeHalf2)
          acc[r][q] = mfma_half2(f[q], &x[r][kb * KU], acc[r][q]);
        else
          acc[r][q] = mfma_kblock<MODE == kModeBF16>(f[q][0], x[r][kb], acc[r][q]);
      }
  };
  auto fread = [&](const u32x4* buf, int kb, u32x4 (&f)[CT][KU]) {
#pragma unroll
    for (int q = 0; q < CT; ++q)
#pragma unroll
      for (int u = 0; u < KU; ++u) f[q][u] = buf[(q * SU + kb * KU + u) * 64 + lane];
  };

  // Column block bi: bias minus stabiliser first (from zero; see
  // mfma_bias_stab), then the block's score products accumulate onto it. M
  // moves only in the LSE after the block, so the fold taken here is the one
  // the block uses. After the products: the fp32 modes' bias instruction,
  // then the online LSE.
  auto block_begin = [&](int bi, float (&Mf)[RT], BiasOp<MODE> (&Bst)[RT], BiasOp<MODE> (&aq)[CT],
                         f32x16 (&acc)[RT][CT]) {
    const int blk = b0 + bi;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      Mf[r] = fold_of(M[r]);
      Bst[r] = stab_of<MODE>(Mf[r], h);
    }
#pragma unroll
    for (int q = 0; q < CT; ++q) {
      const int jt = blk * CT + q;
      const BiasOp<MODE> a = load_bias<MODE>(cbias, cb3, min(jt, ctiles - 1), lane);
      aq[q] = jt < ctiles ? a : sent;  // tiles past the end: sentinel bias
#pragma unroll
      for (int r = 0; r < RT; ++r) acc[r][q] = bias_start<MODE>(aq[q], Bst[r]);
    }
  };
  auto block_end = [&](const float (&Mf)[RT], const BiasOp<MODE> (&Bst)[RT],
                       const BiasOp<MODE> (&aq)[CT], f32x16 (&acc)[RT][CT]) {
#pragma unroll
    for (int q = 0; q < CT; ++q)
#pragma unroll
      for (int r = 0; r < RT; ++r) acc[r][q] = bias_finish<MODE>(aq[q], Bst[r], h, acc[r][q]);
#pragma unroll
    for (int q = 0; q < CT; ++q) {
      f32x16 col[RT];
#pragma unroll
      for (int r = 0; r < RT; ++r) col[r] = acc[r][q];
      lse_tail<MODE, RT, false>(col, Mf, M, S, ks);
    }
  };

  if constexpr (KU == 1) {
    // One unit per k-block (bf16 points, fp32 MFMA): three column buffers in
    // LDS. Stage t reads buffer t % 3 and, ahead of its own end, the first
    // k-block of stage t + 1 from buffer (t + 1) % 3, which every wave
    // stored before the barrier ending stage t - 1. At the end of stage t the
    // columns of stage t + 2 go to buffer (t + 2) % 3, last read in stage
    // t - 1. One barrier per stage covers both hazards, and no stage starts
    // by waiting on LDS reads (c4: 4.81 -> 4.61 ms per pass). Column loads:
    // stage t + 2's arrive in one register set (issued at the start of stage
    // t - 1), stage t + 3's load is issued at the start of stage t. Row
    // slices: stage t's in set t & 1, refilled with stage t + 2's once read.
    // The two-unit modes keep the double buffer below: their next-stage
    // fragments do not fit the register budget.
    u32x4 fc[CT][KU];  // fragments of the next k-block to multiply
    gload(0, gA);
    gload(1, gB);
    rload(0, xA);
    rload(1, xB);
    sstore(lds[0], gA);
    sstore(lds[1], gB);
    gload(2, gA);
    __syncthreads();
    fread(lds[0], 0, fc);
    auto stage = [&](int step, u32x4 (&x)[RT][SU], u32x4 (&gload_to)[NL],
                     u32x4 (&gstore_from)[NL], f32x16 (&acc)[RT][CT]) {
      gload(step + 3, gload_to);
#pragma unroll
      for (int kb = 0; kb < BK; ++kb) {
        u32x4 fn[CT][KU];
        if (kb + 1 < BK) fread(lds[step % 3], kb + 1, fn);
        else fread(lds[(step + 1) % 3], 0, fn);
        kblock(fc, x, kb, acc);
#pragma unroll
        for (int q = 0; q < CT; ++q) fc[q][0] = fn[q][0];
      }
      rload(step + 2, x);
      sstore(lds[(step + 2) % 3], gstore_from);
      __syncthreads();
    };
    int step = 0;  // even at the top of every stage pair (nstages is even)
    for (int bi = 0; bi < nb; ++bi) {
      float Mf[RT];
      BiasOp<MODE> Bst[RT], aq[CT];
      f32x16 acc[RT][CT];
      block_begin(bi, Mf, Bst, aq, acc);
      for (int st = 0; st < nstages; st += 2, step += 2) {
        stage(step, xA, gB, gA, acc);      // stage step + 2's columns were in gA
        stage(step + 1, xB, gA, gB, acc);  // stage step + 3's in gB
      }
      block_end(Mf, Bst, aq, acc);
    }
  } else {
    // Two column staging sets and a double buffer: the load of stage t is
    // issued at the start of stage t - 2 and stored to LDS at the end of
    // stage t - 1, so it has two stages of matrix work to arrive. Row slices:
    // set A holds the even stages, set B the odd ones; each is refilled once
    // its stage has been computed. nstages is even (padded by the host).
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
            if constexpr (MODE == kModeSplit)
              acc[r][q] = mfma_split(yf[q], &x[r][kb * KU], acc[r][q]);
            else if constexpr (MODE == kModeHalf2)
              acc[r][q] = mfma_half2(yf[q], &x[r][kb * KU], acc[r][q]);
            else
              acc[r][q] = mfma_kblock<MODE == kModeBF16>(yf[q][0], x[r][kb], acc[r][q]);
          }
      }
    };
    int step = 0;  // even at the top of every stage pair
    for (int bi = 0; bi < nb; ++bi) {
      const int blk = b0 + bi;
      float Mf[RT];
      BiasOp<MODE> Bst[RT], aq[CT];
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        Mf[r] = fold_of(M[r]);
        Bst[r] = stab_of<MODE>(Mf[r], h);
      }
      f32x16 acc[RT][CT];
#pragma unroll
      for (int q = 0; q < CT; ++q) {
        const int jt = blk * CT + q;
        const BiasOp<MODE> a = load_bias<MODE>(cbias, cb3, min(jt, ctiles - 1), lane);
        aq[q] = jt < ctiles ? a : sent;
#pragma unroll
        for (int r = 0; r < RT; ++r) acc[r][q] = bias_start<MODE>(aq[q], Bst[r]);
      }
      for (int st = 0; st < nstages; st += 2, step += 2) {
        // stage `step`: columns in lds[0], rows in xA; gB / xB hold stage step + 1
        gload(step + 2, gA);
        compute(lds[0], xA, acc);
        rload(step + 2, xA);
        sstore(lds[1], gB);  // lds[1] was last read in stage step - 1
        __syncthreads();
        // stage step + 1: columns in lds[1], rows in xB; gA / xA hold stage step + 2
        gload(step + 3, gB);
        compute(lds[1], xB, acc);
        rload(step + 3, xB);
        sstore(lds[0], gA);  // after the final stage nobody reads these stores
        __syncthreads();
      }
      block_end(Mf, Bst, aq, acc);
    }
  }

#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const float St = S[r] + __shfl_xor(S[r], 32);
    const int rt = rt0 + wave * RT + r;
    if (h == 0 && rt < rtiles)
      part[(size_t)s * rpad + (size_t)rt * kTile + (lane & 31)] = make_float2(ks * M[r], St);
  }
}

template <int MODE, int RT, int CT, int BK>
static void lse_wide_go(const PassShape& s, const void* Rp, const void* Cp, const float* cbias,
                        float c, float2* part, hipStream_t st, const LaunchTimer* t) {
  // Row groups padded to a multiple of 8 (one slice per XCD); padding
  // workgroups exit at once.
  const int grid = (s.nrowgroups + 7) / 8 * 8 * s.splits;
  launch_timed(lse_wide_kernel<MODE, RT, CT, BK>, dim3(grid), dim3(256), st, t,
               (const u32x4*)Rp, (const u32x4*)Cp, cbias, s.rtiles, s.ctiles, s.kbp, s.splits,
               s.tps, s.nrowgroups, c, part, s.rtiles * kTile);
}

hipError_t launch_lse_wide(const PassShape& s, int mode, const void* Rp, const void* Cp,
                           const float* cbias, float c, float2* part, hipStream_t st,
                           const LaunchTimer* t) {
  if (s.xres) return hipErrorInvalidValue;
#define WIDE_CASE(M, R, C, K)                                                   \
  if (mode == M && s.ri == R && s.ct == C && s.bk == K) {                      \
    lse_wide_go<M, R, C, K>(s, Rp, Cp, cbias, c, part, st, t);                 \
    return hipGetLastError();                                                   \
  }
  // Shapes measured best on gfx950 among RT in {2, 4}, CT in {2, 4},
  // BK in {1, 2, 4} (larger ones exceed 256 VGPRs or starve LDS / L2).
  WIDE_CASE(kModeSplit, 2, 4, 1)
  WIDE_CASE(kModeHalf2, 2, 4, 1)
  WIDE_CASE(kModeHalf2, 2, 4, 2)
  WIDE_CASE(kModeBF16, 2, 4, 2)
  WIDE_CASE(kModeF32, 2, 4, 2)
#undef WIDE_CASE
  return hipErrorInvalidValue;
}

}  // namespace flashot
