// Internal interface between the host drivers (api.hip, hvp_api.hip) and the
// gfx950 kernels (kernels.hip, kernels_wide.hip, apply_kernels.hip,
// aux_kernels.hip, hvp_kernels.hip). Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace flashot {

// Every packed operand is a sequence of 32-row tiles. A tile holds `kbp`
// k-blocks of 1 KiB: 64 lanes x 16 bytes. Lane l of k-block kb carries row
// (l % 32) and the (l / 32)-th half of the block's k range, i.e. 4 fp32
// (k-block = 8 values of the dimension) or 8 bf16 (k-block = 16 values).
// Rows past the end and dimensions past d are zero.
constexpr int kTile = 32;
constexpr int kWaves = 4;  // waves per workgroup of the streamed kernels
constexpr float kSentinel = -1.0e20f;  // bias of padded columns: exp underflows to 0
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Operand modes of the streamed passes.
constexpr int kModeF32 = 0;    // fp32 operands, fp32 MFMA (32x32x2)
constexpr int kModeBF16 = 1;   // bf16 operands, bf16 MFMA (32x32x16)
constexpr int kModeSplit = 2;  // fp32 operands as hi + mid + lo bf16 parts, bf16 MFMA
constexpr int kModeHalf2 = 3;  // fp32 operands as hi + lo fp16 parts, fp16 MFMA

// Shape of one streamed pass: "rows" are the outputs (one LSE per row) and
// "cols" are streamed. For the f half-step rows = x, cols = y.
struct PassShape {
  int rtiles, ctiles;   // 32-row tiles of the row and column operands
  int kbp;              // k-blocks per tile (padded)
  int kb;               // k-blocks held in registers at a time (1,2,4,8,16)
  bool xres;            // row operand resident in registers (kbp == kb)
  bool lds;             // resident pass with the column tile shared through LDS
  int ri;               // 32-row tiles per wave
  int ct, bk;           // wide pass: column tiles per block, k-blocks per stage
  int splits, tps;      // column splits and column tiles (wide pass: blocks) per split
  int nrowgroups;       // workgroups along the rows
  int solo;             // small problem: the half-step may run as one launch (launch_lse_solo)
};
// Waves per workgroup of the single-launch half-step (launch_lse_solo).
constexpr int kSoloWaves = 4;

hipError_t launch_sqnorms(const void* pts, int bf16, int64_t rows, int64_t d, int64_t ld,
                          float* out, hipStream_t st);
hipError_t launch_pack_points(const void* src, int bf16, int64_t rows, int64_t d, int64_t ld,
                              int rtiles, int kbp, float scale, void* dst, hipStream_t st);
// Packs fp32 points (times `scale`) as three bf16 parts hi, mid, lo per
// k-block of 16 values: units (3 kb, 3 kb + 1, 3 kb + 2) of a tile hold the
// parts of k-block kb in the lane layout of a bf16 k-block.
hipError_t launch_pack_split(const float* src, int64_t rows, int64_t d, int64_t ld, int rtiles,
                             int units, float scale, void* dst, hipStream_t st);
// Range plan of the half2 operand mode (two fp16 parts per fp32 value):
// the largest |x| and |y| (float bits), the exact factors 2^a, 2^-a applied
// to X and Y, whether both clouds fit fp16 with them, and the per-block
// maxima it is reduced from.
constexpr int kHalf2Parts = 1024;
struct Half2Plan {
  unsigned amax[2];
  float xmul, ymul;
  int ok;
  int pad[3];
  unsigned part[2 * kHalf2Parts];
};
// Computes the plan from X, Y (fp32) and the factor cx that X is packed with.
hipError_t launch_half2_plan(const float* X, int64_t n, int64_t ldx, const float* Y, int64_t m,
                             int64_t ldy, int64_t d, float cx, Half2Plan* plan, hipStream_t st);
// Packs fp32 points times scale * (side ? ymul : xmul) as hi, lo fp16 parts:
// units (2 kb, 2 kb + 1) of a tile hold k-block kb in the lane layout of a
// bf16 k-block. X (side 0) is written as NaN when the plan is out of range.
hipError_t launch_pack_half2(const float* src, int64_t rows, int64_t d, int64_t ld, int rtiles,
                             int units, float scale, const Half2Plan* plan, int side, void* dst,
                             hipStream_t st);
// Value columns of the fp16 value product are scaled by 2^b, b from the
// column's largest |v| (float bits), so that they lie in [2^14, 2^15); b = 0
// for an all-zero or non-finite column. Shared by packing and merge.
__host__ __device__ inline int vcol_shift(unsigned amax_bits) {
  const int eb = (int)((amax_bits >> 23) & 0xff);
  if (amax_bits == 0 || eb == 255) return 0;
  const int b = 141 - (eb > 0 ? eb : 1);
  return b < -100 ? -100 : (b > 100 ? 100 : b);
}
// Column maxima |V[:, p]| (float bits) into amax[0, cols), which is zeroed first.
hipError_t launch_vcol_absmax(const void* V, int bf16, int64_t rows, int64_t cols, int64_t ldv,
                              unsigned* amax, hipStream_t st);
// Packs V (rows streamed x cols) for the fp16 value product: per column tile
// jt, value block pb, k-chunk q (16 streamed rows) and part (hi, lo of
// V[j][p] 2^b_p), lane l holds the 8 fp16 values of column 32 pb + l % 32 and
// rows 32 jt + 8 (2q + e/4) + 4 (l/32) + e%4, e = 0..7 -- the order in which
// a lane's score accumulator entries 8q .. 8q + 7 enter the matrix product.
hipError_t launch_pack_values_h2(const void* V, int bf16, int64_t rows, int64_t cols,
                                 int64_t ldv, int ctiles, int pblocks, const unsigned* amax,
                                 void* dst, hipStream_t st);
// Transport application with the exponentiated scores split into two fp16
// parts against the fp16 value layout (three products per 16 streamed rows).
// smode: kModeHalf2 (fp32 points, scores in log2 units, c = 1), kModeBF16 or
// kModeF32 (fp32 operands, dot-product units, times c). cbias: a column-bias
// buffer with the bias-MFMA parts (bias_buffer_bytes) for kModeHalf2 and
// kModeBF16, fp32 biases alone for kModeF32. Partial stabilisers are written
// in log2 units (merge with c = 1).
// Column tiles per block of the wide transport application; its passes need
// the column tiles per split (PassShape::tps) to be a multiple of it.
constexpr int kApplyWideCT = 4;
// vparts: fp16 parts of each value the product uses, 2 (hi and lo: fp32
// values) or 1 (hi alone: bf16 values, whose lo part in the layout is always
// zero); kModeF32 scores always take both.
hipError_t launch_apply_stream(const PassShape& s, int smode, int pblocks, int pb_per_pass,
                               int vparts, const void* Rp, const void* Cp, const float* cbias,
                               const void* Vh, float c, float2* partMS, float* partO, int ppad,
                               hipStream_t st);
hipError_t launch_pack_values(const void* V, int bf16, int64_t rows, int64_t cols, int64_t ldv,
                              int ctiles, int pblocks, float* dst, hipStream_t st);
hipError_t launch_weights(const float* w, int rows, int rpad, float eps, float* wgt, float* hlw,
                          hipStream_t st);
hipError_t launch_fill(float* p, float v, int64_t count, hipStream_t st);
// Column-bias buffers of the log-sum-exp passes hold rpad fp32 biases followed
// by the operand of the bias MFMA: per 32-column tile, 64 entries of 8 bytes
// (one per lane). Entry l < 32 holds the three bf16 parts of the bias of
// column l of the tile (bits: part1 | part2 << 16, part3); entries 32..63
// hold three bf16 ones. A buffer that feeds only transport applications
// needs the fp32 biases alone.
inline size_t bias_buffer_bytes(int rpad) { return (size_t)rpad * 4 + (size_t)(rpad / kTile) * 512; }
__host__ __device__ inline const uint2* bias_parts(const float* bias, int rpad) {
  return reinterpret_cast<const uint2*>(bias + rpad);
}
constexpr uint32_t kBf16OnesLo = 0x3F803F80u;  // bf16 1.0, 1.0
constexpr uint32_t kBf16OnesHi = 0x00003F80u;  // bf16 1.0, 0
// bf16 rounding (to nearest, ties to even) of an fp32 value, as bits; NaN
// stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_bits_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
// v as three bf16 parts p1 + p2 + p3 (each the rounding of what the previous
// ones left); for normal fp32 v the sum is exact. Packed as (p1 | p2 << 16, p3).
// No contraction: a product that produced v must not be fused into the first
// remainder, or the parts would describe the unrounded product instead of the
// stored v (and differ between kernels that compute v the same way).
__device__ __forceinline__ uint2 bf16x3_parts(float v) {
#pragma clang fp contract(off)
  const uint32_t b1 = bf16_bits_rne(v);
  const float r1 = v - __uint_as_float(b1 << 16);
  const uint32_t b2 = bf16_bits_rne(r1);
  const float r2 = r1 - __uint_as_float(b2 << 16);
  return make_uint2(b1 | (b2 << 16), bf16_bits_rne(r2));
}
// Bias-MFMA operand of column i of a bias buffer of rpad columns: the parts
// of its bias in lane i % 32 of its tile, three bf16 ones in lane 32 + i % 32.
__device__ __forceinline__ void write_bias_parts(float* bias, int rpad, int i, float v) {
  uint2* parts = reinterpret_cast<uint2*>(bias + rpad);
  const size_t at = (size_t)(i / kTile) * 64 + (i % kTile);
  parts[at] = bf16x3_parts(v);
  parts[at + kTile] = make_uint2(kBf16OnesLo, kBf16OnesHi);
}
// End of a half-step for one row, shared by the merge of split partials and
// the single-launch small pass ("FlashSinkhorn: IO-Aware Entropic Optimal
// Transport on GPU", App. D.1-D.2: the potential is written once; App. E.1:
// the induced marginal of the previous iterate). From the row's merged
// (M in log2 units, S):
//   h_i = norm_i - eps ln2 (M + log2 S)            (the half-step value),
//   pot_i = h_i, or (pot_old_i + h_i) / 2 when avg (symmetric schedule),
//   next bias_i = bscale ((pot_i - norm_i) / 2 + hlw_i) with its MFMA operand,
// written only when write_pot; returns w_i |exp((pot_old_i - h_i)/eps) - 1|
// when with_err, else 0. bscale = 2 log2(e)/eps when the streamed kernels
// work in log2 units, 1 in dot-product units. Rows rows..rpad-1 of a written
// bias buffer hold the sentinel (finish_pad_row).
struct RowFinish {
  float bscale, eps;
  const float* norm;
  const float* hlw;
  const float* wgt;
  float* pot;
  float* bias_out;
  int rows, rpad, with_err, write_pot, avg;
};
// The row's inputs of finish_row, loaded ahead of the reduction that feeds it.
struct RowIn {
  float nrm, hlw, wgt, pold;
};
__device__ __forceinline__ RowIn load_row_in(const RowFinish& r, int i) {
  RowIn in;
  in.nrm = r.norm[i];
  in.hlw = r.write_pot ? r.hlw[i] : 0.f;
  in.wgt = r.with_err ? r.wgt[i] : 0.f;
  in.pold = (r.with_err || r.avg) ? r.pot[i] : 0.f;
  return in;
}
__device__ __forceinline__ float finish_row(const RowFinish& r, int i, float M, float S,
                                            const RowIn& in) {
  const float shifted = -r.eps * kLn2 * (M + log2f(S));
  const float half = in.nrm + shifted;
  float e = 0.f;
  if (r.with_err) e = in.wgt * fabsf(exp2f((in.pold - half) * (kLog2e / r.eps)) - 1.f);
  const float pnew = r.avg ? 0.5f * (in.pold + half) : half;
  if (r.write_pot) {
    r.pot[i] = pnew;
    const float v = r.bscale * (0.5f * (pnew - in.nrm) + in.hlw);
    r.bias_out[i] = v;
    write_bias_parts(r.bias_out, r.rpad, i, v);
  }
  return e;
}
__device__ __forceinline__ void finish_pad_row(const RowFinish& r, int i) {
  if (r.write_pot) {
    r.bias_out[i] = kSentinel;
    write_bias_parts(r.bias_out, r.rpad, i, kSentinel);
  }
}
// parts = 1: also write the bias-MFMA operand after the rpad biases (the
// buffer then has bias_buffer_bytes(rpad) bytes).
hipError_t launch_bias_from_pot(const float* pot, const float* norm, const float* hlw, int rows,
                                int rpad, float bscale, float* bias, int parts, hipStream_t st);
// mode: 0 fp32 operands, 1 bf16 operands, 2 fp32 operands packed as three bf16 parts,
// 3 fp32 operands packed as two fp16 parts.
// Register-resident passes (s.xres, kernels.hip) and k-chunked wide passes (kernels_wide.hip).
// Per-launch timing: when a LaunchTimer is given, the kernel is launched with
// hipExtLaunchKernelGGL, whose dispatch records its own start and end into
// the two events, so no separate event commands sit between launches.
struct LaunchTimer {
  hipEvent_t start;
  hipEvent_t stop;
};
hipError_t launch_lse_resident(const PassShape& s, int mode, const void* Rp, const void* Cp,
                               const float* cbias, float c, float2* part, hipStream_t st,
                               const LaunchTimer* timer = nullptr);
// Transport-vector pass (P v, one value column) on the register-resident
// layouts: (M, S) partials as launch_lse_resident plus T = sum exp2(score -
// M) v per split and row in partT. vcol: the column side's values, padded
// with zeros to whole tiles.
hipError_t launch_vec_resident(const PassShape& s, int mode, const void* Rp, const void* Cp,
                               const float* cbias, const float* vcol, float c, float2* part,
                               float* partT, hipStream_t st);
hipError_t launch_lse_wide(const PassShape& s, int mode, const void* Rp, const void* Cp,
                           const float* cbias, float c, float2* part, hipStream_t st,
                           const LaunchTimer* timer = nullptr);
// Single-launch half-step of a small problem (s.solo; modes 1 and 3, row
// operand resident, per-wave column loads): one workgroup of kSoloWaves
// waves per 32-row tile, the waves splitting the column tiles; the waves' partials
// are merged in a fixed order on chip and the row end (finish_row) follows
// in the same launch. err_part receives one weighted marginal-error sum per
// row tile (as launch_lse_merge's per-block sums, lse_merge_blocks(rpad) of
// them) when fin.with_err. Not for the symmetric schedule, whose second pass
// must read the biases this one overwrites.
hipError_t launch_lse_solo(const PassShape& s, int mode, const void* Rp, const void* Cp,
                           const float* cbias, float c, const RowFinish& fin, float* err_part,
                           hipStream_t st, const LaunchTimer* timer = nullptr);
// Whether launch_lse_solo serves this shape and mode.
bool lse_solo_supported(const PassShape& s, int mode);
inline hipError_t launch_lse_partial(const PassShape& s, int mode, const void* Rp, const void* Cp,
                                     const float* cbias, float c, float2* part, hipStream_t st,
                                     const LaunchTimer* timer = nullptr) {
  return s.xres ? launch_lse_resident(s, mode, Rp, Cp, cbias, c, part, st, timer)
                : launch_lse_wide(s, mode, Rp, Cp, cbias, c, part, st, timer);
}
// avg = 1: symmetric schedule, the new potential is the average of the old
// one and the half-step value. With write_pot, bias_out receives the biases
// and the bias-MFMA operand (bias_buffer_bytes(rpad) bytes).
hipError_t launch_lse_merge(const float2* part, int splits, int rpad, int rows, float bscale, float eps,
                            const float* norm, const float* hlw, const float* wgt, float* pot,
                            float* bias_out, float* err_part, int with_err, int write_pot,
                            int avg, hipStream_t st);
int lse_merge_blocks(int rows);
// Sinkhorn divergence from three potential pairs: out = [S, OT(mu, nu),
// OT(mu, mu), OT(nu, nu)], dual values summed in fp64 (a, b NULL: uniform).
hipError_t launch_dual_values(const float* a, const float* b, int n, int m, const float* f,
                              const float* g, const float* fxx, const float* gxx, const float* fyy,
                              const float* gyy, float* out, hipStream_t st);
hipError_t launch_err_reduce(const float* part, int count, float* out, hipStream_t st);
hipError_t launch_nonfinite(const float* f, int n, const float* g, int m, float* out,
                            hipStream_t st);
hipError_t launch_apply_partial(const PassShape& s, int bf16, int pblocks, int pb_per_pass,
                                const void* Rp, const void* Cp, const float* cbias,
                                const float* Vp, float c, float2* partMS, float* partO, int ppad,
                                hipStream_t st);
// Hadamard-weighted transport (P . A Y^T) V (fp32 operands): Ap holds the rows
// of A packed like Rp.
hipError_t launch_apply_hadamard(const PassShape& s, int pblocks, int pb_per_pass, const void* Rp,
                                 const void* Cp, const void* Ap, const float* cbias,
                                 const float* Vp, float c, float2* partMS, float* partO, int ppad,
                                 hipStream_t st);
// c: the partials' stabilisers are in units of c * M log2 units (c = 1:
// log2 units). vamax (or NULL): column maxima of the fp16 value layout, whose
// 2^b_p scale is removed.
hipError_t launch_apply_merge(const float2* partMS, const float* partO, int splits, int rpad,
                              int ppad, int rows, int cols, float c, float eps, const float* pot,
                              const float* norm, const float* wgt, int mode, const void* Xsrc,
                              int xbf16, int64_t ldx, const unsigned* vamax, float* out,
                              float* marg, hipStream_t st);

// apply_merge modes
constexpr int kApplyPlain = 0;
constexpr int kApplyBary = 1;
constexpr int kApplyGrad = 2;

// ---- Hessian-vector product (hvp_kernels.hip) ------------------------------------
// Conjugate-gradient state in device memory (scalars of the recurrence and
// the stop flags), so that iterations need no host round trip.
struct CgState {
  float rr;      // ||res||^2
  float bb;      // ||rhs||^2
  float alpha;
  float beta;
  int iters;     // iterations completed
  int breakdown; // non-positive curvature met
  int done;      // converged, broke down, or zero right side
  int pad;
};
constexpr int kCgMaxParts = 256;  // partial sums per reduction
int cg_parts(int len);
hipError_t launch_hvp_prep(int n, int d, const float* X, int64_t ldx, const float* A, int64_t lda,
                           const float* PY, const float* r, float* xa, float* ra1, float* VB,
                           hipStream_t st);
hipError_t launch_hvp_rhs(int m, int d, const float* Y, int64_t ldy, const float* PTV, float* rhs,
                          float* w2, float* res, float* pdir, hipStream_t st);
hipError_t launch_cg_start(int m, const float* rhs, float* part, CgState* cs, hipStream_t st);
hipError_t launch_cg_div(int n, const float* Pp, const float* r, float* u, const CgState* cs,
                         hipStream_t st);
hipError_t launch_cg_update(int m, const float* c, const float* PTu, float tau, float tol,
                            float* pdir, float* q, float* w2, float* res, float* part,
                            CgState* cs, hipStream_t st);
hipError_t launch_hvp_vf(int m, int d, const float* Y, int64_t ldy, const float* w2, float* VF,
                         hipStream_t st);
hipError_t launch_vec_merge(const float2* part, const float* partT, int splits, int rpad,
                            int rows, float eps, const float* pot, const float* norm,
                            const float* wgt, float* out, hipStream_t st);
hipError_t launch_hvp_final(int n, int d, float eps, const float* X, int64_t ldx, const float* A,
                            int64_t lda, const float* PY, const float* r, const float* xa,
                            const float* ra1, const float* PF, const float* B5, float* out,
                            hipStream_t st);

}  // namespace flashot
