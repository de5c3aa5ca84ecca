// C ABI and host driver of the streamed Sinkhorn solver (declarations and
// semantics in include/flashot.h).
//
// The driver validates arguments on the host, carves the caller's workspace,
// packs both point clouds once per call into the MFMA operand layout, and
// enqueues one f half-step (streamed LSE partials + merge) and one g
// half-step per iteration on the caller's stream (alternating schedule of
// "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU", §3.1 eq. 2-3).
// Blocks of iterations are captured once into a HIP graph and replayed.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "flashot.h"
#include "host_common.h"
#include "kernels.h"

using namespace flashot;

namespace flashot {
namespace host {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}


// fp32 operand mode of a problem: two fp16 parts per value by default, three
// bf16 parts (OT_SPLIT_BF16) or fp32 MFMA (OT_NATIVE_F32) on request.
int f32_operand_mode(int32_t flags) {
  if (flags & OT_NATIVE_F32) return kModeF32;
  return (flags & OT_SPLIT_BF16) ? kModeSplit : kModeHalf2;
}

// Operand layout and pass shape for a point dimension / storage type.
//  - fp32 points (f32_mode: kModeHalf2, kModeSplit or kModeF32) use the
//    requested split, or fp32 operands;
//  - d <= 128 (split or native fp32) / 256 bf16: register-resident rows; the
//    three-part split keeps one row tile per wave above d = 64 (24 KiB of
//    row operand in registers), the two-part split two (16 KiB each);
//  - wider: the tiled pass (column blocks of ct tiles, LDS stages of bk
//    k-blocks), with the units per tile padded to whole stages.
// Transport application keeps its own layout (for_apply): fp32 or bf16
// operands, chunks of 8 k-blocks when the row operand is not resident.
KConf kernel_conf(int64_t d, int bf16, int f32_mode, bool for_apply) {
  KConf k{};
  if (for_apply && !bf16 && f32_mode == kModeHalf2) {
    // transport application on two fp16 parts: resident rows up to d = 128,
    // else chunks of 4 k-blocks (8 units)
    k.mode = kModeHalf2;
    k.kbw = 16;
    k.kblocks = ceil_div(d, 16);
    int kl = 1;
    while (kl < k.kblocks) kl *= 2;
    k.xres = k.kblocks <= 8;
    k.kb = k.xres ? 2 * kl : 8;
    k.kbp = k.xres ? k.kb : ceil_div(k.kblocks, 4) * 8;
    k.ri = 1;
    return k;
  }
  const bool split = !bf16 && f32_mode != kModeF32 && !for_apply;
  const int ku = !split ? 1 : (f32_mode == kModeSplit ? 3 : 2);  // units per k-block
  if (split && d <= 128) {
    k.mode = f32_mode;
    k.kbw = 16;
    k.kblocks = ceil_div(d, 16);
    int kl = 1;
    while (kl < k.kblocks) kl *= 2;
    k.kb = ku * kl;
    k.kbp = k.kb;
    k.xres = true;
    if (f32_mode == kModeHalf2) {
      // two row tiles per wave; per-wave column loads up to d = 64, columns
      // through LDS above (measured best on gfx950)
      k.lds = k.kb >= 16;
      k.ri = 2;
    } else {
      k.lds = k.kb >= 12;
      k.ri = k.kb <= 12 ? 2 : 1;
    }
  } else {
    k.mode = split ? f32_mode : (bf16 ? 1 : 0);
    k.kbw = (bf16 || split) ? 16 : 8;
    k.kblocks = ceil_div(d, k.kbw);
    if (!split && k.kblocks <= 16) {
      k.kb = 1;
      while (k.kb < k.kblocks) k.kb *= 2;
      k.kbp = k.kb;
      k.xres = true;
      // Wide fp32 tiles: share the column tile through LDS, which leaves room
      // for two resident row tiles per wave.
      k.lds = !bf16 && k.kb >= 8;
      k.ri = (k.kb <= 8 || k.lds) ? 2 : 1;
    } else if (for_apply) {
      k.kb = 8;
      k.kbp = (k.kblocks + 7) / 8 * 8;
      k.xres = false;
      k.ri = 1;
    } else {
      k.ri = 2;
      k.ct = 4;
      k.bk = k.mode == kModeSplit ? 1 : 2;
      k.kb = k.bk * ku;
      k.kbp = ceil_div(k.kblocks, 2 * k.bk) * 2 * k.bk * ku;  // an even number of stages
      k.xres = false;
    }
  }
  return k;
}

// Column splits: enough workgroups to fill 256 CUs several times over
// (`target` workgroups, and at least `min_splits` splits), at least ~4
// column units (tiles, or blocks of the wide pass) per split, a multiple of 8
// when large (XCD locality).
void choose_splits(PassShape& s, int cunits, int forced, int max_splits, int target,
                   int min_splits) {
  int S;
  if (forced > 0) {
    S = forced;
  } else {
    S = ceil_div(target, s.nrowgroups);
    if (S < min_splits) S = min_splits;
    const int most = cunits / 4 > 1 ? cunits / 4 : 1;
    if (S > most) S = most;
    if (S >= 8) S = (S + 7) / 8 * 8;
  }
  if (S > max_splits) S = max_splits;
  if (S > cunits) S = cunits;
  if (S < 1) S = 1;
  s.tps = ceil_div(cunits, S);
  s.splits = ceil_div(cunits, s.tps);
}

PassShape make_pass(int rtiles, int ctiles, const KConf& k, int ri, int forced, int max_splits,
                    int target, int min_splits) {
  PassShape s{};
  s.rtiles = rtiles;
  s.ctiles = ctiles;
  s.kbp = k.kbp;
  s.kb = k.kb;
  s.xres = k.xres;
  s.lds = k.lds;
  s.ri = ri;
  s.ct = k.ct;
  s.bk = k.bk;
  s.nrowgroups = ceil_div(rtiles, (int64_t)kWaves * ri);
  const int cunits = (k.xres || k.ct == 0) ? ctiles : ceil_div(ctiles, k.ct);
  choose_splits(s, cunits, forced, max_splits, target, min_splits);
  return s;
}

int check_problem(const ot_problem* p) {
  if (!p) return fail(OT_ERR_INVALID_ARG, "problem is NULL");
  if (!p->x || !p->y) return fail(OT_ERR_INVALID_ARG, "x or y is NULL");
  if (p->n < 1 || p->m < 1) return fail(OT_ERR_INVALID_ARG, "n and m must be >= 1");
  if (p->d < 1) return fail(OT_ERR_INVALID_ARG, "d must be >= 1");
  if (p->ldx < p->d || p->ldy < p->d) return fail(OT_ERR_INVALID_ARG, "ldx and ldy must be >= d");
  if (p->dtype != OT_F32 && p->dtype != OT_BF16) return fail(OT_ERR_UNSUPPORTED, "dtype must be OT_F32 or OT_BF16");
  if (p->flags & ~(OT_NATIVE_F32 | OT_COST_AFFINE | OT_SPLIT_BF16))
    return fail(OT_ERR_INVALID_ARG, "unknown problem flag");
  if ((p->flags & OT_NATIVE_F32) && (p->flags & OT_SPLIT_BF16))
    return fail(OT_ERR_INVALID_ARG, "OT_NATIVE_F32 and OT_SPLIT_BF16 are exclusive");
  if ((p->flags & OT_COST_AFFINE) && (!p->x_sqn || !p->y_sqn))
    return fail(OT_ERR_INVALID_ARG, "OT_COST_AFFINE needs x_sqn (alpha) and y_sqn (beta)");
  if (p->d > OT_MAX_D) return fail(OT_ERR_UNSUPPORTED, "d exceeds OT_MAX_D");
  if (p->n > (int64_t)1 << 30 || p->m > (int64_t)1 << 30) return fail(OT_ERR_UNSUPPORTED, "n or m exceeds 2^30");
  if (!(p->eps > 0.f) || !std::isfinite(p->eps)) return fail(OT_ERR_INVALID_ARG, "eps must be finite and > 0");
  const float c = 2.f * kLog2e / p->eps;
  if (!std::isfinite(c)) return fail(OT_ERR_UNSUPPORTED, "eps too small: 2 log2(e)/eps overflows fp32");
  const size_t es = p->dtype == OT_BF16 ? 2 : 4;
  if (((uintptr_t)p->x % es) || ((uintptr_t)p->y % es)) return fail(OT_ERR_INVALID_ARG, "x or y misaligned for its dtype");
  return OT_OK;
}

int check_ws(void* ws, size_t* ws_bytes, size_t need, bool* query) {
  if (!ws_bytes) return fail(OT_ERR_INVALID_ARG, "ws_bytes is NULL");
  if (!ws) {
    *ws_bytes = need;
    *query = true;
    return OT_OK;
  }
  *query = false;
  if (*ws_bytes < need) return fail(OT_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes");
  if ((uintptr_t)ws % 256) return fail(OT_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return OT_OK;
}

const char* last_error() { return g_err.c_str(); }

int check_half2_range(const Half2Plan* plan, hipStream_t st) {
  int ok = 0;
  OT_HIP(hipMemcpyAsync(&ok, &plan->ok, sizeof(int), hipMemcpyDeviceToHost, st));
  OT_HIP(hipStreamSynchronize(st));
  if (!ok)
    return fail(OT_ERR_UNSUPPORTED,
                "fp32 coordinates too large for the two-part fp16 scores "
                "((2/eps) log2(e) max|x| max|y| at or above 2^29); OT_SPLIT_BF16 or OT_NATIVE_F32 "
                "cover the fp32 range");
  return OT_OK;
}

}  // namespace host
}  // namespace flashot

namespace {

using namespace flashot::host;

// Workspace of the half-step / solve entry points.
struct SolveWs {
  KConf k;
  int ntiles, mtiles, npad, mpad;
  PassShape F, G;
  size_t o_xp, o_yp, o_nx, o_ny, o_wx, o_hx, o_bx, o_wy, o_hy, o_by, o_part, o_part2, o_errp,
      o_errv, o_plan;
  int errblocks_f, errblocks_g;
  size_t total;
};

// The single-launch half-step serves problems whose passes are too small to
// fill the chip: at most kSoloMaxTiles 32-row tiles on either side and at
// most kSoloMaxWork tile pairs x operand units. Measured on MI355X against
// the best split count, per iteration: it wins up to 2048 x 2048 at d = 64
// fp32 and bf16 d = 128, and at 3000 x 3000 bf16 d = 16; it ties at
// 4096 x 4096 d = 16 fp32 and loses at 4096 x 4096 d = 64.
constexpr int kSoloMaxTiles = 96;
constexpr int64_t kSoloMaxWork = 64 * 64 * 8;
bool solo_fits(const PassShape& s, int mode) {
  return lse_solo_supported(s, mode) && s.rtiles <= kSoloMaxTiles && s.ctiles <= kSoloMaxTiles &&
         (int64_t)s.rtiles * s.ctiles * s.kb <= kSoloMaxWork;
}

// Column splits a half-step runs with: the split count, or, for the
// single-launch pass, the waves that hold column tiles.
int used_splits(const PassShape& s, bool sym) {
  if (!s.solo || sym) return s.splits;
  const int tpw = ceil_div(s.ctiles, kSoloWaves);
  return ceil_div(s.ctiles, tpw);
}

SolveWs solve_layout(const ot_problem* p, int splits_f, int splits_g) {
  SolveWs w{};
  w.k = kernel_conf(p->d, p->dtype == OT_BF16, f32_operand_mode(p->flags));
  w.ntiles = ceil_div(p->n, kTile);
  w.mtiles = ceil_div(p->m, kTile);
  w.npad = w.ntiles * kTile;
  w.mpad = w.mtiles * kTile;
  const int target = w.k.xres ? kTargetWorkgroupsResident : kTargetWorkgroups;
  const int min_splits = w.k.xres ? 1 : kMinSplitsWide;
  w.F = make_pass(w.ntiles, w.mtiles, w.k, w.k.ri, splits_f, 4096, target, min_splits);
  w.G = make_pass(w.mtiles, w.ntiles, w.k, w.k.ri, splits_g, 4096, target, min_splits);
  // Small problems run each half-step as one launch (unless a split count is
  // forced); the split shapes stay valid for the symmetric schedule.
  w.F.solo = splits_f == 0 && solo_fits(w.F, w.k.mode);
  w.G.solo = splits_g == 0 && solo_fits(w.G, w.k.mode);
  w.errblocks_f = lse_merge_blocks(w.npad);
  w.errblocks_g = lse_merge_blocks(w.mpad);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  w.o_xp = take((size_t)w.ntiles * w.k.kbp * 1024);
  w.o_yp = take((size_t)w.mtiles * w.k.kbp * 1024);
  w.o_nx = take((size_t)w.npad * 4);
  w.o_ny = take((size_t)w.mpad * 4);
  w.o_wx = take((size_t)w.npad * 4);
  w.o_hx = take((size_t)w.npad * 4);
  w.o_bx = take(bias_buffer_bytes(w.npad));  // biases + bias-MFMA operand (kernels.h)
  w.o_wy = take((size_t)w.mpad * 4);
  w.o_hy = take((size_t)w.mpad * 4);
  w.o_by = take(bias_buffer_bytes(w.mpad));
  const size_t pf = (size_t)w.F.splits * w.npad, pg = (size_t)w.G.splits * w.mpad;
  w.o_part = take((pf > pg ? pf : pg) * 8);
  w.o_part2 = take(pg * 8);  // g partials of the symmetric schedule (both passes in flight)
  w.o_errp = take((size_t)(w.errblocks_f + w.errblocks_g) * 4);
  w.o_errv = take(64);
  w.o_plan = take(sizeof(Half2Plan));
  w.total = o;
  return w;
}

// Resolved device pointers of one solve / half-step call.
struct Ctx {
  const ot_problem* p;
  SolveWs L;
  char* ws;
  float c, eps;
  // Units of the streamed LSE kernels: fp32 X is packed pre-multiplied by c
  // and biases are written times c, so scores are log2 values (kc = 1); bf16
  // operands stay in dot-product units and the kernel multiplies by kc = c.
  float bscale, kc, xscale;
  const float* nx;
  const float* ny;
  float *wx, *hx, *bx, *wy, *hy, *by, *errp, *errv;
  float2* part;
  float2* part2;
  bool sym;  // symmetric (averaged) schedule
  void *xp, *yp;
  Half2Plan* plan;  // range plan of the half2 operand mode
  float *f, *g;
};

// The eps-dependent constants of a context: score scale c = 2 log2(e) / eps and
// the units of operands and biases.
void set_eps_params(Ctx& x, float eps) {
  x.eps = eps;
  x.c = 2.f * kLog2e / eps;
  const bool bf = x.p->dtype == OT_BF16;
  x.bscale = bf ? 1.f : x.c;
  x.kc = bf ? x.c : 1.f;
  // affine cost: x packed halved (exact), so the score's 2 <x, y> is <x, y>
  x.xscale = (bf ? 1.f : x.c) * ((x.p->flags & OT_COST_AFFINE) ? 0.5f : 1.f);
}

Ctx make_ctx(const ot_problem* p, const SolveWs& L, void* ws, float* f, float* g) {
  Ctx x{};
  x.p = p;
  x.L = L;
  x.ws = (char*)ws;
  set_eps_params(x, p->eps);
  x.xp = x.ws + L.o_xp;
  x.yp = x.ws + L.o_yp;
  x.nx = p->x_sqn ? p->x_sqn : (const float*)(x.ws + L.o_nx);
  x.ny = p->y_sqn ? p->y_sqn : (const float*)(x.ws + L.o_ny);
  x.wx = (float*)(x.ws + L.o_wx);
  x.hx = (float*)(x.ws + L.o_hx);
  x.bx = (float*)(x.ws + L.o_bx);
  x.wy = (float*)(x.ws + L.o_wy);
  x.hy = (float*)(x.ws + L.o_hy);
  x.by = (float*)(x.ws + L.o_by);
  x.part = (float2*)(x.ws + L.o_part);
  x.part2 = (float2*)(x.ws + L.o_part2);
  x.errp = (float*)(x.ws + L.o_errp);
  x.errv = (float*)(x.ws + L.o_errv);
  x.plan = (Half2Plan*)(x.ws + L.o_plan);
  x.f = f;
  x.g = g;
  return x;
}

// The eps-dependent operands: X packed pre-scaled by xscale, and the
// log-weights (eps/2) log a, (eps/2) log b.
int prepare_eps(const Ctx& x, hipStream_t st) {
  const ot_problem* p = x.p;
  const int bf = p->dtype == OT_BF16;
  if (x.L.k.mode == kModeHalf2)
    OT_HIP(launch_pack_half2((const float*)p->x, p->n, p->d, p->ldx, x.L.ntiles, x.L.k.kbp, x.xscale,
                             x.plan, 0, x.xp, st));
  else if (x.L.k.mode == kModeSplit)
    OT_HIP(launch_pack_split((const float*)p->x, p->n, p->d, p->ldx, x.L.ntiles, x.L.k.kbp, x.xscale,
                             x.xp, st));
  else
    OT_HIP(launch_pack_points(p->x, bf, p->n, p->d, p->ldx, x.L.ntiles, x.L.k.kbp, x.xscale, x.xp, st));
  OT_HIP(launch_weights(p->a, (int)p->n, x.L.npad, x.eps, x.wx, x.hx, st));
  OT_HIP(launch_weights(p->b, (int)p->m, x.L.mpad, x.eps, x.wy, x.hy, st));
  return OT_OK;
}

// Norms, packed operands, weights: once per call.
int prepare(const Ctx& x, hipStream_t st) {
  const ot_problem* p = x.p;
  const int bf = p->dtype == OT_BF16;
  if (!p->x_sqn) OT_HIP(launch_sqnorms(p->x, bf, p->n, p->d, p->ldx, (float*)x.nx, st));
  if (!p->y_sqn) OT_HIP(launch_sqnorms(p->y, bf, p->m, p->d, p->ldy, (float*)x.ny, st));
  if (x.L.k.mode == kModeHalf2) {
    // the range plan is taken at the problem's eps, the largest X scale of the call
    OT_HIP(launch_half2_plan((const float*)p->x, p->n, p->ldx, (const float*)p->y, p->m, p->ldy, p->d,
                             x.xscale, x.plan, st));
    const int rc = check_half2_range(x.plan, st);
    if (rc) return rc;
    OT_HIP(launch_pack_half2((const float*)p->y, p->m, p->d, p->ldy, x.L.mtiles, x.L.k.kbp, 1.f,
                             x.plan, 1, x.yp, st));
  } else if (x.L.k.mode == kModeSplit)
    OT_HIP(launch_pack_split((const float*)p->y, p->m, p->d, p->ldy, x.L.mtiles, x.L.k.kbp, 1.f, x.yp,
                             st));
  else
    OT_HIP(launch_pack_points(p->y, bf, p->m, p->d, p->ldy, x.L.mtiles, x.L.k.kbp, 1.f, x.yp, st));
  return prepare_eps(x, st);
}

// Bias of the next f half-step from the stored g (and of the g half-step
// from f for the symmetric schedule), in the context's current units.
int rebuild_biases(const Ctx& x, hipStream_t st) {
  const ot_problem* p = x.p;
  OT_HIP(launch_bias_from_pot(x.g, x.ny, x.hy, (int)p->m, x.L.mpad, x.bscale, x.by, 1, st));
  if (x.sym)
    OT_HIP(launch_bias_from_pot(x.f, x.nx, x.hx, (int)p->n, x.L.npad, x.bscale, x.bx, 1, st));
  return OT_OK;
}

int enqueue_iteration(const Ctx& x, hipStream_t st, int with_err, hipEvent_t* ev);

// eps-scaling: iterations at eps_k = eps_start * decay^k while that exceeds
// the problem's eps (plain launches; X and the log-weights are rebuilt for
// every eps_k), then the context is put back to the problem's eps. Returns
// the number of iterations run in *done.
int run_eps_scaling(Ctx& x, hipStream_t st, int max_iters, float eps_start, float decay,
                    int* done) {
  *done = 0;
  float e = eps_start;
  while (*done < max_iters && e > x.p->eps) {
    set_eps_params(x, e);
    int rc = prepare_eps(x, st);
    if (rc) return rc;
    rc = rebuild_biases(x, st);
    if (rc) return rc;
    rc = enqueue_iteration(x, st, 0, nullptr);
    if (rc) return rc;
    ++*done;
    e *= decay;
  }
  if (*done > 0) {
    set_eps_params(x, x.p->eps);
    const int rc = prepare_eps(x, st);
    if (rc) return rc;
  }
  return rebuild_biases(x, st);
}

RowFinish finish_f(const Ctx& x, int with_err, int write, int avg) {
  return RowFinish{x.bscale, x.eps, x.nx, x.hx, x.wx, x.f, x.bx, (int)x.p->n, x.L.npad,
                   with_err, write, avg};
}

RowFinish finish_g(const Ctx& x, int with_err, int write, int avg) {
  return RowFinish{x.bscale, x.eps, x.ny, x.hy, x.wy, x.g, x.by, (int)x.p->m, x.L.mpad,
                   with_err, write, avg};
}

// f half-step: LSE over columns y with bias by, ending in f (and, when
// written, the g side's bias bx); as one launch for small problems, else the
// split pass and the merge of its partials. ev, if given, holds two events
// that the log-sum-exp dispatch records at its start and end.
int half_f(const Ctx& x, hipStream_t st, int with_err, int write, hipEvent_t* ev = nullptr) {
  const RowFinish fin = finish_f(x, with_err, write, 0);
  const LaunchTimer tm{ev ? ev[0] : nullptr, ev ? ev[1] : nullptr};
  const LaunchTimer* t = ev ? &tm : nullptr;
  if (x.L.F.solo) {
    OT_HIP(launch_lse_solo(x.L.F, x.L.k.mode, x.xp, x.yp, x.by, x.kc, fin, x.errp, st, t));
    return OT_OK;
  }
  OT_HIP(launch_lse_partial(x.L.F, x.L.k.mode, x.xp, x.yp, x.by, x.kc, x.part, st, t));
  OT_HIP(launch_lse_merge(x.part, x.L.F.splits, x.L.npad, (int)x.p->n, x.bscale, x.eps, x.nx, x.hx, x.wx,
                          x.f, x.bx, x.errp, with_err, write, 0, st));
  return OT_OK;
}

int half_g(const Ctx& x, hipStream_t st, int with_err, int write, hipEvent_t* ev = nullptr) {
  const RowFinish fin = finish_g(x, with_err, write, 0);
  float* errp = x.errp + x.L.errblocks_f;
  const LaunchTimer tm{ev ? ev[0] : nullptr, ev ? ev[1] : nullptr};
  const LaunchTimer* t = ev ? &tm : nullptr;
  if (x.L.G.solo) {
    OT_HIP(launch_lse_solo(x.L.G, x.L.k.mode, x.yp, x.xp, x.bx, x.kc, fin, errp, st, t));
    return OT_OK;
  }
  OT_HIP(launch_lse_partial(x.L.G, x.L.k.mode, x.yp, x.xp, x.bx, x.kc, x.part, st, t));
  OT_HIP(launch_lse_merge(x.part, x.L.G.splits, x.L.mpad, (int)x.p->m, x.bscale, x.eps, x.ny, x.hy, x.wy,
                          x.g, x.by, errp, with_err, write, 0, st));
  return OT_OK;
}

// One iteration on the stream. Alternating schedule (§3.1 eq. 2-3): the f
// half-step (new f and its bias), then the g half-step from the new f.
// Symmetric schedule (§3.1 eq. 4-5): both passes read the previous biases,
// so both split passes run before either merge; the merges average old and
// new values. ev, if given, holds four events: the start and end of each of
// the two log-sum-exp dispatches, recorded by the dispatches themselves.
int enqueue_iteration(const Ctx& x, hipStream_t st, int with_err, hipEvent_t* ev) {
  if (!x.sym) {
    const int rc = half_f(x, st, with_err, 1, ev);
    if (rc) return rc;
    return half_g(x, st, 0, 1, ev ? ev + 2 : nullptr);
  }
  const LaunchTimer tf{ev ? ev[0] : nullptr, ev ? ev[1] : nullptr};
  const LaunchTimer tg{ev ? ev[2] : nullptr, ev ? ev[3] : nullptr};
  OT_HIP(launch_lse_partial(x.L.F, x.L.k.mode, x.xp, x.yp, x.by, x.kc, x.part, st,
                            ev ? &tf : nullptr));
  OT_HIP(launch_lse_partial(x.L.G, x.L.k.mode, x.yp, x.xp, x.bx, x.kc, x.part2, st,
                            ev ? &tg : nullptr));
  OT_HIP(launch_lse_merge(x.part, x.L.F.splits, x.L.npad, (int)x.p->n, x.bscale, x.eps, x.nx, x.hx,
                          x.wx, x.f, x.bx, x.errp, with_err, 1, 1, st));
  OT_HIP(launch_lse_merge(x.part2, x.L.G.splits, x.L.mpad, (int)x.p->m, x.bscale, x.eps, x.ny, x.hy, x.wy,
                          x.g, x.by, x.errp + x.L.errblocks_f, 0, 1, 1, st));
  return OT_OK;
}

int enqueue_iterations(const Ctx& x, hipStream_t st, int count, int with_err) {
  for (int t = 0; t < count; ++t) {
    const int rc = enqueue_iteration(x, st, with_err, nullptr);
    if (rc) return rc;
  }
  return OT_OK;
}

// ---- HIP graph cache: one entry per distinct (device, problem, workspace, options) ----
struct GraphKey {
  int device;
  uintptr_t ws, f, g, nx, ny;
  int64_t n, m, d;
  int dtype;
  float eps;
  int count, with_err, mode, sym;
  PassShape F, G;
  bool operator==(const GraphKey& o) const { return std::memcmp(this, &o, sizeof(*this)) == 0; }
};

struct GraphEntry {
  GraphKey key;
  hipGraphExec_t exec;
};

std::mutex g_graph_mu;
std::vector<GraphEntry> g_graphs;  // most recent last
hipStream_t g_capture_stream[64] = {};

int get_graph(const Ctx& x, int count, int with_err, hipGraphExec_t* out) {
  int dev = 0;
  OT_HIP(hipGetDevice(&dev));
  GraphKey key;
  std::memset(&key, 0, sizeof(key));
  key.device = dev;
  key.ws = (uintptr_t)x.ws;
  key.f = (uintptr_t)x.f;
  key.g = (uintptr_t)x.g;
  key.nx = (uintptr_t)x.nx;
  key.ny = (uintptr_t)x.ny;
  key.n = x.p->n;
  key.m = x.p->m;
  key.d = x.p->d;
  key.dtype = x.p->dtype;
  key.eps = x.p->eps;
  key.count = count;
  key.with_err = with_err;
  key.mode = x.L.k.mode;
  key.sym = x.sym ? 1 : 0;
  key.F = x.L.F;
  key.G = x.L.G;
  std::lock_guard<std::mutex> lk(g_graph_mu);
  for (size_t i = 0; i < g_graphs.size(); ++i) {
    if (g_graphs[i].key == key) {
      GraphEntry e = g_graphs[i];
      g_graphs.erase(g_graphs.begin() + i);
      g_graphs.push_back(e);
      *out = e.exec;
      return OT_OK;
    }
  }
  if (dev < 0 || dev >= 64) return fail(OT_ERR_UNSUPPORTED, "device index >= 64");
  if (!g_capture_stream[dev]) OT_HIP(hipStreamCreateWithFlags(&g_capture_stream[dev], hipStreamNonBlocking));
  hipStream_t cs = g_capture_stream[dev];
  OT_HIP(hipStreamBeginCapture(cs, hipStreamCaptureModeRelaxed));
  const int rc = enqueue_iterations(x, cs, count, with_err);
  hipGraph_t graph = nullptr;
  const hipError_t ec = hipStreamEndCapture(cs, &graph);
  if (rc) {
    if (graph) (void)hipGraphDestroy(graph);
    return rc;
  }
  if (ec != hipSuccess) return fail(OT_ERR_HIP, std::string("hipStreamEndCapture: ") + hipGetErrorString(ec));
  hipGraphExec_t exec = nullptr;
  const hipError_t ei = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  (void)hipGraphDestroy(graph);
  if (ei != hipSuccess) return fail(OT_ERR_HIP, std::string("hipGraphInstantiate: ") + hipGetErrorString(ei));
  if (g_graphs.size() >= 8) {
    (void)hipGraphExecDestroy(g_graphs.front().exec);
    g_graphs.erase(g_graphs.begin());
  }
  g_graphs.push_back(GraphEntry{key, exec});
  *out = exec;
  return OT_OK;
}

int run_iterations(const Ctx& x, hipStream_t st, int count, int with_err, bool use_graph) {
  if (count <= 0) return OT_OK;
  if (!use_graph) return enqueue_iterations(x, st, count, with_err);
  const int block = count < 16 ? count : 16;
  hipGraphExec_t gb = nullptr;
  int rc = get_graph(x, block, with_err, &gb);
  if (rc) return rc;
  int done = 0;
  for (; done + block <= count; done += block) OT_HIP(hipGraphLaunch(gb, st));
  if (done < count) {
    hipGraphExec_t g1 = nullptr;
    rc = get_graph(x, 1, with_err, &g1);
    if (rc) return rc;
    for (; done < count; ++done) OT_HIP(hipGraphLaunch(g1, st));
  }
  return OT_OK;
}

// Timed variant: plain launches, every LSE kernel recording a HIP event pair
// at its start and end.
struct EventPool {
  std::vector<hipEvent_t> ev;
  int ensure(size_t count) {
    while (ev.size() < count) {
      hipEvent_t e;
      OT_HIP(hipEventCreate(&e));
      ev.push_back(e);
    }
    return OT_OK;
  }
};
thread_local EventPool g_events;

int run_iterations_timed(const Ctx& x, hipStream_t st, int count, int with_err, float* ms,
                         int* launches) {
  const size_t need = (size_t)count * 4;
  int rc = g_events.ensure(need);
  if (rc) return rc;
  for (int t = 0; t < count; ++t) {
    rc = enqueue_iteration(x, st, with_err, &g_events.ev[(size_t)t * 4]);
    if (rc) return rc;
  }
  OT_HIP(hipStreamSynchronize(st));
  float tot = 0.f;
  for (int t = 0; t < count; ++t) {
    hipEvent_t* e = &g_events.ev[(size_t)t * 4];
    float a = 0.f, b = 0.f;
    OT_HIP(hipEventElapsedTime(&a, e[0], e[1]));
    OT_HIP(hipEventElapsedTime(&b, e[2], e[3]));
    tot += a + b;
  }
  *ms += tot;
  *launches += 2 * count;
  return OT_OK;
}


int update_impl(const ot_problem* p, const float* other, float* pot, float* err, void* ws,
                size_t* ws_bytes, void* stream, bool is_f) {
  int rc = check_problem(p);
  if (rc) return rc;
  const SolveWs L = solve_layout(p, 0, 0);
  bool query = false;
  rc = check_ws(ws, ws_bytes, L.total, &query);
  if (rc || query) return rc;
  if (!other || !pot) return fail(OT_ERR_INVALID_ARG, "potential pointer is NULL");
  hipStream_t st = (hipStream_t)stream;
  Ctx x = make_ctx(p, L, ws, is_f ? pot : const_cast<float*>(other), is_f ? const_cast<float*>(other) : pot);
  rc = prepare(x, st);
  if (rc) return rc;
  const int with_err = err != nullptr;
  if (is_f) {
    OT_HIP(launch_bias_from_pot(x.g, x.ny, x.hy, (int)p->m, L.mpad, x.bscale, x.by, 1, st));
    rc = half_f(x, st, with_err, 1);
    if (rc) return rc;
    if (with_err) OT_HIP(launch_err_reduce(x.errp, L.errblocks_f, err, st));
  } else {
    OT_HIP(launch_bias_from_pot(x.f, x.nx, x.hx, (int)p->n, L.npad, x.bscale, x.bx, 1, st));
    rc = half_g(x, st, with_err, 1);
    if (rc) return rc;
    if (with_err) OT_HIP(launch_err_reduce(x.errp + L.errblocks_f, L.errblocks_g, err, st));
  }
  return OT_OK;
}

// ---- transport application ------------------------------------------------
// Scores: two fp16 parts (fp32 points by default), bf16, or fp32 operands
// (OT_NATIVE_F32 / OT_SPLIT_BF16). The value product runs on two fp16 parts
// except in the fp32-operand case.
struct ApplyWs {
  KConf k;
  int rtiles, ctiles, rpad, cpad, pblocks, pb_per_pass, ppad;
  PassShape S;
  size_t o_xp, o_yp, o_nx, o_ny, o_wr, o_hr, o_wc, o_hc, o_bc, o_vp, o_ms, o_o, o_vamax, o_plan;
  size_t total;
};

ApplyWs apply_layout(const ot_problem* p, int64_t cols, bool transpose) {
  ApplyWs w{};
  w.k = kernel_conf(p->d, p->dtype == OT_BF16,
                    f32_operand_mode(p->flags) == kModeHalf2 ? kModeHalf2 : kModeF32, true);
  const int64_t rows = transpose ? p->m : p->n;
  const int64_t strm = transpose ? p->n : p->m;
  w.rtiles = ceil_div(rows, kTile);
  w.ctiles = ceil_div(strm, kTile);
  w.rpad = w.rtiles * kTile;
  w.cpad = w.ctiles * kTile;
  w.pblocks = ceil_div(cols, 32);
  w.pb_per_pass = w.pblocks >= 4 ? 4 : (w.pblocks >= 2 ? 2 : 1);
  w.ppad = w.pblocks * 32;
  if (w.k.xres) {
    w.S = make_pass(w.rtiles, w.ctiles, w.k, 1, 0, 64);
  } else {
    // Wide rows: the smallest power-of-two split count that gives about 4096
    // workgroups, at most 32. Measured on MI355X: P V at n = m = 70000,
    // d = 512 bf16, 7.69 ms with 8 splits against 7.89 with 4 and 8.03 with
    // 32; at n = 200000, m = 10000, d = 1024 fp32, 16.8 ms with 4 against
    // 18.2 with 2 (3 and 5 splits are slower than both), and P^T U there
    // 18.0 ms with 32 against 18.9 with 16.
    const int nrg = ceil_div(w.rtiles, kWaves);
    int S = 1;
    while (S < 32 && (int64_t)S * nrg < 4096) S *= 2;
    w.S = make_pass(w.rtiles, w.ctiles, w.k, 1, S, 64);
    whole_block_splits(w.S);
  }
  const int ntiles = ceil_div(p->n, kTile), mtiles = ceil_div(p->m, kTile);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  w.o_xp = take((size_t)ntiles * w.k.kbp * 1024);
  w.o_yp = take((size_t)mtiles * w.k.kbp * 1024);
  w.o_nx = take((size_t)ntiles * kTile * 4);
  w.o_ny = take((size_t)mtiles * kTile * 4);
  w.o_wr = take((size_t)w.rpad * 4);
  w.o_hr = take((size_t)w.rpad * 4);
  w.o_wc = take((size_t)w.cpad * 4);
  w.o_hc = take((size_t)w.cpad * 4);
  w.o_bc = take(bias_buffer_bytes(w.cpad));  // biases + bias-MFMA operand
  w.o_vp = take((size_t)w.ctiles * w.pblocks * 4096);
  w.o_ms = take((size_t)w.S.splits * w.rpad * 8);
  w.o_o = take((size_t)w.S.splits * w.ppad * w.rpad * 4);
  w.o_vamax = take((size_t)w.ppad * 4);
  w.o_plan = take(sizeof(Half2Plan));
  w.total = o;
  return w;
}

// ---- static scratch of ot_solve_static ---------------------------------------
// For callers that cannot allocate device memory: ot_solve_static runs
// ot_solve with this array as its workspace. Each device the library runs on
// holds one copy from module load until the process ends. In host code the
// array's name is only a stand-in: its device address on the current device
// comes from hipGetSymbolAddress, taken once per device and kept.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on first use).
int static_scratch(void** out) {
  int dev = 0;
  OT_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(OT_ERR_UNSUPPORTED, "device index >= 64");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(OT_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return OT_OK;
}

}  // namespace

extern "C" {

size_t ot_static_scratch_bytes(void) { return kStaticScratchBytes; }

int ot_solve_static(const ot_problem* p, float* f, float* g, const ot_solve_opts* opts,
                    ot_solve_info* info, void* stream) {
  try {
    if (!opts) return fail(OT_ERR_INVALID_ARG, "opts is NULL");
    // Plain launches only: capturing and instantiating a HIP graph, and the
    // per-launch timing events, would allocate.
    ot_solve_opts o = *opts;
    o.use_graph = 0;
    o.timing = 0;
    size_t need = 0;
    int rc = ot_solve(p, nullptr, nullptr, &o, nullptr, nullptr, &need, nullptr);
    if (rc) return rc;
    if (need > kStaticScratchBytes)
      return fail(OT_ERR_WORKSPACE, "problem needs " + std::to_string(need) +
                                        " bytes of scratch; ot_solve_static holds " +
                                        std::to_string(kStaticScratchBytes) +
                                        " (use ot_solve with a workspace)");
    void* ws = nullptr;
    rc = static_scratch(&ws);
    if (rc) return rc;
    size_t sz = kStaticScratchBytes;
    return ot_solve(p, f, g, &o, info, ws, &sz, stream);
  } catch (...) {
    return fail(OT_ERR_HIP, "unexpected host exception");
  }
}

const char* ot_last_error(void) { return flashot::host::last_error(); }

const char* ot_version(void) { return "flashot 0.1 gfx950"; }

int ot_sqnorms(const void* pts, int dtype, int64_t rows, int64_t d, int64_t ld, float* out,
               void* stream) {
  try {
    if (!pts || !out) return fail(OT_ERR_INVALID_ARG, "pts or out is NULL");
    if (rows < 1 || d < 1 || ld < d) return fail(OT_ERR_INVALID_ARG, "need rows >= 1, d >= 1, ld >= d");
    if (dtype != OT_F32 && dtype != OT_BF16) return fail(OT_ERR_UNSUPPORTED, "dtype must be OT_F32 or OT_BF16");
    if (d > OT_MAX_D) return fail(OT_ERR_UNSUPPORTED, "d exceeds OT_MAX_D");
    OT_HIP(launch_sqnorms(pts, dtype == OT_BF16, rows, d, ld, out, (hipStream_t)stream));
    return OT_OK;
  } catch (...) {
    return fail(OT_ERR_HIP, "unexpected host exception");
  }
}

int ot_update_f(const ot_problem* p, const float* g, float* f, float* err, void* ws,
                size_t* ws_bytes, void* stream) {
  try {
    return update_impl(p, g, f, err, ws, ws_bytes, stream, true);
  } catch (...) {
    return fail(OT_ERR_HIP, "unexpected host exception");
  }
}

int ot_update_g(const ot_problem* p, const float* f, float* g, float* err, void* ws,
                size_t* ws_bytes, void* stream) {
  try {
    return update_impl(p, f, g, err, ws, ws_bytes, stream, false);
  } catch (...) {
    return fail(OT_ERR_HIP, "unexpected host exception");
  }
}

int ot_solve(const ot_problem* p, float* f, float* g, const ot_solve_opts* o,
             ot_solve_info* info, void* ws, size_t* ws_bytes, void* stream) {
  try {
    int rc = check_problem(p);
    if (rc) return rc;
    if (!o) return fail(OT_ERR_INVALID_ARG, "opts is NULL");
    if (o->iters < 0) return fail(OT_ERR_INVALID_ARG, "iters must be >= 0");
    if (!(o->tol >= 0.f) || !std::isfinite(o->tol)) return fail(OT_ERR_INVALID_ARG, "tol must be finite and >= 0");
    if (o->tol > 0.f && o->check_every < 1) return fail(OT_ERR_INVALID_ARG, "check_every must be >= 1 when tol > 0");
    if (o->init != OT_INIT_ZERO && o->init != OT_INIT_GIVEN) return fail(OT_ERR_INVALID_ARG, "init must be OT_INIT_ZERO or OT_INIT_GIVEN");
    if (o->splits_f < 0 || o->splits_g < 0) return fail(OT_ERR_INVALID_ARG, "splits must be >= 0");
    if (o->timing && !info) return fail(OT_ERR_INVALID_ARG, "timing needs info");
    if (o->schedule != OT_SCHED_ALTERNATING && o->schedule != OT_SCHED_SYMMETRIC)
      return fail(OT_ERR_INVALID_ARG, "schedule must be OT_SCHED_ALTERNATING or OT_SCHED_SYMMETRIC");
    if (!(o->eps_start >= 0.f) || !std::isfinite(o->eps_start))
      return fail(OT_ERR_INVALID_ARG, "eps_start must be finite and >= 0");
    const bool scaling = o->eps_start > p->eps;
    if (scaling && !(o->eps_decay > 0.f && o->eps_decay < 1.f))
      return fail(OT_ERR_INVALID_ARG, "eps_decay must lie in (0, 1) with eps-scaling");
    if (scaling && !std::isfinite(2.f * kLog2e / (o->eps_start)))
      return fail(OT_ERR_UNSUPPORTED, "eps_start out of range");
    const SolveWs L = solve_layout(p, o->splits_f, o->splits_g);
    bool query = false;
    rc = check_ws(ws, ws_bytes, L.total, &query);
    if (rc || query) return rc;
    if (!f || !g) return fail(OT_ERR_INVALID_ARG, "f or g is NULL");
    hipStream_t st = (hipStream_t)stream;
    Ctx x = make_ctx(p, L, ws, f, g);
    rc = prepare(x, st);
    if (rc) return rc;
    if (o->init == OT_INIT_ZERO) {
      OT_HIP(launch_fill(f, 0.f, p->n, st));
      OT_HIP(launch_fill(g, 0.f, p->m, st));
    }
    x.sym = o->schedule == OT_SCHED_SYMMETRIC;
    int done = 0;
    if (scaling) {
      rc = run_eps_scaling(x, st, o->iters, o->eps_start, o->eps_decay, &done);
      if (rc) return rc;
    } else {
      rc = rebuild_biases(x, st);
      if (rc) return rc;
    }
    const bool use_graph = o->use_graph != 0 && st != nullptr;
    float lse_ms = 0.f;
    int lse_launches = 0;
    const int annealed = done;
    if (o->tol > 0.f) {
      while (done < o->iters) {
        const int chunk = (o->iters - done) < o->check_every ? (o->iters - done) : o->check_every;
        rc = o->timing ? run_iterations_timed(x, st, chunk, 1, &lse_ms, &lse_launches)
                       : run_iterations(x, st, chunk, 1, use_graph);
        if (rc) return rc;
        done += chunk;
        OT_HIP(launch_err_reduce(x.errp, L.errblocks_f, x.errv, st));
        float herr = 0.f;
        OT_HIP(hipMemcpyAsync(&herr, x.errv, sizeof(float), hipMemcpyDeviceToHost, st));
        OT_HIP(hipStreamSynchronize(st));
        if (!(herr >= o->tol)) break;  // also stops on NaN
      }
    } else {
      const int rest = o->iters - annealed;
      rc = o->timing ? run_iterations_timed(x, st, rest, 0, &lse_ms, &lse_launches)
                     : run_iterations(x, st, rest, 0, use_graph);
      if (rc) return rc;
      done = o->iters;
    }
    if (info) {
      // Marginal errors of the returned (f, g). Rows: one dry f pass from g
      // (the bias `by` is current: written by the last g merge or by
      // rebuild_biases). Columns: in the alternating schedule, when the last
      // iteration ran at the problem's eps, its g half-step fit the columns
      // and the error is 0 by construction (a dry pass would reproduce g
      // bitwise); otherwise (symmetric schedule, no iteration, or every
      // iteration annealed) one dry g pass from f, with the bias of f rebuilt
      // at the problem's eps where it is stale.
      rc = half_f(x, st, 1, 0);
      if (rc) return rc;
      OT_HIP(launch_err_reduce(x.errp, L.errblocks_f, x.errv, st));
      if (!x.sym && done > annealed) {
        OT_HIP(launch_fill(x.errv + 1, 0.f, 1, st));
      } else {
        if (!x.sym)
          OT_HIP(launch_bias_from_pot(f, x.nx, x.hx, (int)p->n, L.npad, x.bscale, x.bx, 1, st));
        rc = half_g(x, st, 1, 0);
        if (rc) return rc;
        OT_HIP(launch_err_reduce(x.errp + L.errblocks_f, L.errblocks_g, x.errv + 1, st));
      }
      OT_HIP(launch_nonfinite(f, (int)p->n, g, (int)p->m, x.errv + 2, st));
      float h[3] = {0.f, 0.f, 0.f};
      OT_HIP(hipMemcpyAsync(h, x.errv, sizeof(h), hipMemcpyDeviceToHost, st));
      OT_HIP(hipStreamSynchronize(st));
      info->iters_done = done;
      info->marg_err_row = h[0];
      info->marg_err_col = h[1];
      info->nonfinite = h[2] != 0.f;
      info->lse_ms = lse_ms;
      info->lse_launches = lse_launches;
      info->splits_f = used_splits(L.F, x.sym);
      info->splits_g = used_splits(L.G, x.sym);
      info->operand_mode = L.k.mode;
      if (info->nonfinite) return fail(OT_ERR_NONFINITE, "potentials are not finite");
    }
    return OT_OK;
  } catch (...) {
    return fail(OT_ERR_HIP, "unexpected host exception");
  }
}

int ot_sinkhorn_divergence(const ot_problem* p, const ot_solve_opts* opts, float* f, float* g,
                           float* f_xx, float* g_yy, float* out, void* ws, size_t* ws_bytes,
                           void* stream) {
  try {
    int rc = check_problem(p);
    if (rc) return rc;
    if (!opts) return fail(OT_ERR_INVALID_ARG, "opts is NULL");
    if (p->flags & OT_COST_AFFINE)
      return fail(OT_ERR_UNSUPPORTED, "the self-transport terms need the squared-Euclidean cost");
    // (mu, nu), (mu, mu), (nu, nu): same points, weights and norms
    ot_problem pxx = *p, pyy = *p;
    pxx.y = p->x;
    pxx.m = p->n;
    pxx.ldy = p->ldx;
    pxx.b = p->a;
    pxx.y_sqn = p->x_sqn;
    pyy.x = p->y;
    pyy.n = p->m;
    pyy.ldx = p->ldy;
    pyy.a = p->b;
    pyy.x_sqn = p->y_sqn;
    ot_solve_opts o = *opts;
    o.timing = 0;
    ot_solve_opts oz = o;
    oz.init = OT_INIT_ZERO;
    size_t need[3] = {0, 0, 0};
    const ot_problem* ps[3] = {p, &pxx, &pyy};
    for (int k = 0; k < 3; ++k) {
      rc = ot_solve(ps[k], nullptr, nullptr, k ? &oz : &o, nullptr, nullptr, &need[k], nullptr);
      if (rc) return rc;
    }
    size_t solve_ws = need[0] > need[1] ? need[0] : need[1];
    solve_ws = align_up(solve_ws > need[2] ? solve_ws : need[2], 256);
    const size_t o_gxx = solve_ws, o_fyy = align_up(o_gxx + (size_t)p->n * 4, 256);
    const size_t total = align_up(o_fyy + (size_t)p->m * 4, 256);
    bool query = false;
    rc = check_ws(ws, ws_bytes, total, &query);
    if (rc || query) return rc;
    if (!f || !g || !f_xx || !g_yy || !out) return fail(OT_ERR_INVALID_ARG, "f, g, f_xx, g_yy or out is NULL");
    char* w = (char*)ws;
    float* g_xx = (float*)(w + o_gxx);
    float* f_yy = (float*)(w + o_fyy);
    size_t sz = solve_ws;
    rc = ot_solve(p, f, g, &o, nullptr, ws, &sz, stream);
    if (rc) return rc;
    rc = ot_solve(&pxx, f_xx, g_xx, &oz, nullptr, ws, &sz, stream);
    if (rc) return rc;
    rc = ot_solve(&pyy, f_yy, g_yy, &oz, nullptr, ws, &sz, stream);
    if (rc) return rc;
    OT_HIP(launch_dual_values(p->a, p->b, (int)p->n, (int)p->m, f, g, f_xx, g_xx, f_yy, g_yy, out,
                              (hipStream_t)stream));
    return OT_OK;
  } catch (...) {
    return fail(OT_ERR_HIP, "unexpected host exception");
  }
}

int ot_apply_plan(const ot_problem* p, const float* f, const float* g, const void* V, int v_dtype,
                  int64_t cols, int64_t ldv, int flags, float* out, float* marg, void* ws,
                  size_t* ws_bytes, void* stream) {
  try {
    int rc = check_problem(p);
    if (rc) return rc;
    if (flags & ~(OT_TRANSPOSE | OT_GRAD | OT_BARY)) return fail(OT_ERR_INVALID_ARG, "unknown flag");
    if ((flags & OT_GRAD) && (flags & OT_BARY)) return fail(OT_ERR_INVALID_ARG, "OT_GRAD and OT_BARY are exclusive");
    if ((flags & OT_GRAD) && (p->flags & OT_COST_AFFINE))
      return fail(OT_ERR_UNSUPPORTED, "OT_GRAD is the squared-Euclidean gradient: not with OT_COST_AFFINE");
    const bool tr = (flags & OT_TRANSPOSE) != 0;
    const bool grad = (flags & OT_GRAD) != 0;
    if (grad) {  // V is the other cloud itself
      V = tr ? p->x : p->y;
      v_dtype = p->dtype;
      cols = p->d;
      ldv = tr ? p->ldx : p->ldy;
    }
    if (cols < 1) return fail(OT_ERR_INVALID_ARG, "cols must be >= 1");
    if (cols > OT_MAX_COLS) return fail(OT_ERR_UNSUPPORTED, "cols exceeds OT_MAX_COLS");
    if (v_dtype != OT_F32 && v_dtype != OT_BF16) return fail(OT_ERR_UNSUPPORTED, "v_dtype must be OT_F32 or OT_BF16");
    const ApplyWs L = apply_layout(p, cols, tr);
    bool query = false;
    rc = check_ws(ws, ws_bytes, L.total, &query);
    if (rc || query) return rc;
    if (!f || !g || !V || !out) return fail(OT_ERR_INVALID_ARG, "f, g, V or out is NULL");
    if (ldv < cols) return fail(OT_ERR_INVALID_ARG, "ldv must be >= cols");
    if ((uintptr_t)V % (v_dtype == OT_BF16 ? 2 : 4)) return fail(OT_ERR_INVALID_ARG, "V misaligned");
    hipStream_t st = (hipStream_t)stream;
    char* w = (char*)ws;
    const int bf = p->dtype == OT_BF16;
    const float eps = p->eps, c = 2.f * kLog2e / p->eps;
    const int ntiles = ceil_div(p->n, kTile), mtiles = ceil_div(p->m, kTile);
    void* xp = w + L.o_xp;
    void* yp = w + L.o_yp;
    const float* nx = p->x_sqn ? p->x_sqn : (const float*)(w + L.o_nx);
    const float* ny = p->y_sqn ? p->y_sqn : (const float*)(w + L.o_ny);
    if (!p->x_sqn) OT_HIP(launch_sqnorms(p->x, bf, p->n, p->d, p->ldx, (float*)nx, st));
    if (!p->y_sqn) OT_HIP(launch_sqnorms(p->y, bf, p->m, p->d, p->ldy, (float*)ny, st));
    const float xs = (p->flags & OT_COST_AFFINE) ? 0.5f : 1.f;
    // Units of the scores: log2 units for the fp16 parts (X packed times c,
    // the kernel's multiplier kc = 1), dot-product units otherwise (kc = c).
    const bool h2 = L.k.mode == kModeHalf2;
    const bool fp16_values = L.k.mode != kModeF32;
    const float kc = h2 ? 1.f : c;
    if (h2) {
      Half2Plan* plan = (Half2Plan*)(w + L.o_plan);
      OT_HIP(launch_half2_plan((const float*)p->x, p->n, p->ldx, (const float*)p->y, p->m, p->ldy,
                               p->d, c * xs, plan, st));
      rc = check_half2_range(plan, st);
      if (rc) return rc;
      OT_HIP(launch_pack_half2((const float*)p->x, p->n, p->d, p->ldx, ntiles, L.k.kbp, c * xs,
                               plan, 0, xp, st));
      OT_HIP(launch_pack_half2((const float*)p->y, p->m, p->d, p->ldy, mtiles, L.k.kbp, 1.f, plan,
                               1, yp, st));
    } else {
      OT_HIP(launch_pack_points(p->x, bf, p->n, p->d, p->ldx, ntiles, L.k.kbp, xs, xp, st));
      OT_HIP(launch_pack_points(p->y, bf, p->m, p->d, p->ldy, mtiles, L.k.kbp, 1.f, yp, st));
    }
    // Row side r (outputs) and column side s (streamed).
    const int64_t rows = tr ? p->m : p->n, srows = tr ? p->n : p->m;
    const float* wr_user = tr ? p->b : p->a;
    const float* ws_user = tr ? p->a : p->b;
    const float* pot_r = tr ? g : f;
    const float* pot_s = tr ? f : g;
    const float* norm_r = tr ? ny : nx;
    const float* norm_s = tr ? nx : ny;
    const void* Rp = tr ? yp : xp;
    const void* Cp = tr ? xp : yp;
    float* wr = (float*)(w + L.o_wr);
    float* hr = (float*)(w + L.o_hr);
    float* wc = (float*)(w + L.o_wc);
    float* hc = (float*)(w + L.o_hc);
    float* bc = (float*)(w + L.o_bc);
    float* vp = (float*)(w + L.o_vp);
    float2* pms = (float2*)(w + L.o_ms);
    float* po = (float*)(w + L.o_o);
    OT_HIP(launch_weights(wr_user, (int)rows, L.rpad, eps, wr, hr, st));
    OT_HIP(launch_weights(ws_user, (int)srows, L.cpad, eps, wc, hc, st));
    OT_HIP(launch_bias_from_pot(pot_s, norm_s, hc, (int)srows, L.cpad, h2 ? c : 1.f, bc, 1, st));
    unsigned* vamax = fp16_values ? (unsigned*)(w + L.o_vamax) : nullptr;
    if (fp16_values) {
      OT_HIP(launch_vcol_absmax(V, v_dtype == OT_BF16, srows, cols, ldv, vamax, st));
      OT_HIP(launch_pack_values_h2(V, v_dtype == OT_BF16, srows, cols, ldv, L.ctiles, L.pblocks,
                                   vamax, vp, st));
      OT_HIP(launch_apply_stream(L.S, L.k.mode, L.pblocks, L.pb_per_pass,
                                 v_dtype == OT_BF16 ? 1 : 2, Rp, Cp, bc, vp, kc, pms, po, L.ppad,
                                 st));
    } else {
      OT_HIP(launch_pack_values(V, v_dtype == OT_BF16, srows, cols, ldv, L.ctiles, L.pblocks, vp,
                                st));
      OT_HIP(launch_apply_partial(L.S, bf, L.pblocks, L.pb_per_pass, Rp, Cp, bc, vp, c, pms, po,
                                  L.ppad, st));
    }
    const int mode = grad ? kApplyGrad : ((flags & OT_BARY) ? kApplyBary : kApplyPlain);
    const void* Xsrc = tr ? p->y : p->x;
    const int64_t ldx = tr ? p->ldy : p->ldx;
    // the fp16-value kernels write their stabilisers in log2 units
    OT_HIP(launch_apply_merge(pms, po, L.S.splits, L.rpad, L.ppad, (int)rows, (int)cols,
                              fp16_values ? 1.f : c, eps,
                              pot_r, norm_r, wr, mode, Xsrc, bf, ldx, vamax, out, marg, st));
    return OT_OK;
  } catch (...) {
    return fail(OT_ERR_HIP, "unexpected host exception");
  }
}

}  // extern "C"
