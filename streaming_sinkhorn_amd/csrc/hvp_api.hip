// C ABI of the second-order entry points: the Hadamard-weighted transport
// (Algorithm 5) and the streaming Hessian-vector product (§3.3 Thm. 5,
// App. F) of "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU".
// Declarations and semantics in include/flashot.h.
//
// Both clouds are packed once per call in the transport layout; every
// product with the coupling is one streamed apply pass (partials + merge) in
// either direction, from the potentials. The conjugate-gradient recurrence
// runs on device scalars, so a fixed iteration count needs no host round trip.
#include <hip/hip_runtime.h>

#include <cmath>
#include <string>

#include "flashot.h"
#include "host_common.h"
#include "kernels.h"

using namespace flashot;
using namespace flashot::host;

namespace {

// Value columns of one apply pass: 32-column blocks and blocks per workgroup.
struct Cols {
  int pblocks, pb_per_pass, ppad;
};

Cols cols_of(int64_t cols) {
  Cols c{};
  c.pblocks = ceil_div(cols, 32);
  c.pb_per_pass = c.pblocks >= 4 ? 4 : (c.pblocks >= 2 ? 2 : 1);
  c.ppad = c.pblocks * 32;
  return c;
}

// Workspace of the transport passes in both directions: F = P V (rows x,
// columns y), T = P^T U (rows y, columns x). cols_f / cols_t are the widest
// value matrices each direction is used with.
struct TransportWs {
  KConf k;
  int ntiles, mtiles, npad, mpad;
  PassShape F, T;
  size_t o_xp, o_yp, o_ap, o_nx, o_ny, o_wx, o_hx, o_wy, o_hy, o_bx, o_by, o_vp, o_ms, o_o,
      o_vamax;
};

template <typename Take>
TransportWs transport_layout(const ot_problem* p, int64_t cols_f, int64_t cols_t, bool with_a,
                             Take&& take) {
  TransportWs w{};
  w.k = kernel_conf(p->d, 0, kModeF32, true);
  w.ntiles = ceil_div(p->n, kTile);
  w.mtiles = ceil_div(p->m, kTile);
  w.npad = w.ntiles * kTile;
  w.mpad = w.mtiles * kTile;
  w.F = make_pass(w.ntiles, w.mtiles, w.k, 1, 0, 64);
  w.T = make_pass(w.mtiles, w.ntiles, w.k, 1, 0, 64);
  if (!w.k.xres) {
    whole_block_splits(w.F);
    whole_block_splits(w.T);
  }
  const Cols cf = cols_of(cols_f), ct = cols_of(cols_t > 0 ? cols_t : 1);
  w.o_xp = take((size_t)w.ntiles * w.k.kbp * 1024);
  w.o_yp = take((size_t)w.mtiles * w.k.kbp * 1024);
  w.o_ap = with_a ? take((size_t)w.ntiles * w.k.kbp * 1024) : 0;
  w.o_nx = take((size_t)w.npad * 4);
  w.o_ny = take((size_t)w.mpad * 4);
  w.o_wx = take((size_t)w.npad * 4);
  w.o_hx = take((size_t)w.npad * 4);
  w.o_wy = take((size_t)w.mpad * 4);
  w.o_hy = take((size_t)w.mpad * 4);
  w.o_bx = take((size_t)w.npad * 4);
  w.o_by = take((size_t)w.mpad * 4);
  const size_t vf = (size_t)w.mtiles * cf.pblocks, vt = (size_t)w.ntiles * ct.pblocks;
  w.o_vp = take((vf > vt ? vf : vt) * 4096);
  const size_t mf = (size_t)w.F.splits * w.npad, mt = (size_t)w.T.splits * w.mpad;
  w.o_ms = take((mf > mt ? mf : mt) * 8);
  const size_t of = mf * cf.ppad, ot = mt * ct.ppad;
  w.o_o = take((of > ot ? of : ot) * 4);
  w.o_vamax = take((size_t)(cf.ppad > ct.ppad ? cf.ppad : ct.ppad) * 4);
  return w;
}

// Resolved pointers of the transport workspace, with the potentials.
struct Transport {
  const ot_problem* p;
  TransportWs L;
  float c, eps;
  void *xp, *yp, *ap;
  const float *nx, *ny, *f, *g;
  float *wx, *hx, *wy, *hy, *bx, *by, *vp, *po;
  float2* pms;
  unsigned* vamax;
};

Transport make_transport(const ot_problem* p, const TransportWs& L, char* w, const float* f,
                         const float* g) {
  Transport t{};
  t.p = p;
  t.L = L;
  t.eps = p->eps;
  t.c = 2.f * kLog2e / p->eps;
  t.xp = w + L.o_xp;
  t.yp = w + L.o_yp;
  t.ap = L.o_ap ? w + L.o_ap : nullptr;
  t.nx = p->x_sqn ? p->x_sqn : (const float*)(w + L.o_nx);
  t.ny = p->y_sqn ? p->y_sqn : (const float*)(w + L.o_ny);
  t.f = f;
  t.g = g;
  t.wx = (float*)(w + L.o_wx);
  t.hx = (float*)(w + L.o_hx);
  t.wy = (float*)(w + L.o_wy);
  t.hy = (float*)(w + L.o_hy);
  t.bx = (float*)(w + L.o_bx);
  t.by = (float*)(w + L.o_by);
  t.vp = (float*)(w + L.o_vp);
  t.po = (float*)(w + L.o_o);
  t.pms = (float2*)(w + L.o_ms);
  t.vamax = (unsigned*)(w + L.o_vamax);
  return t;
}

// Norms, packed operands (X, Y and optionally A, fp32, dot-product units),
// weights, and the column bias of each direction (from g for P, from f for
// P^T).
int prepare_transport(const Transport& t, const float* A, int64_t lda, hipStream_t st) {
  const ot_problem* p = t.p;
  const TransportWs& L = t.L;
  if (!p->x_sqn) OT_HIP(launch_sqnorms(p->x, 0, p->n, p->d, p->ldx, (float*)t.nx, st));
  if (!p->y_sqn) OT_HIP(launch_sqnorms(p->y, 0, p->m, p->d, p->ldy, (float*)t.ny, st));
  OT_HIP(launch_pack_points(p->x, 0, p->n, p->d, p->ldx, L.ntiles, L.k.kbp, 1.f, t.xp, st));
  OT_HIP(launch_pack_points(p->y, 0, p->m, p->d, p->ldy, L.mtiles, L.k.kbp, 1.f, t.yp, st));
  if (A) OT_HIP(launch_pack_points(A, 0, p->n, p->d, lda, L.ntiles, L.k.kbp, 1.f, t.ap, st));
  OT_HIP(launch_weights(p->a, (int)p->n, L.npad, t.eps, t.wx, t.hx, st));
  OT_HIP(launch_weights(p->b, (int)p->m, L.mpad, t.eps, t.wy, t.hy, st));
  OT_HIP(launch_bias_from_pot(t.g, t.ny, t.hy, (int)p->m, L.mpad, 1.f, t.by, 0, st));
  OT_HIP(launch_bias_from_pot(t.f, t.nx, t.hx, (int)p->n, L.npad, 1.f, t.bx, 0, st));
  return OT_OK;
}

// out = P V (tr = false, V: m x cols) or P^T V (tr = true, V: n x cols), fp32
// with row stride ldv; with hadamard, out = (P . A Y^T) V. marg (or NULL)
// receives r = P 1 (resp. c = P^T 1). Scores on fp32 operands; the value
// product on fp16 parts, except in the Hadamard-weighted pass.
int transport(const Transport& t, bool tr, const float* V, int64_t cols, int64_t ldv, float* out,
              float* marg, bool hadamard, hipStream_t st) {
  const ot_problem* p = t.p;
  const PassShape& S = tr ? t.L.T : t.L.F;
  const Cols cc = cols_of(cols);
  const int64_t rows = tr ? p->m : p->n, srows = tr ? p->n : p->m;
  const int rpad = tr ? t.L.mpad : t.L.npad;
  const void* Rp = tr ? t.yp : t.xp;
  const void* Cp = tr ? t.xp : t.yp;
  const float* bc = tr ? t.bx : t.by;
  if (hadamard) {
    OT_HIP(launch_pack_values(V, 0, srows, cols, ldv, S.ctiles, cc.pblocks, t.vp, st));
    OT_HIP(launch_apply_hadamard(S, cc.pblocks, cc.pb_per_pass, Rp, Cp, t.ap, bc, t.vp, t.c,
                                 t.pms, t.po, cc.ppad, st));
  } else {
    OT_HIP(launch_vcol_absmax(V, 0, srows, cols, ldv, t.vamax, st));
    OT_HIP(launch_pack_values_h2(V, 0, srows, cols, ldv, S.ctiles, cc.pblocks, t.vamax, t.vp, st));
    OT_HIP(launch_apply_stream(S, kModeF32, cc.pblocks, cc.pb_per_pass, 2, Rp, Cp, bc, t.vp, t.c,
                               t.pms, t.po, cc.ppad, st));
  }
  // the fp16-value kernels write their stabilisers in log2 units
  OT_HIP(launch_apply_merge(t.pms, t.po, S.splits, rpad, cc.ppad, (int)rows, (int)cols,
                            hadamard ? t.c : 1.f,
                            t.eps, tr ? t.g : t.f, tr ? t.ny : t.nx, tr ? t.wy : t.wx, kApplyPlain,
                            nullptr, 0, 0, hadamard ? nullptr : t.vamax, out, marg, st));
  return OT_OK;
}

int check_f32_problem(const ot_problem* p) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (p->dtype != OT_F32) return fail(OT_ERR_UNSUPPORTED, "second-order entry points take fp32 points");
  if (p->flags & OT_COST_AFFINE)
    return fail(OT_ERR_UNSUPPORTED, "second-order entry points assume the squared-Euclidean cost");
  return OT_OK;
}

// Bump allocator over a workspace of unknown size (sizing pass) or a real one.
struct Carver {
  size_t o = 0;
  size_t operator()(size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  }
};

// Transport-vector passes of the conjugate gradients (P p, P^T u) on the
// log-sum-exp layout: both clouds packed as for the Sinkhorn half-steps
// (three-part bf16 split by default), column biases in log2 units, and the
// register-resident passes with a value column. Used when that layout is
// register-resident (d <= 128); wider points use the apply passes.
struct VecWs {
  bool on;
  KConf k;
  PassShape F, G;  // F: rows x, columns y; G: rows y, columns x
  size_t o_xs, o_ys, o_bx, o_by, o_part, o_partT, o_ones, o_rv, o_cv, o_plan;
};

// HVP vectors beyond the transport workspace. pd and u are padded to whole
// tiles (zeros) because the vector passes read their values tile by tile.
struct HvpWs {
  TransportWs T;
  VecWs V;
  size_t o_py, o_r, o_c, o_xa, o_ra1, o_vb, o_ptv, o_rhs, o_w2, o_res, o_pd, o_q, o_pp, o_u,
      o_ptu, o_vf, o_pf, o_b5, o_part, o_cs;
  size_t total;
};

HvpWs hvp_layout(const ot_problem* p) {
  HvpWs w{};
  Carver take;
  const int64_t n = p->n, m = p->m, d = p->d;
  w.T = transport_layout(p, d + 1, d + 2, true, take);
  w.o_py = take((size_t)n * d * 4);
  w.o_r = take((size_t)n * 4);
  w.o_c = take((size_t)m * 4);
  w.o_xa = take((size_t)n * 4);
  w.o_ra1 = take((size_t)n * 4);
  w.o_vb = take((size_t)n * (d + 2) * 4);
  w.o_ptv = take((size_t)m * (d + 2) * 4);
  w.o_rhs = take((size_t)m * 4);
  w.o_w2 = take((size_t)m * 4);
  w.o_res = take((size_t)m * 4);
  w.o_pd = take((size_t)w.T.mpad * 4);
  w.o_q = take((size_t)m * 4);
  w.o_pp = take((size_t)n * 4);
  w.o_u = take((size_t)w.T.npad * 4);
  w.o_ptu = take((size_t)m * 4);
  w.o_vf = take((size_t)m * (d + 1) * 4);
  w.o_pf = take((size_t)n * (d + 1) * 4);
  w.o_b5 = take((size_t)n * d * 4);
  w.o_part = take((size_t)kCgMaxParts * 4);
  w.o_cs = take(sizeof(CgState));
  VecWs& v = w.V;
  v.k = kernel_conf(p->d, 0, f32_operand_mode(p->flags));
  if (v.k.mode == kModeHalf2 && v.k.xres) {
    // the value column and T take registers: LDS-shared columns from d = 64
    // and one row tile per wave at d = 128 keep two waves per SIMD
    v.k.lds = v.k.kb >= 8;
    v.k.ri = v.k.kb >= 16 ? 1 : 2;
  }
  v.on = v.k.xres;
  if (v.on) {
    const int nt = w.T.ntiles, mt = w.T.mtiles;
    // transport-vector passes keep the 2048-workgroup target: at n = m = 50000
    // (196 row groups) it gives 16 column splits instead of 6, about 1 %
    // faster per HVP
    v.F = make_pass(nt, mt, v.k, v.k.ri, 0, 4096);
    v.G = make_pass(mt, nt, v.k, v.k.ri, 0, 4096);
    v.o_xs = take((size_t)nt * v.k.kbp * 1024);
    v.o_ys = take((size_t)mt * v.k.kbp * 1024);
    v.o_bx = take(bias_buffer_bytes(w.T.npad));  // feed log-sum-exp passes: with the
    v.o_by = take(bias_buffer_bytes(w.T.mpad));  // bias-MFMA operand (kernels.h)
    const size_t pf = (size_t)v.F.splits * w.T.npad, pg = (size_t)v.G.splits * w.T.mpad;
    const size_t pm = pf > pg ? pf : pg;
    v.o_part = take(pm * 8);
    v.o_partT = take(pm * 4);
    v.o_ones = take((size_t)(w.T.npad > w.T.mpad ? w.T.npad : w.T.mpad) * 4);
    v.o_rv = take((size_t)w.T.npad * 4);
    v.o_cv = take((size_t)w.T.mpad * 4);
    v.o_plan = take(sizeof(Half2Plan));
  }
  w.total = take.o;
  return w;
}

// Operands of the vector passes: X packed pre-scaled by c = 2 log2(e) / eps
// (two-part fp16, three-part bf16 or fp32 layout; the fp16 one with its range
// plan), Y unscaled, biases c ((pot - |.|^2) / 2 + (eps/2) log w) from the
// transport context's log-weights.
int prepare_vec(const Transport& t, const VecWs& v, char* w, hipStream_t st) {
  const ot_problem* p = t.p;
  const TransportWs& L = t.L;
  void* xs = w + v.o_xs;
  void* ys = w + v.o_ys;
  if (v.k.mode == kModeHalf2) {
    Half2Plan* plan = (Half2Plan*)(w + v.o_plan);
    OT_HIP(launch_half2_plan((const float*)p->x, p->n, p->ldx, (const float*)p->y, p->m, p->ldy,
                             p->d, t.c, plan, st));
    const int rc = check_half2_range(plan, st);
    if (rc) return rc;
    OT_HIP(launch_pack_half2((const float*)p->x, p->n, p->d, p->ldx, L.ntiles, v.k.kbp, t.c, plan,
                             0, xs, st));
    OT_HIP(launch_pack_half2((const float*)p->y, p->m, p->d, p->ldy, L.mtiles, v.k.kbp, 1.f, plan,
                             1, ys, st));
  } else if (v.k.mode == kModeSplit) {
    OT_HIP(launch_pack_split((const float*)p->x, p->n, p->d, p->ldx, L.ntiles, v.k.kbp, t.c, xs, st));
    OT_HIP(launch_pack_split((const float*)p->y, p->m, p->d, p->ldy, L.mtiles, v.k.kbp, 1.f, ys, st));
  } else {
    OT_HIP(launch_pack_points(p->x, 0, p->n, p->d, p->ldx, L.ntiles, v.k.kbp, t.c, xs, st));
    OT_HIP(launch_pack_points(p->y, 0, p->m, p->d, p->ldy, L.mtiles, v.k.kbp, 1.f, ys, st));
  }
  OT_HIP(launch_bias_from_pot(t.g, t.ny, t.hy, (int)p->m, L.mpad, t.c, (float*)(w + v.o_by), 1, st));
  OT_HIP(launch_bias_from_pot(t.f, t.nx, t.hx, (int)p->n, L.npad, t.c, (float*)(w + v.o_bx), 1, st));
  return OT_OK;
}

// out = P v (tr = false; v: m values padded to whole tiles) or P^T v (tr =
// true; v: n values, padded), one streamed pass plus the merge.
int vec_pass(const Transport& t, const VecWs& v, char* w, bool tr, const float* vals, float* out,
             hipStream_t st) {
  const ot_problem* p = t.p;
  const PassShape& S = tr ? v.G : v.F;
  const void* Rp = w + (tr ? v.o_ys : v.o_xs);
  const void* Cp = w + (tr ? v.o_xs : v.o_ys);
  const float* bias = (const float*)(w + (tr ? v.o_bx : v.o_by));
  float2* part = (float2*)(w + v.o_part);
  float* partT = (float*)(w + v.o_partT);
  const int rows = (int)(tr ? p->m : p->n);
  const int rpad = tr ? t.L.mpad : t.L.npad;
  OT_HIP(launch_vec_resident(S, v.k.mode, Rp, Cp, bias, vals, 1.f, part, partT, st));
  OT_HIP(launch_vec_merge(part, partT, S.splits, rpad, rows, t.eps, tr ? t.g : t.f,
                          tr ? t.ny : t.nx, tr ? t.wy : t.wx, out, st));
  return OT_OK;
}

}  // namespace

extern "C" {

int ot_apply_hadamard(const ot_problem* p, const float* f, const float* g, const float* A,
                      int64_t lda, const float* V, int64_t cols, int64_t ldv, float* out, void* ws,
                      size_t* ws_bytes, void* stream) {
  try {
    int rc = check_f32_problem(p);
    if (rc) return rc;
    if (cols < 1) return fail(OT_ERR_INVALID_ARG, "cols must be >= 1");
    if (cols > OT_MAX_COLS) return fail(OT_ERR_UNSUPPORTED, "cols exceeds OT_MAX_COLS");
    Carver take;
    const TransportWs L = transport_layout(p, cols, 0, true, take);
    bool query = false;
    rc = check_ws(ws, ws_bytes, take.o, &query);
    if (rc || query) return rc;
    if (!f || !g || !A || !V || !out) return fail(OT_ERR_INVALID_ARG, "f, g, A, V or out is NULL");
    if (lda < p->d) return fail(OT_ERR_INVALID_ARG, "lda must be >= d");
    if (ldv < cols) return fail(OT_ERR_INVALID_ARG, "ldv must be >= cols");
    if ((uintptr_t)A % 4 || (uintptr_t)V % 4) return fail(OT_ERR_INVALID_ARG, "A or V misaligned");
    hipStream_t st = (hipStream_t)stream;
    const Transport t = make_transport(p, L, (char*)ws, f, g);
    rc = prepare_transport(t, A, lda, st);
    if (rc) return rc;
    return transport(t, false, V, cols, ldv, out, nullptr, true, st);
  } catch (...) {
    return fail(OT_ERR_HIP, "unexpected host exception");
  }
}

int ot_hvp(const ot_problem* p, const float* f, const float* g, const float* A, int64_t lda,
           const ot_hvp_opts* opts, float* out, ot_hvp_info* info, void* ws, size_t* ws_bytes,
           void* stream) {
  try {
    int rc = check_f32_problem(p);
    if (rc) return rc;
    if (!opts) return fail(OT_ERR_INVALID_ARG, "opts is NULL");
    if (!(opts->tau >= 0.f) || !std::isfinite(opts->tau)) return fail(OT_ERR_INVALID_ARG, "tau must be finite and >= 0");
    if (!(opts->tol >= 0.f) || !std::isfinite(opts->tol)) return fail(OT_ERR_INVALID_ARG, "tol must be finite and >= 0");
    if (opts->max_iters < 0) return fail(OT_ERR_INVALID_ARG, "max_iters must be >= 0");
    if (p->d + 2 > OT_MAX_COLS) return fail(OT_ERR_UNSUPPORTED, "d + 2 exceeds OT_MAX_COLS");
    const HvpWs L = hvp_layout(p);
    bool query = false;
    rc = check_ws(ws, ws_bytes, L.total, &query);
    if (rc || query) return rc;
    if (!f || !g || !A || !out) return fail(OT_ERR_INVALID_ARG, "f, g, A or out is NULL");
    if (lda < p->d) return fail(OT_ERR_INVALID_ARG, "lda must be >= d");
    if ((uintptr_t)A % 4) return fail(OT_ERR_INVALID_ARG, "A misaligned");
    hipStream_t st = (hipStream_t)stream;
    char* w = (char*)ws;
    const Transport t = make_transport(p, L.T, w, f, g);
    rc = prepare_transport(t, A, lda, st);
    if (rc) return rc;
    const int n = (int)p->n, m = (int)p->m, d = (int)p->d;
    const float* X = (const float*)p->x;
    const float* Y = (const float*)p->y;
    float* PY = (float*)(w + L.o_py);
    float* r = (float*)(w + L.o_r);
    float* c = (float*)(w + L.o_c);
    float* xa = (float*)(w + L.o_xa);
    float* ra1 = (float*)(w + L.o_ra1);
    float* VB = (float*)(w + L.o_vb);
    float* PTV = (float*)(w + L.o_ptv);
    float* rhs = (float*)(w + L.o_rhs);
    float* w2 = (float*)(w + L.o_w2);
    float* res = (float*)(w + L.o_res);
    float* pd = (float*)(w + L.o_pd);
    float* q = (float*)(w + L.o_q);
    float* Pp = (float*)(w + L.o_pp);
    float* u = (float*)(w + L.o_u);
    float* PTu = (float*)(w + L.o_ptu);
    float* VF = (float*)(w + L.o_vf);
    float* PF = (float*)(w + L.o_pf);
    float* B5 = (float*)(w + L.o_b5);
    float* part = (float*)(w + L.o_part);
    CgState* cs = (CgState*)(w + L.o_cs);

    // P Y and r = P 1 (cached transport-matrix product, App. F.3).
    rc = transport(t, false, Y, d, p->ldy, PY, r, false, st);
    if (rc) return rc;
    // Row terms, then one P^T pass for P^T A, P^T xa, P^T (R1 / r) and c.
    OT_HIP(launch_hvp_prep(n, d, X, p->ldx, A, lda, PY, r, xa, ra1, VB, st));
    rc = transport(t, true, VB, d + 2, d + 2, PTV, c, false, st);
    if (rc) return rc;
    OT_HIP(launch_hvp_rhs(m, d, Y, p->ldy, PTV, rhs, w2, res, pd, st));
    // Marginals used by the conjugate gradients. With the vector passes they
    // are taken from those passes too (P 1, P^T 1), so that the Schur
    // operator diag c - P^T diag(1/r) P annihilates the constant vector in
    // the same arithmetic as its products (its damped null direction then
    // has eigenvalue tau exactly, whatever rounding the passes carry).
    const float* rs = r;
    const float* csum = c;
    if (L.V.on) {
      // zero tile padding of the CG vectors (finite values for padded columns)
      OT_HIP(launch_fill(pd + m, 0.f, L.T.mpad - m, st));
      OT_HIP(launch_fill(u, 0.f, L.T.npad, st));
      rc = prepare_vec(t, L.V, w, st);
      if (rc) return rc;
      float* ones = (float*)(w + L.V.o_ones);
      float* rv = (float*)(w + L.V.o_rv);
      float* cv = (float*)(w + L.V.o_cv);
      OT_HIP(launch_fill(ones, 1.f, L.T.npad > L.T.mpad ? L.T.npad : L.T.mpad, st));
      rc = vec_pass(t, L.V, w, false, ones, rv, st);
      if (rc) return rc;
      rc = vec_pass(t, L.V, w, true, ones, cv, st);
      if (rc) return rc;
      rs = rv;
      csum = cv;
    }
    // Conjugate gradients on (S + tau I) w2 = rhs: two transport-vector
    // products per iteration.
    OT_HIP(launch_cg_start(m, rhs, part, cs, st));
    for (int it = 0; it < opts->max_iters; ++it) {
      if (opts->tol > 0.f && it > 0) {
        int done = 0;
        OT_HIP(hipMemcpyAsync(&done, &cs->done, sizeof(int), hipMemcpyDeviceToHost, st));
        OT_HIP(hipStreamSynchronize(st));
        if (done) break;
      }
      rc = L.V.on ? vec_pass(t, L.V, w, false, pd, Pp, st)
                  : transport(t, false, pd, 1, 1, Pp, nullptr, false, st);
      if (rc) return rc;
      OT_HIP(launch_cg_div(n, Pp, rs, u, cs, st));
      rc = L.V.on ? vec_pass(t, L.V, w, true, u, PTu, st)
                  : transport(t, true, u, 1, 1, PTu, nullptr, false, st);
      if (rc) return rc;
      OT_HIP(launch_cg_update(m, csum, PTu, opts->tau, opts->tol, pd, q, w2, res, part, cs, st));
    }
    // Back-substitution values [w2 y_j, w2_j]: P diag(w2) Y and P w2 in one pass.
    OT_HIP(launch_hvp_vf(m, d, Y, p->ldy, w2, VF, st));
    rc = transport(t, false, VF, d + 1, d + 1, PF, nullptr, false, st);
    if (rc) return rc;
    // B5 = (P . A Y^T) Y (Algorithm 5).
    rc = transport(t, false, Y, d, p->ldy, B5, nullptr, true, st);
    if (rc) return rc;
    OT_HIP(launch_hvp_final(n, d, p->eps, X, p->ldx, A, lda, PY, r, xa, ra1, PF, B5, out, st));
    if (info) {
      CgState h{};
      OT_HIP(hipMemcpyAsync(&h, cs, sizeof(h), hipMemcpyDeviceToHost, st));
      OT_HIP(hipStreamSynchronize(st));
      info->cg_iters = h.iters;
      info->breakdown = h.breakdown;
      info->cg_rel_residual = h.bb > 0.f ? std::sqrt(h.rr / h.bb) : 0.f;
    }
    return OT_OK;
  } catch (...) {
    return fail(OT_ERR_HIP, "unexpected host exception");
  }
}

}  // extern "C"
