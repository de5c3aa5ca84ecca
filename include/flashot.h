/*
 * flashot.h -- streamed log-domain Sinkhorn for squared-Euclidean entropic
 * optimal transport on AMD Instinct MI355X (gfx950).
 *
 * The method is the one on the page "FlashSinkhorn: IO-Aware Entropic
 * Optimal Transport on GPU" (arXiv 2602.03067): each stabilised Sinkhorn
 * half-step is a row-wise log-sum-exp of a biased dot-product score
 * (Prop. 1, §3.1, App. D.1), evaluated tile by tile with an online max /
 * sum-of-exponentials so that only the n- and m-length potentials are
 * written to memory (App. D.2, D.3, G.1-G.2); the transport plan is applied
 * to a matrix the same way without ever forming it (§3.2, Prop. 3, App. E.1).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Measures mu = sum_i a_i delta_{x_i} (n points) and nu = sum_j b_j
 *    delta_{y_j} (m points) in R^d, cost C_ij = ||x_i - y_j||^2.
 *  - Potentials f (n) and g (m) are the UNSHIFTED dual potentials. The
 *    coupling they induce is P_ij = a_i b_j exp((f_i + g_j - C_ij) / eps).
 *  - Half-steps (§3.1, alternating schedule eq. 2-3):
 *        f_i = -eps * LSE_j((g_j - C_ij)/eps + log b_j)
 *        g_j = -eps * LSE_i((f_i - C_ij)/eps + log a_i)
 *    computed as f_i = ||x_i||^2 - eps * LSE_j(2 x_i.y_j/eps + (g_j - ||y_j||^2)/eps
 *    + log b_j), the biased dot-product form of Prop. 1 / App. D.1.
 *  - All array arguments are DEVICE pointers on the current HIP device unless
 *    stated otherwise; the caller owns every buffer. The library never
 *    allocates or frees device memory: scratch comes from the caller's
 *    workspace. Calling with ws == NULL writes the required workspace size to
 *    *ws_bytes and does nothing else (returns OT_OK).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and returns without synchronising, except where a function says so.
 *    One such case is shared by every entry point that forms scores: fp32
 *    points in the default operand mode (see ot_problem flags) are checked
 *    against the fp16 range on the device, and the call waits for that
 *    check (one stream synchronisation, before its passes are enqueued).
 *  - Point arrays are row-major: element (i, k) of X is at x[i * ldx + k],
 *    ldx >= d. Their storage type is OT_F32 (float) or OT_BF16 (bfloat16);
 *    products are accumulated in fp32, potentials and weights are fp32.
 *  - Outputs must not alias inputs, except that f (resp. g) may be updated in
 *    place where documented.
 *  - Weights a, b must be strictly positive; NULL means uniform (1/n, 1/m).
 *    They are used as given (not renormalised).
 *  - Return value: an OT_* status. Argument checks run on the host before any
 *    HIP call. A HIP failure (launch, runtime) returns OT_ERR_HIP; the message
 *    of the last failure is available from ot_last_error().
 */
#ifndef FLASHOT_H
#define FLASHOT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define OT_OK              0
#define OT_ERR_INVALID_ARG 1  /* null pointer, size < 1, eps <= 0, ld < d, bad flag */
#define OT_ERR_UNSUPPORTED 2  /* dtype or size outside what the kernels handle */
#define OT_ERR_WORKSPACE   3  /* workspace smaller than required */
#define OT_ERR_HIP         4  /* HIP runtime / launch error */
#define OT_ERR_NONFINITE   5  /* a potential became NaN or infinite (reported by ot_solve) */

/* Storage types of point / value arrays. */
#define OT_F32  0
#define OT_BF16 1

/* ot_solve initialisation. */
#define OT_INIT_ZERO  0  /* start from f = g = 0 */
#define OT_INIT_GIVEN 1  /* start from the caller's f, g (warm start / resume) */

/* ot_solve schedules. */
#define OT_SCHED_ALTERNATING 0  /* f from g, then g from the new f (§3.1 eq. 2-3) */
#define OT_SCHED_SYMMETRIC   1  /* f <- (f + T_f(g))/2, g <- (g + T_g(f))/2 from the previous
                                   iterate (§3.1 eq. 4-5, the GeomLoss-style schedule) */

/* ot_apply_plan flags. */
#define OT_TRANSPOSE 1  /* compute P^T U (U has n rows) instead of P V (V has m rows) */
#define OT_GRAD      2  /* out = 2 (r * X - P Y), the X-gradient (Y-gradient with OT_TRANSPOSE); V is ignored */
#define OT_BARY      4  /* out = (P V) / r row-wise: entropic barycentric projection */

/* Largest supported point dimension and value-column count. */
#define OT_MAX_D    8192
#define OT_MAX_COLS 8192

/* ot_problem flags. */
#define OT_NATIVE_F32 1  /* fp32 points: form scores with fp32 MFMA instead of the default
                            two-part fp16 split on the fp16 MFMA */
#define OT_COST_AFFINE 2 /* general affine cost C_ij = alpha_i + beta_j - <x_i, y_j>
                            (§3.1 "Scope of cost structure"): x_sqn carries alpha and
                            y_sqn carries beta, both required */
#define OT_SPLIT_BF16 4  /* fp32 points: form scores from three bf16 parts per value on the
                            bf16 MFMA (full fp32 exponent range); exclusive with
                            OT_NATIVE_F32 */

/*
 * The problem: two point clouds, their weights and eps (App. H.2 problem
 * statement: discrete measures, squared-Euclidean cost, entropic
 * regularisation eps).
 *   x, y        device, row-major n x d (resp. m x d), storage `dtype`
 *   n, m        number of points, >= 1
 *   d           dimension, 1 <= d <= OT_MAX_D
 *   ldx, ldy    row strides in elements, >= d
 *   dtype       OT_F32 or OT_BF16 (both clouds)
 *   eps         regularisation, > 0
 *   a, b        device fp32 weights (n, m) or NULL for uniform
 *   x_sqn,y_sqn device fp32 squared norms ||x_i||^2, ||y_j||^2, or NULL to
 *               have them computed into the workspace
 *   flags       0, or one of OT_NATIVE_F32 / OT_SPLIT_BF16, and / or
 *               OT_COST_AFFINE.
 *               OT_COST_AFFINE replaces the squared-Euclidean cost by
 *               C_ij = alpha_i + beta_j - <x_i, y_j> with alpha = x_sqn and
 *               beta = y_sqn (both must be given): x, y are the features Q, K
 *               of §3.1. The kernels are the same (x is packed halved, which
 *               is exact, so that the squared-Euclidean score 2 <x, y> becomes
 *               <x, y>). The cosine and label-augmented costs are affine
 *               costs built by ot_prep_cosine / ot_prep_labels. OT_GRAD,
 *               ot_hvp and ot_apply_hadamard assume the squared-Euclidean
 *               cost and reject the flag.
 *               For fp32 points the log-sum-exp passes by default write
 *               every coordinate as two fp16 parts (hi + lo, 22 significant
 *               bits; X scaled by 2^a and Y by 2^-a, exact powers of two
 *               chosen on the device to fit fp16) and form each score from
 *               the three largest partial products on the fp16 matrix cores:
 *               each coordinate product is off by at most about 3 * 2^-22 of
 *               its size, the order of fp32 rounding over a dot product.
 *               This covers every problem with
 *               (2/eps) log2(e) max|x_ik| max|y_jk| < 2^29 (scores in log2
 *               units that fp32 still resolves) and none at or above 2^30.
 *               The check runs on the device before the passes; a problem
 *               outside the range makes ot_update_f, ot_update_g, ot_solve,
 *               ot_apply_plan and ot_hvp return OT_ERR_UNSUPPORTED (after
 *               one stream synchronisation, the same in range) without
 *               enqueuing their passes. OT_SPLIT_BF16 uses three bf16 parts
 *               (24 significant bits, six products, fp32 exponent range) and
 *               OT_NATIVE_F32 the fp32 matrix instruction; neither
 *               synchronises. Transport application (ot_apply_plan) forms
 *               its scores the same way, and multiplies the exponentiated
 *               scores into the values on the fp16 matrix cores: each score
 *               p (below 2^15 against a lazily raised stabiliser) as two
 *               fp16 parts and each value column, scaled by a power of two,
 *               as two fp16 parts, three partial products per term, each
 *               within about 2^-22 of its size (bf16 values: their lo part
 *               is zero, two products). Under OT_NATIVE_F32 / OT_SPLIT_BF16
 *               both products are fp32.
 */
typedef struct ot_problem {
  const void* x;
  const void* y;
  int64_t n, m, d, ldx, ldy;
  int32_t dtype;
  float eps;
  const float* a;
  const float* b;
  const float* x_sqn;
  const float* y_sqn;
  int32_t flags;  /* OT_NATIVE_F32, OT_SPLIT_BF16, OT_COST_AFFINE */
} ot_problem;

/* ot_solve options. Zero-initialise and set what you need. */
typedef struct ot_solve_opts {
  int32_t iters;        /* number of alternating iterations T (>= 0) */
  float tol;            /* > 0: stop early once the row-marginal L1 error falls below tol */
  int32_t check_every;  /* iterations between tolerance checks (>= 1 when tol > 0) */
  int32_t init;         /* OT_INIT_ZERO or OT_INIT_GIVEN */
  int32_t use_graph;    /* 1: replay a captured HIP graph per block of iterations; 0: plain launches */
  int32_t splits_f;     /* column splits of the f half-step (0 = automatic; automatic runs
                           the half-steps of small problems, at most 3072 points a side,
                           as one launch each in the alternating schedule) */
  int32_t splits_g;     /* column splits of the g half-step (0 = automatic) */
  int32_t timing;       /* 1: time every log-sum-exp kernel with HIP events that its
                           dispatch records (needs info; the iterations then run as
                           plain launches) */
  int32_t schedule;     /* OT_SCHED_ALTERNATING (0) or OT_SCHED_SYMMETRIC */
  float eps_start;      /* eps-scaling: 0 = off; > eps: iteration k runs at
                           max(eps, eps_start * eps_decay^k) */
  float eps_decay;      /* eps-scaling factor per iteration, 0 < eps_decay < 1 */
} ot_solve_opts;

/* ot_solve results (host memory). */
typedef struct ot_solve_info {
  int32_t iters_done;    /* iterations actually run */
  int32_t nonfinite;     /* 1 if the final f or g holds NaN / Inf */
  float marg_err_row;    /* ||P 1 - a||_1 of the returned (f, g), from one extra row pass */
  float marg_err_col;    /* ||P^T 1 - b||_1 of the returned (f, g). Alternating schedule with
                            its last iteration at eps: the last g half-step fit the columns,
                            and this is 0 by construction (no pass; the true value is that
                            half-step's fp32 rounding). Symmetric schedule, iters = 0 or
                            every iteration annealed: from one extra column pass. */
  float lse_ms;          /* with opts.timing: summed duration of the log-sum-exp kernels (ms) */
  int32_t lse_launches;  /* with opts.timing: number of log-sum-exp kernel launches timed */
  int32_t splits_f;      /* column splits used by the f half-step (single-launch half-step:
                            the waves of a workgroup that hold column tiles) */
  int32_t splits_g;      /* column splits used by the g half-step */
  int32_t operand_mode;  /* scores formed from: 0 fp32 MFMA, 1 bf16 MFMA, 2 fp32 split into
                            three bf16 parts on the bf16 MFMA (six products per pair),
                            3 fp32 split into two fp16 parts on the fp16 MFMA (three) */
} ot_solve_info;

/*
 * ot_sqnorms -- out[i] = sum_k pts[i*ld + k]^2 in fp32 (App. D.1: alpha_i =
 * ||x_i||^2, beta_j = ||y_j||^2, the per-point terms of the affine cost
 * decomposition of §3.1 "Scope of cost structure").
 *   pts    device, rows x d, storage dtype (OT_F32 / OT_BF16), row stride ld
 *   out    device fp32, rows
 * Errors: OT_ERR_INVALID_ARG (null, rows < 1, d < 1, ld < d),
 *         OT_ERR_UNSUPPORTED (dtype, d > OT_MAX_D), OT_ERR_HIP.
 */
int ot_sqnorms(const void* pts, int dtype, int64_t rows, int64_t d, int64_t ld,
               float* out, void* stream);

/*
 * ot_update_f -- one f half-step from g (Algorithm 1 of the page, §3.1 eq. 2,
 * Prop. 1): f_i = -eps * LSE_j((g_j - C_ij)/eps + log b_j), streamed over the
 * columns with an online max / sum of exponentials (App. D.3).
 *   g     device fp32, m (input)
 *   f     device fp32, n (output; may be the caller's previous f, updated in place)
 *   err   device fp32 scalar or NULL. When set, f must hold the previous
 *         potential f_old on entry and *err receives ||P(f_old, g) 1 - a||_1
 *         = sum_i a_i |exp((f_old_i - f_i)/eps) - 1| (App. E.1 induced row
 *         marginal), the row-marginal error of the coupling before the update.
 *   ws, ws_bytes  workspace (see conventions)
 * Errors: OT_ERR_INVALID_ARG, OT_ERR_UNSUPPORTED (also for fp32 points out
 * of the fp16 range, see ot_problem flags), OT_ERR_WORKSPACE, OT_ERR_HIP.
 */
int ot_update_f(const ot_problem* p, const float* g, float* f, float* err,
                void* ws, size_t* ws_bytes, void* stream);

/*
 * ot_update_g -- one g half-step from f (Algorithm 3 of the page, §3.1 eq. 3,
 * App. D.1 "the g-hat update"): g_j = -eps * LSE_i((f_i - C_ij)/eps + log a_i),
 * the f half-step with the roles of (x, a, f) and (y, b, g) exchanged.
 *   f     device fp32, n (input);  g  device fp32, m (output, in place allowed)
 *   err   as in ot_update_f with columns: ||P(f, g_old)^T 1 - b||_1.
 * Errors: as ot_update_f.
 */
int ot_update_g(const ot_problem* p, const float* f, float* g, float* err,
                void* ws, size_t* ws_bytes, void* stream);

/*
 * ot_solve -- `opts->iters` Sinkhorn iterations (§4.1 / App. H.2: fixed
 * iteration count, no eps-scaling, no debiasing) in one of two schedules:
 *   OT_SCHED_ALTERNATING (§3.1 eq. 2-3): an f half-step from the current g,
 *     then a g half-step from the new f;
 *   OT_SCHED_SYMMETRIC (§3.1 eq. 4-5, the GeomLoss-style schedule): both
 *     half-steps read the previous iterate, f <- (f + T_f(g))/2 and
 *     g <- (g + T_g(f))/2.
 *   f, g   device fp32 (n, m): output potentials; with OT_INIT_GIVEN also the
 *          starting point (k then k' iterations equal k + k' iterations).
 *   opts   host, required
 *   info   host or NULL. When non-NULL the call synchronises the stream at the
 *          end and fills every field; marg_err_row is then the L1 row-marginal
 *          error of the returned (f, g), from one extra streamed pass, and
 *          marg_err_col the column one (see ot_solve_info).
 *   With opts->tol > 0 the row-marginal error of the coupling of the previous
 *   iterate is evaluated inside every f half-step (it is r - a for r of App.
 *   E.1) and the host reads it every opts->check_every iterations (one
 *   synchronisation per check); the loop stops after the iteration in which
 *   it fell below tol.
 *   eps-scaling (opts->eps_start > eps): the first iterations run at the
 *   decreasing eps_k = eps_start * eps_decay^k while that exceeds eps (the
 *   potentials carry over), then every iteration runs at eps; all of them
 *   count in opts->iters. The page's benchmarks turn it off (App. H.2); the
 *   geometric schedule is this library's reading. The tolerance check runs
 *   only in the iterations at eps.
 * Errors: as ot_update_f, plus OT_ERR_NONFINITE when info is given and the
 * final potentials are not finite. OT_ERR_UNSUPPORTED also when fp32 points
 * are too large for the default two-part fp16 scores (see ot_problem flags).
 */
int ot_solve(const ot_problem* p, float* f, float* g, const ot_solve_opts* opts,
             ot_solve_info* info, void* ws, size_t* ws_bytes, void* stream);

/*
 * ot_solve_static -- ot_solve for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same iterations and results as ot_solve, with the
 * library's own static device scratch as the workspace instead of a
 * caller-supplied one. The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine): it launches plain kernels (opts->use_graph
 * and opts->timing are ignored, since capturing a graph and the timing
 * events allocate).
 *   p, f, g, opts, info, stream   as in ot_solve (info may be NULL)
 * Scratch: ot_static_scratch_bytes() bytes (64 MiB) per device, held from
 * the library's load on that device until the process ends. Every call on a
 * device shares that device's scratch and leaves the last call's contents in
 * it; calls that overlap on one device (concurrent streams or threads) race
 * and must be serialised by the caller.
 * Errors: as ot_solve, plus OT_ERR_WORKSPACE when the problem needs more
 * scratch than the static array holds (its ot_solve workspace size query,
 * ws == NULL, exceeds ot_static_scratch_bytes()).
 */
int ot_solve_static(const ot_problem* p, float* f, float* g, const ot_solve_opts* opts,
                    ot_solve_info* info, void* stream);

/* Bytes of the static device scratch ot_solve_static uses (per device). */
size_t ot_static_scratch_bytes(void);

/*
 * ot_sinkhorn_divergence -- debiased Sinkhorn divergence
 *     S_eps(mu, nu) = OT_eps(mu, nu) - OT_eps(mu, mu) / 2 - OT_eps(nu, nu) / 2
 * (the quantity of §1, "debiasing" of App. H.2), each OT_eps the dual value
 * <a, f> + <b, g> of its own ot_solve with the same opts (schedule,
 * iterations, eps-scaling), on the same stream.
 *   f, g    device fp32 (n, m): potentials of (mu, nu) (outputs; with
 *           OT_INIT_GIVEN also the start of that solve)
 *   f_xx    device fp32 (n): f-side potential of (mu, mu) (output)
 *   g_yy    device fp32 (m): g-side potential of (nu, nu) (output)
 *   out     device fp32 [4]: S, OT(mu, nu), OT(mu, mu), OT(nu, nu); the dual
 *           values are summed in fp64 in a fixed order before rounding
 *   opts    host, required; OT_INIT_GIVEN applies to (mu, nu) only (the
 *           self-transport solves start from zero); timing is ignored
 * The self-transport problems reuse the problem's points, weights and norms
 * (x against x, y against y). Errors: as ot_solve; OT_COST_AFFINE is
 * rejected (OT_ERR_UNSUPPORTED: the roles of x and y differ in an affine
 * cost, so x against x is not the same cost).
 */
int ot_sinkhorn_divergence(const ot_problem* p, const ot_solve_opts* opts, float* f, float* g,
                           float* f_xx, float* g_yy, float* out, void* ws, size_t* ws_bytes,
                           void* stream);

/*
 * ot_apply_plan -- apply the coupling induced by (f, g) to a matrix without
 * forming it (Algorithm 2 / Prop. 3 for P V, Algorithm 4 / App. E.1 for
 * P^T U): out = P V, or P^T U with OT_TRANSPOSE. The identity holds for any
 * potentials (§3.2), so early-stopped potentials apply their own coupling.
 *   f, g    device fp32 (n, m)
 *   V       device, (m x cols) for P V or (n x cols) for P^T U, row stride ldv,
 *           storage v_dtype (OT_F32 / OT_BF16). The value product runs on
 *           the fp16 matrix cores with two fp16 parts per score and per
 *           (power-of-two scaled) value, three partial products per term
 *           (two for OT_BF16 values, whose lo part is zero); fp32 under
 *           OT_NATIVE_F32 / OT_SPLIT_BF16 (see ot_problem flags)
 *   cols    1 <= cols <= OT_MAX_COLS
 *   flags   0 or OT_TRANSPOSE, optionally with one of OT_GRAD / OT_BARY
 *   out     device fp32, row-major (n x cols) or (m x cols), stride cols
 *           - default:      out = P V            (resp. P^T U)
 *           - OT_BARY:      out = (P V) / r      (resp. (P^T U) / c), the
 *                           entropic barycentric projection of §3.2
 *           - OT_GRAD:      out = 2 (r * X - P Y) (n x d), the gradient in X of
 *                           sum_ij P_ij ||x_i - y_j||^2 with P held fixed
 *                           (§2.2 / App. G.1, induced marginals); with
 *                           OT_TRANSPOSE the Y-gradient 2 (c * Y - P^T X)
 *                           (m x d). V, v_dtype, cols and ldv are ignored:
 *                           the other cloud is the value matrix.
 *   marg    device fp32 (n, or m with OT_TRANSPOSE) or NULL: receives the
 *           induced marginal r = P 1 (resp. c = P^T 1)
 * Errors: OT_ERR_INVALID_ARG, OT_ERR_UNSUPPORTED (also for fp32 points out
 * of the fp16 range, see ot_problem flags), OT_ERR_WORKSPACE, OT_ERR_HIP.
 */
int ot_apply_plan(const ot_problem* p, const float* f, const float* g,
                  const void* V, int v_dtype, int64_t cols, int64_t ldv, int flags,
                  float* out, float* marg, void* ws, size_t* ws_bytes, void* stream);

/*
 * ot_apply_hadamard -- Hadamard-weighted transport from potentials
 * (Algorithm 5 of the page, §3.3, App. F.3): out = (P . (A Y^T)) V, i.e.
 * out_i = sum_j P_ij <a_i, y_j> v_j, without forming P or A Y^T. Used by the
 * explicit term of the Hessian-vector product (B5 of App. F.1 with V = Y).
 *   p       fp32 points only (OT_BF16: OT_ERR_UNSUPPORTED)
 *   f, g    device fp32 (n, m)
 *   A       device fp32, n x d, row stride lda >= d
 *   V       device fp32, m x cols, row stride ldv >= cols; 1 <= cols <= OT_MAX_COLS
 *   out     device fp32, n x cols, stride cols
 * Errors: OT_ERR_INVALID_ARG, OT_ERR_UNSUPPORTED, OT_ERR_WORKSPACE, OT_ERR_HIP.
 */
int ot_apply_hadamard(const ot_problem* p, const float* f, const float* g,
                      const float* A, int64_t lda, const float* V, int64_t cols,
                      int64_t ldv, float* out, void* ws, size_t* ws_bytes, void* stream);

/* ot_hvp options. Zero-initialise and set what you need. */
typedef struct ot_hvp_opts {
  float tau;          /* damping tau >= 0: the Schur system is solved as S + tau I */
  int32_t max_iters;  /* conjugate-gradient iterations K >= 0 */
  float tol;          /* > 0: stop once ||res|| <= tol ||rhs|| (relative residual eta);
                         0: run all K iterations */
} ot_hvp_opts;

/* ot_hvp results (host memory). */
typedef struct ot_hvp_info {
  int32_t cg_iters;       /* conjugate-gradient iterations run */
  int32_t breakdown;      /* 1: a direction with non-positive curvature stopped the solve */
  float cg_rel_residual;  /* ||res|| / ||rhs|| when the solve ended (recursive residual) */
} ot_hvp_info;

/*
 * ot_hvp -- Hessian-vector product G = T A of OT_eps in the source points X
 * (Y fixed), streamed from the potentials (§3.3 Thm. 5, App. F, App. G.1
 * "HVP"):
 *     G = E A + (1/eps) R^T w,   H* w = R A,   H* = [[diag r, P], [P^T, diag c]]
 * with r = P 1, c = P^T 1 the induced marginals of the coupling of (f, g).
 *   - E A = 2 r*A - (4/eps)(B2 - B3 - B4 + B5) (App. F.1, F.3), with B5 the
 *     Hadamard-weighted transport (P . A Y^T) Y;
 *   - R A_i = 2 sum_j P_ij (x_i - y_j).a_i (rows), and the same sum over i
 *     for the columns; R^T w_i = 2 sum_j P_ij (w1_i + w2_j)(x_i - y_j);
 *   - w2 solves the damped Schur system (S + tau I) w2 = R2 - P^T (R1 / r),
 *     S = diag c - P^T diag(1/r) P, by conjugate gradients from 0 (§3.3:
 *     damping tau, stop at relative residual eta = tol or after K = max_iters
 *     iterations); then w1 = (R1 - P w2) / r (App. F.2).
 * Every transport product is streamed (3 with d or more value columns, one
 * Hadamard-weighted, and 2 per conjugate-gradient iteration with one column);
 * memory is O((n + m) d) beyond the split partials.
 *   p       fp32 points only (OT_BF16: OT_ERR_UNSUPPORTED)
 *   f, g    device fp32 (n, m): potentials, usually converged (ot_solve)
 *   A       device fp32, n x d, row stride lda >= d: the direction
 *   opts    host, required
 *   out     device fp32, n x d, stride d
 *   info    host or NULL. With tol > 0 the host reads the solver state after
 *           every iteration (one synchronisation each); when info is non-NULL
 *           the call synchronises the stream at the end and fills it.
 * The conjugate-gradient products (d <= 128) form their scores in the
 * problem's fp32 operand mode (see ot_problem flags).
 * Errors: OT_ERR_INVALID_ARG (null pointer, lda < d, tau < 0, tol < 0,
 * max_iters < 0, non-finite option), OT_ERR_UNSUPPORTED (also for points
 * too large for the default two-part fp16 scores),
 * OT_ERR_WORKSPACE, OT_ERR_HIP.
 */
int ot_hvp(const ot_problem* p, const float* f, const float* g, const float* A, int64_t lda,
           const ot_hvp_opts* opts, float* out, ot_hvp_info* info, void* ws,
           size_t* ws_bytes, void* stream);

/*
 * ot_prep_cosine -- features of the cosine cost C_ij = 1 - <x_i, y_j> /
 * (||x_i|| ||y_j||) as an affine cost (§3.1 "Scope of cost structure": the
 * cosine cost is reached by L2-normalising the points). Writes
 * out_i = pts_i / ||pts_i|| (a row of zero norm stays zero, giving cost 1
 * against every point) and half_i = 1/2, so that with OT_COST_AFFINE,
 * x = out_x, y = out_y, x_sqn = half_x, y_sqn = half_y the problem's cost is
 * 1/2 + 1/2 - <x^_i, y^_j>.
 *   pts     device, rows x d, row stride ld >= d, storage dtype (OT_F32 / OT_BF16)
 *   out     device fp32, rows x d, stride d
 *   half    device fp32, rows
 * Errors: OT_ERR_INVALID_ARG (null pointer, rows or d < 1, ld < d),
 * OT_ERR_UNSUPPORTED (dtype, d > OT_MAX_D), OT_ERR_HIP. Enqueued on stream.
 */
int ot_prep_cosine(const void* pts, int dtype, int64_t rows, int64_t d, int64_t ld, float* out,
                   float* half, void* stream);

/*
 * ot_prep_labels -- features of the label-augmented cost
 * C_ij = ||x_i - y_j||^2 + W[l_i, l_j] (the OTDD cost of §4.2: feature
 * distance plus a label-to-label term, looked up per pair) as an affine
 * cost. The lookup is folded into the matrix product by one-hot label
 * features, with L = n_labels extra columns:
 *   side 0 (source x):  out_i = [2 x_i, -W[l_i, 0..L-1]]
 *   side 1 (target y):  out_j = [y_j, e_{l_j}]           (one-hot)
 * so that <out_i, out_j> = 2 <x_i, y_j> - W[l_i, l_j]; sqn receives
 * ||pts_i||^2 (alpha or beta). Use the outputs with OT_COST_AFFINE (x_sqn =
 * source sqn, y_sqn = target sqn), dimension d + L.
 *   pts      device, rows x d, row stride ld >= d, storage dtype
 *   labels   device int32, rows, each in [0, n_labels); a label outside that
 *            range gets zero label features (no label term for its pairs)
 *   W        device fp32, n_labels x n_labels, row-major
 *   out      device fp32, rows x (d + n_labels), stride d + n_labels
 *   sqn      device fp32, rows
 * Errors: OT_ERR_INVALID_ARG (null pointer, sizes < 1, ld < d, side not 0/1),
 * OT_ERR_UNSUPPORTED (dtype, d + n_labels > OT_MAX_D), OT_ERR_HIP.
 */
int ot_prep_labels(const void* pts, int dtype, int64_t rows, int64_t d, int64_t ld,
                   const int32_t* labels, const float* W, int32_t n_labels, int32_t side,
                   float* out, float* sqn, void* stream);

/* Text of the most recent error in this thread ("" if none). Host pointer, valid until the next call. */
const char* ot_last_error(void);

/* Library version, e.g. "flashot 0.1 gfx950". */
const char* ot_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLASHOT_H */
