/*
 * fs_sinkhorn.h -- C ABI of the streaming log-domain Sinkhorn solver for
 * entropic optimal transport with squared-Euclidean cost on AMD MI355X
 * (gfx950).
 *
 * What it computes.  "FlashSinkhorn: IO-Aware Entropic Optimal Transport on
 * GPU" (gist.science explainer), section "Method", part 1: for point clouds
 * X (n x d) with weights a and Y (m x d) with weights b, the stabilised
 * log-domain Sinkhorn update
 *     f_i <- -eps * LSE_j [ (g_j - C_ij)/eps + log b_j ],  C_ij = |x_i - y_j|^2,
 * equals a row-wise log-sum-exp of the biased dot-product score matrix
 * (2 x_i.y_j + g_j - |y_j|^2 + eps log b_j)/eps, plus |x_i|^2; the g-update is
 * the mirror image with (Y, b, g) and (X, a, f) exchanged.  Part 2 of the same
 * section: the n x m matrix is never stored; tiles of the other cloud are
 * streamed past a resident block of rows while a running maximum and
 * exp-sum are kept on chip.  Part 3: the transport plan
 *     P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps)
 * is applied to a matrix V (U = P.V, or the barycentric projection P.V / a)
 * by the same streaming traversal, again without storing P.
 *
 * Conventions (every entry point):
 *  - Array arguments are DEVICE pointers to float32, row-major, unless stated.
 *    Point rows are contiguous: X[i*d + t].
 *  - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *    All work is enqueued on it and is asynchronous unless stated.  Inputs must
 *    stay valid until the enqueued work has finished.
 *  - Every call returns an fs_status.  Argument errors detected on the host are
 *    returned before anything is enqueued; fs_last_error() then gives a
 *    thread-local message.  The library never aborts and never throws.
 *  - The library never allocates device memory.  The caller passes one
 *    workspace of fs_workspace_bytes() bytes, 256-byte aligned, which must
 *    outlive the problem handle and must not be shared by two live handles.
 *  - Results are deterministic: the same inputs, launch and device give
 *    bit-identical outputs (no atomics in any reduction; fixed merge order).
 */
#ifndef FS_SINKHORN_H
#define FS_SINKHORN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FS_OK = 0,
    FS_ERR_INVALID_ARG = 1,   /* null pointer, bad size/enum/eps, forbidden alias */
    FS_ERR_WORKSPACE = 2,     /* workspace too small or misaligned */
    FS_ERR_DEVICE = 3,        /* no usable gfx950 device, or a HIP runtime error */
    FS_ERR_NONFINITE = 4,     /* NaN/Inf in X, Y, a, b, or a weight <= 0 */
    FS_ERR_NOT_CONVERGED = 5  /* tol > 0 and the residual stayed above tol */
} fs_status;

/* Element type of the score contraction 2 x.y (everything after it is fp32).
 * AUTO, FP32: fp32-accurate scores on the matrix cores.  For d <= 8 the
 *   whole biased score is one small matrix product per 32x32 block of pairs,
 *   so that the vector unit is left almost entirely to the one exponential
 *   per pair: for d <= 4 on fp16 hi/lo splits of the operands where their
 *   error bound holds, else on bf16 three-part splits (six products per
 *   coordinate, fp32 accumulation, the error of fp32 products), for
 *   5 <= d <= 8 on fp32 operands; for 8 < d <= 512 the points are
 *   zero-padded fp32 matrix operands.
 * FP32_VALU (d <= 8 only): fp32 scores by vector FMA, one lane per row (the
 *   plain vector formulation; slower on gfx950, where exponentials and vector
 *   instructions share issue slots).
 * BF16 / FP16: the centred points (below) are rounded to bfloat16 /
 *   float16 with round-to-nearest-even and multiplied on matrix cores with
 *   fp32 accumulation; the per-point cost terms A, B stay fp32 from the
 *   unrounded points, so only the product x'.y' carries the rounding.
 *   The effective cost is C~_ij = A_i + B_j - 2 x~'_i.y~'_j, where x~', y~'
 *   are the rounded centred points.  Both run at the same matrix-core rate;
 *   they differ in precision.  bf16 keeps 8 significant bits: measured
 *   against the float64 iteration on the original points, it meets the
 *   2e-2 eps potential bar on two 10-component Gaussian mixtures in d >= 64
 *   at eps = 0.1 (2.2e-3 eps at d = 512), but not at d = 16 (3e-2 eps) nor
 *   on the sphere-against-shifted-Gaussian clouds in d = 1024 annealed to
 *   eps = 0.01 (4.5e-2 eps).  fp16 (11 bits) met the bar in every case
 *   measured (5e-3 eps on the latter) and is the choice where the spread of
 *   a centred cloud is far above eps.  Neither is rejected: the error depends
 *   on the data and on eps, which init does not see. */
typedef enum {
    FS_PREC_AUTO = 0,
    FS_PREC_FP32 = 1,
    FS_PREC_BF16 = 2,
    FS_PREC_FP16 = 3,
    FS_PREC_FP32_VALU = 4,
    FS_PREC_BF16_REFINE = 5
} fs_score_prec;
/* BF16_REFINE (d > 8): the problem keeps both a bf16 and an fp16 copy of the
 *   centred points.  fs_lse_update_f/g and the iterations of
 *   fs_sinkhorn_solve use the bf16 copy, except the last refine_iters
 *   iterations of a fixed-count schedule (fs_solve_opts; default 1, counted
 *   over all stages), which use the fp16 copy, as does every pass evaluated at
 *   given potentials (fs_marginal_residual, the transports, fs_gradient,
 *   fs_hvp).  With tol > 0 the residual checks measure the bf16 iterations
 *   and refine_iters fp16 iterations follow the stop (counted in iters_done;
 *   residual is the last check's).  Iterations on the fp16 copy from
 *   bf16-converged potentials bring them within the fp16 error of the exact
 *   iteration: on two 10-component Gaussian mixtures at 50k x 50k x 512, eps
 *   0.1, 100 iterations, one fp16 iteration gives 3.9e-4 eps (bf16 throughout:
 *   3.2e-3 eps) and the barycentric projection 1.6e-4 relative (bf16
 *   throughout: 1.2e-3); at 50k x 30k x 1024 annealed 1 -> 0.01 over 10 x 20
 *   iterations, an fp16 last stage (refine_iters = 20) gives 8.4e-3 eps and
 *   P.V 8.6e-4 relative, as fp16 throughout (one fp16 iteration: 3.5e-2 eps;
 *   bf16 throughout: 6.4e-2 eps, 1.2e-2).  The bf16 iterations run about 7%
 *   faster than fp16 ones on real data (same instruction rate, less power).
 *   Twice the operand workspace; an fp16 range overflow of a centred
 *   coordinate is reported as for FS_PREC_FP16.  fs_problem_info reports
 *   path 5. */

/* Ground cost.  SQEUCLIDEAN: C_ij = |x_i - y_j|^2.  COSINE: C_ij =
 * 2 - 2 cos(x_i, y_j) = |x_i/|x_i| - y_j/|y_j||^2, the squared-Euclidean
 * cost of the normalised points (the "FlashSinkhorn" explainer, section
 * "Significance and claims", names cosine distance, via normalisation, among
 * the costs the attention form covers); every point must have non-zero
 * length. */
typedef enum { FS_COST_SQEUCLIDEAN = 0, FS_COST_COSINE = 1 } fs_cost;

/* Opaque host handle.  It owns no device memory; it points into the
 * caller's workspace.  Not thread-safe; distinct handles are independent. */
typedef struct fs_problem fs_problem;

/* Solve schedule.  Stage s (0..n_stages-1) uses
 *   eps_s = eps_start * (eps_end/eps_start)^(s/(n_stages-1))   (n_stages > 1),
 *   eps_s = eps_end                                             (n_stages == 1),
 * for iters_per_stage alternating iterations (f-update, then g-update using the
 * new f), carrying f and g across stages.  With tol > 0 the L1 marginal
 * residual  sum_i |sum_j P_ij - a_i| + sum_j |sum_i P_ij - b_j|  of the current
 * (f, g) is evaluated after every check_every-th iteration and the solve stops
 * at the first one <= tol, returning that (f, g).  Both terms are evaluated
 * (each by a dry-run update: two extra half-steps per check; the row term's
 * f-update is then reused as the next iteration's).  warm_start != 0 starts from
 * the f, g passed in (g is what the first f-update reads); otherwise g starts
 * at 0.  Small d <= 8 problems can run the whole fixed-count schedule in one
 * launch (single_launch below): up to 64 workgroups, each holding both clouds
 * in LDS, fp32 vector scores, the potentials of each half-step passed between
 * workgroups as words in the workspace tagged with the half-step's number; a
 * wait that cannot complete (workgroups not resident together) ends the
 * launch with f and g set to NaN.  Two solves of the same problem must not
 * overlap (they share those words). */
typedef struct {
    int32_t n_stages;        /* >= 1 */
    float eps_start;         /* > 0, used when n_stages > 1 */
    float eps_end;           /* > 0 */
    int32_t iters_per_stage; /* >= 0 */
    float tol;               /* <= 0: fixed iteration count, never synchronises */
    int32_t check_every;     /* >= 1 when tol > 0 */
    int32_t warm_start;
    int32_t time_kernels;    /* != 0: time every streaming LSE kernel launch with HIP
                                events on `stream` (synchronises once at the end) */
    int32_t single_launch;   /* the whole schedule as one kernel launch (d <= 8, tol <= 0,
                                at most 32 stages, n + m within the single-launch limit:
                                2389 points for d <= 3, 1433 for d <= 7, 1024 for d = 8):
                                0 = when the problem is also small (n m <= 2^19 pairs),
                                1 = whenever allowed, -1 = never */
    int32_t refine_iters;    /* FS_PREC_BF16_REFINE: the last refine_iters iterations
                                (0 = 1) run on the fp16 copy; >= 0, ignored otherwise */
} fs_solve_opts;

/* Filled on the host by fs_sinkhorn_solve (synchronises at the end when tol > 0). */
typedef struct {
    int32_t iters_done;
    float final_eps;
    float residual;          /* last evaluated residual; -1 if none was evaluated */
    int32_t lse_launches;    /* time_kernels: number of streaming LSE kernels timed */
    float lse_ms;            /* time_kernels: their summed duration in milliseconds
                                (the split-merge pass, when any, is not included) */
    int32_t single_launch;   /* 1 if the schedule ran as one launch, else 0 */
} fs_solve_info;

/* Bytes of workspace needed for a problem of this shape.  dv_max bounds the
 * width of V in later fs_apply_transport calls (0: no transport).  Returns 0
 * for invalid arguments.  Pure host function. */
size_t fs_workspace_bytes(int64_t n, int64_t m, int32_t d, int32_t dv_max,
                          fs_score_prec prec);

/* Creates a problem: copies X (n x d) and Y (m x d) into the workspace after
 * centring each cloud on the midpoint of its own bounding box (nu for X, mu
 * for Y, each computed as (min + max) * 0.5f per coordinate in fp32),
 * converts the centred points x' = x - nu, y' = y - mu (fp32 subtraction) to
 * the score element type, and precomputes the per-point cost terms
 * A_i = |x_i - mu|^2 - |nu - mu|^2/2 and B_j = |y_j - nu|^2 - |nu - mu|^2/2
 * (fp32, from the unrounded points) and the log-weights.  Exactly,
 * C_ij = |x_i - y_j|^2 = A_i + B_j - 2 x'_i.y'_j, so f and g do not depend
 * on the centres.  Writes f = 0
 * and g = 0 (f: n floats, g: m floats; either may be NULL to skip).
 * a (n) and b (m) are the weights; they must be > 0 and finite (sums are used
 * as given).  Synchronises once to read back a validity flag:
 * FS_ERR_NONFINITE if X, Y, a or b holds NaN/Inf or a weight is <= 0.
 * Limits: 1 <= n, m <= 2^31 - 1; 1 <= d <= 1024; dv_max 0..4096. */
fs_status fs_potentials_init(const float* X, const float* Y, const float* a,
                             const float* b, int64_t n, int64_t m, int32_t d,
                             int32_t dv_max, fs_score_prec prec, void* workspace,
                             size_t workspace_bytes, float* f, float* g, void* stream,
                             fs_problem** out);

/* fs_potentials_init with a choice of ground cost.  COSINE normalises the
 * points inside the preparation pass (X and Y are read as given, never
 * written) and otherwise runs the squared-Euclidean path on the unit
 * vectors; the workspace size is the same.  Every later call (updates,
 * solve, transport, gradient) uses that cost; fs_gradient returns the
 * gradient with respect to the points as given, taken back through the
 * normalisation.  FS_ERR_INVALID_ARG for an unknown cost or, for COSINE, a
 * point of zero length. */
fs_status fs_potentials_init_cost(const float* X, const float* Y, const float* a,
                                  const float* b, int64_t n, int64_t m, int32_t d,
                                  int32_t dv_max, fs_score_prec prec, fs_cost cost,
                                  void* workspace, size_t workspace_bytes, float* f, float* g,
                                  void* stream, fs_problem** out);

/* One f-update: f_out_i = -eps LSE_j[(g_j - C_ij)/eps + log b_j], all i.
 * g (m floats) is read, f_out (n floats) is written.  If f_cur (n floats) is
 * given, the row term of the residual of (f_cur, g),
 *   sum_i |sum_j P_ij - a_i| = sum_i a_i |exp((f_cur_i - f_out_i)/eps) - 1|,
 * is written to *row_resid (device, 1 float); row_resid may be NULL.
 * f_out may alias f_cur only when row_resid is NULL. */
fs_status fs_lse_update_f(fs_problem* p, float eps, const float* g, float* f_out,
                          const float* f_cur, float* row_resid, void* stream);

/* One g-update: g_out_j = -eps LSE_i[(f_i - C_ij)/eps + log a_i], all j; with
 * g_cur given, *col_resid = sum_j b_j |exp((g_cur_j - g_out_j)/eps) - 1|, the
 * column term of the residual of (f, g_cur). */
fs_status fs_lse_update_g(fs_problem* p, float eps, const float* f, float* g_out,
                          const float* g_cur, float* col_resid, void* stream);

/* Both terms of the L1 marginal residual of (f, g): out2[0] = row term,
 * out2[1] = column term (device, 2 floats).  Costs two dry-run updates. */
fs_status fs_marginal_residual(fs_problem* p, float eps, const float* f, const float* g,
                               float* out2, void* stream);

/* The alternating solve described at fs_solve_opts, in place on f (n) and g (m).
 * With tol <= 0 it is fully asynchronous.  info may be NULL.  Returns
 * FS_ERR_NOT_CONVERGED (with valid f, g and info) if tol > 0 was not reached. */
fs_status fs_sinkhorn_solve(fs_problem* p, const fs_solve_opts* opts, float* f, float* g,
                            fs_solve_info* info, void* stream);

/* Transport application: U = P.V with V (m x dv) and U (n x dv), P from (f, g)
 * at this eps, or the barycentric projection U_i = (P.V)_i / a_i when
 * divide_by_a != 0.  1 <= dv <= dv_max of the problem; U must not overlap V.
 * On the matrix paths with rows of up to 512 two-byte (256 fp32) values the
 * plan's weights are referred to each row's value of its own update, read
 * from f (no separate LSE pass); rows whose f is far from that value (the
 * weights out of float16 range or too small for its rounding) are found
 * after the pass and recomputed against their score maxima, so any finite
 * (f, g) gives the same accuracy.  The other paths run an exact LSE pass
 * first. */
fs_status fs_apply_transport(fs_problem* p, float eps, const float* f, const float* g,
                             const float* V, int32_t dv, float* U, int32_t divide_by_a,
                             void* stream);

/* Column-side application (the transposed plan): U_j = sum_i P_ij W_i with W
 * (n x dv) and U (m x dv), or U_j / b_j when divide_by_b != 0.  Same limits
 * and error behaviour as fs_apply_transport.  ("FlashSinkhorn" explainer,
 * "Method" part 3: transport-matrix applications as streamed weighted
 * averages.) */
fs_status fs_apply_transport_t(fs_problem* p, float eps, const float* f, const float* g,
                               const float* W, int32_t dv, float* U, int32_t divide_by_b,
                               void* stream);

/* Gradient of the dual objective
 *   D(f, g; X, Y) = <a,f> + <b,g> - eps sum_ij a_i b_j (exp((f_i+g_j-C_ij)/eps) - 1)
 * with respect to the points at fixed (f, g), for C = |x - y|^2:
 *   grad_x_i = 2 sum_j P_ij (x_i - y_j),  grad_y_j = 2 sum_i P_ij (y_j - x_i).
 * At converged potentials this is the gradient of the entropic OT value
 * (envelope theorem); it is the backward pass of the end-to-end workload
 * ("FlashSinkhorn" explainer, "Method" part 3 and "Results").  X (n x d) and
 * Y (m x d) are the fp32 points passed to fs_potentials_init; grad_x (n x d)
 * and grad_y (m x d) are written, either may be NULL, neither may overlap X
 * or Y.  Each output costs one transport application of width d (so the
 * problem needs dv_max >= d, else FS_ERR_INVALID_ARG), which also gives the
 * row sums of P, plus an exact LSE pass before it where fs_apply_transport
 * runs one.
 * The matrix paths carry the transport's relative error (about 1e-3 of the
 * terms); the transported values are the other cloud's points minus its
 * centre, which keeps that error relative to the cloud's spread. */
fs_status fs_gradient(fs_problem* p, float eps, const float* f, const float* g, const float* X,
                      const float* Y, float* grad_x, float* grad_y, void* stream);

/* out[0] (device, one double) = <a,f> + <b,g>, summed in fp64 in a fixed
 * order.  After an f- or g-update the plan's total mass is sum(a) or sum(b),
 * so with equal totals the exponential term of D vanishes and this is the
 * dual value (the entropic OT loss at convergence). */
fs_status fs_dual_value(fs_problem* p, const float* f, const float* g, double* out,
                        void* stream);

/* Streaming Hessian-vector product of the entropic OT loss with respect to
 * one cloud, X below ("FlashSinkhorn" explainer, "Method" part 3: HVPs as
 * sequences of transport-vector and transport-matrix products; the pages
 * give no formula, the one used is implicit differentiation through the
 * Sinkhorn fixed point).  With P the plan of (f, g), r = P 1, c = P^T 1,
 * dC_ij = 2 (x_i - y_j).v_i and dP_ij = P_ij (df_i + dg_j - dC_ij)/eps where
 * (df, dg) keep both marginals of P fixed:
 *   HV_i = 2 r_i v_i + 2 sum_j dP_ij (x_i - y_j).
 * dg solves K dg = w - P^T (u/r), K = diag(c) - P^T diag(1/r) P, by conjugate
 * gradients preconditioned by diag(c), on the complement of the constant
 * vector (K's null space), until
 * the residual falls to cg_tol of its start or cg_max_iter iterations; each
 * iteration is one row and one column transport of width 1.  Besides that:
 * two exact LSE passes, transports of widths d, d+2, d+1, and the second
 * moment sum_j P_ij ((y_j - c).v_i) (y_j - c): one pass of width d on the
 * bf16/fp16 paths with d_pad 64..512 (the direction rows ride along as a
 * second resident block, rounded to the score type after a per-row power-of-
 * two scaling), else the d*d product columns in passes of at most dv_max
 * (so the problem needs dv_max >= d + 2, else FS_ERR_INVALID_ARG).  At converged potentials r = a,
 * c = b and this is the Hessian of the loss; at other potentials it is that
 * of the plan (f, g) define.
 * wrt = 1 gives the Hessian with respect to Y instead (the same with the
 * clouds, weights and potentials exchanged); other values FS_ERR_INVALID_ARG.
 * X (n x d), Y (m x d): the fp32 points given to fs_potentials_init; V, HV:
 * device arrays the shape of the differentiated cloud (HV may not overlap
 * any input or the workspace).
 * workspace: device memory of at least fs_hvp_workspace_bytes(p) bytes,
 * owned by the caller, overwritten.  info (host, nullable): CG iterations and
 * final relative residual.  Squared-Euclidean cost only.  The host waits for
 * the stream twice per CG iteration (the CG scalars).  The transports' f16
 * weights (about 1e-3 relative) bound the accuracy. */
typedef struct {
    int32_t cg_iters;
    float cg_residual;
} fs_hvp_info;
size_t fs_hvp_workspace_bytes(const fs_problem* p);
fs_status fs_hvp(fs_problem* p, float eps, const float* f, const float* g, const float* X,
                 const float* Y, int32_t wrt, const float* V, float* HV, float cg_tol,
                 int32_t cg_max_iter, void* workspace, size_t workspace_bytes, fs_hvp_info* info,
                 void* stream);

/* ---- Block-sparse form for low-dimensional clouds ----------------------
 * "FlashSinkhorn 2: block-sparse entropic optimal transport" (patty.io
 * explainer).  Section on cutting space: points sorted along a Z-order
 * (Morton) curve, so that a run of consecutive points is a compact group and
 * a block of the cost matrix pairs two groups.  Section on guaranteeing the
 * skip: a block is skipped when a bound on its mass is below a threshold
 * that caps, at every iteration, the error the skipped blocks leave in every
 * row and every column.  The page gives no formula; the reading used:
 *
 *  - Morton order: each coordinate is quantised over the cloud's bounding
 *    box to B = floor(30/d) bits (q = min(2^B - 1, floor((x - lo) * scale)),
 *    scale = 2^B / (hi - lo) or 0 for a flat axis, each step one correctly
 *    rounded float32 operation) and bit k of coordinate c becomes bit
 *    k*d + c of the code; points are ordered by code, ties by index.
 *  - Blocks: 256 consecutive rows (one workgroup of the streaming kernel) and
 *    32 consecutive keys (one matrix-core block).  For the f-update with the
 *    current (f, g), every block carries a least-squares linear fit of its
 *    potential; with c_I = max_{i in I} (f_i - u_I.x_i),
 *    G_J = log sum_{j in J} b_j exp((g_j - v_J.y_j)/eps) and
 *    H = max over the two boxes of u_I.x + v_J.y - |x - y|^2,
 *    beta(I, J) = (c_I + H)/eps + G_J bounds log sum_{j in J} P_ij / a_i for
 *    every row i of I.  J is kept for I when beta >= log(delta / N_J) (N_J key
 *    blocks; the kernel keeps a hair more, a rounding margin), else skipped,
 *    so the skipped mass of every row is below delta * a_i.  The g-update is
 *    screened the same way with the clouds exchanged.
 *  - Consequence (the certificate): with f_cur the potential being replaced,
 *    0 <= f_sparse_i - f_dense_i <= eps log(1 + delta exp((f_sparse_i - f_cur_i)/eps)),
 *    about eps * delta near the fixed point.  delta = 0 keeps every block
 *    (the dense update, evaluated block by block).
 *
 * The clouds are expected in Morton order (fs_morton_sort), which only
 * affects how many blocks are skipped, never the bound.
 */

/* Bytes of workspace for fs_morton_sort of n points in d dimensions
 * (1 <= d <= 8); 0 for invalid arguments.  Pure host function. */
size_t fs_morton_workspace_bytes(int64_t n, int32_t d);

/* Sorts the n points X (n x d, device, fp32) into Morton order:
 * X_sorted[i] = X[perm[i]], w_sorted[i] = w[perm[i]] (w, w_sorted: both NULL
 * or both device arrays of n floats), perm (device, n int32).  Outputs may
 * not overlap inputs.  workspace: fs_morton_workspace_bytes(n, d) bytes,
 * 256-byte aligned, overwritten.  Deterministic (a stable radix sort, no
 * atomics outside workgroup-local counters).  Limits: 1 <= n <= 2^31 - 1. */
fs_status fs_morton_sort(const float* X, const float* w, int64_t n, int32_t d, float* X_sorted,
                         float* w_sorted, int32_t* perm, void* workspace, size_t workspace_bytes,
                         void* stream);

/* dst[perm[i] * width + c] = src[i * width + c]: brings per-point results of
 * a sorted problem back to the caller's order (device arrays; dst may not
 * overlap src). */
fs_status fs_unpermute(const float* src, const int32_t* perm, int64_t n, int32_t width,
                       float* dst, void* stream);

/* Workspace of the block-sparse form of a problem (boxes, fits, kept-block
 * lists; the lists take 4 * ceil(n/256) * ceil(m/32) bytes at most, rounded
 * up); 0 if the problem does not qualify.  Pure host function. */
size_t fs_bs_workspace_bytes(const fs_problem* p);

/* Enables the block-sparse form on a problem built by fs_potentials_init on
 * Morton-ordered clouds with d <= 3, FS_PREC_AUTO or FS_PREC_FP32 and the
 * squared-Euclidean cost (else FS_ERR_INVALID_ARG).  workspace:
 * fs_bs_workspace_bytes(p) bytes, 256-byte aligned, owned by the caller,
 * which must outlive the handle's block-sparse calls.  Computes the blocks'
 * boxes and synchronises once (their magnitude).  Up to 2^27 - 544 points
 * per cloud.  Screening is two-level for a key cloud of at least
 * FS_BS_MIN_CHUNKS (environment, read here; default 64, from 2 to 16384)
 * chunks of 8192 keys: a chunk whose own mass bound (the same two fitted
 * forms over its box) is below the threshold is skipped whole, which keeps
 * the per-block guarantee since a block holds at most its chunk's mass; the
 * blocks of the other chunks, and of the chunk of largest bound, are
 * screened one by one. */
fs_status fs_bs_attach(fs_problem* p, void* workspace, size_t workspace_bytes, void* stream);

/* One block-sparse half-step: screening with (f_cur, g), then
 * f_out_i = -eps log sum over the kept blocks' keys of b_j exp((g_j - C_ij)/eps).
 * f_out may be f_cur (in place) unless row_resid is given; row_resid
 * (device float, nullable) receives sum_i a_i |exp((f_cur_i - f_out_i)/eps) - 1|
 * as fs_lse_update_f does.  delta in [0, 1).  The _g form is the mirror
 * image (keys X, weights a). */
fs_status fs_bs_lse_update_f(fs_problem* p, float eps, float delta, const float* g,
                             const float* f_cur, float* f_out, float* row_resid, void* stream);
fs_status fs_bs_lse_update_g(fs_problem* p, float eps, float delta, const float* f,
                             const float* g_cur, float* g_out, float* col_resid, void* stream);

/* fs_sinkhorn_solve with every half-step block-sparse (screened anew each
 * time).  With tol > 0 the residual is that of the retained blocks' plan
 * (within about delta of the dense one).  time_kernels times the streaming
 * kernels only (not the fits and the screening). */
fs_status fs_bs_sinkhorn_solve(fs_problem* p, const fs_solve_opts* opts, float delta, float* f,
                               float* g, fs_solve_info* info, void* stream);

/* The transport U = P.V (divide_by_a: P.V / a, the barycentric projection
 * when V holds the key points) of the block-sparse form: the f-side
 * screening of (f, g) with this delta, then the sum over the kept blocks'
 * keys only.  Since the skipped mass of every row is below delta * a_i,
 * |U_i - U_dense_i| < delta a_i max_j |V_j| per component (delta max |V|
 * after the division).  V (m x dv, the problem's key order, i.e. Morton-
 * ordered like Y), U (n x dv): device fp32, 1 <= dv <= 16, U overlapping no
 * input.  Leaves the f-side lists as the last screening. */
fs_status fs_bs_apply_transport(fs_problem* p, float eps, float delta, const float* f,
                               const float* g, const float* V, int32_t dv, float* U,
                               int32_t divide_by_a, void* stream);

/* The column side: U_j = sum_i P_ij W_i (divide_by_b: / b_j) over the blocks
 * the g-side screening of (f, g) keeps; the same bound with b_j and max|W_i|.
 * W (n x dv, X's order), U (m x dv).  Leaves the g-side lists. */
fs_status fs_bs_apply_transport_t(fs_problem* p, float eps, float delta, const float* f,
                                 const float* g, const float* W, int32_t dv, float* U,
                                 int32_t divide_by_b, void* stream);

/* The gradient of the dual objective at fixed (f, g) in block-sparse form
 * (squared Euclidean cost): grad_x_i = 2 sum_j P_ij (x_i - y_j) over the
 * blocks the f-side screening keeps, grad_y_j = 2 sum_i P_ij (y_j - x_i)
 * over the g-side ones (NULL skips a side).  Sections of the explainer on
 * the streaming gradient and on block sparsity.  Skipped mass below delta
 * a_i bounds the error of grad_x_i by 2 delta a_i max_j |x_i - y_j| per
 * component (the mirror for grad_y).  grad_x (n x d), grad_y (m x d): device
 * fp32 in the problem's (Morton) order, overlapping neither f, g nor each
 * other.  Leaves the lists of the last side computed. */
fs_status fs_bs_gradient(fs_problem* p, float eps, float delta, const float* f, const float* g,
                         float* grad_x, float* grad_y, void* stream);

/* ---- Coarse (centroid) stage ---------------------------------------------
 * "FlashSinkhorn 2" explainer, solving at a coarse resolution first and
 * trusting the lifted solution (no formula on the page; the reading used):
 * cells are runs of `cell` consecutive points of a Morton-ordered cloud (the
 * last may be shorter); the coarse problem is the transport between the two
 * centroid clouds; its potentials are lifted by giving every point its
 * cell's value; a lift is accepted when the relative L1 marginal errors over
 * sampled rows and columns,
 *     sum_{i in S} |r_i - a_i| / sum_{i in S} a_i,  r_i = sum_j P_ij,
 * (exact, against every point of the other cloud) are at most a tolerance,
 * else the coarse iteration continues.  The lift's error is set by the cell
 * size against sqrt(eps), so the fine block-sparse stage finishes the solve. */

/* Centroids C (nc x d, weighted means, fp64 sums in a fixed order) and
 * weights W (nc, sums) of the runs of `cell` points of P (n x d, d <= 8) with
 * weights w; nc = ceil(n / cell).  Device arrays; outputs may not overlap
 * inputs. */
fs_status fs_centroids(const float* P, const float* w, int64_t n, int32_t d, int32_t cell,
                       float* C, float* W, void* stream);

/* f[i] = F[i / cell] for i < n (device arrays). */
fs_status fs_lift(const float* F, int64_t n, int32_t cell, float* f, void* stream);

/* The sampled marginal check of (f, g) on the clouds X (n x d), Y (m x d)
 * with weights a, b (fp32 device arrays, squared-Euclidean cost computed in
 * fp32 from the points): out2[0] = relative L1 error of the rows listed in
 * `rows` (device int32), out2[1] that of the columns in `cols` (device
 * float[2]); an index outside its cloud is clamped into it.  workspace:
 * fs_sampled_workspace_bytes(nrows, ncols) bytes, 256-byte aligned.  Cost:
 * (nrows m + ncols n) d. */
size_t fs_sampled_workspace_bytes(int32_t nrows, int32_t ncols);
fs_status fs_sampled_marginal_error(const float* X, const float* Y, const float* a,
                                    const float* b, int64_t n, int64_t m, int32_t d, float eps,
                                    const float* f, const float* g, const int32_t* rows,
                                    int32_t nrows, const int32_t* cols, int32_t ncols,
                                    float* out2, void* workspace, size_t workspace_bytes,
                                    void* stream);

typedef struct {
    int32_t rounds;    /* checks made */
    int32_t accepted;  /* 1 if the last check passed */
    float err_rows;    /* the last check's relative errors */
    float err_cols;
} fs_coarse_info;

/* The coarse stage: fs_sinkhorn_solve on `coarse` (a problem built by
 * fs_potentials_init on the fs_centroids of both clouds with this `cell`)
 * with `opts` into F, G; then repeatedly lift them into f (n) and g (m),
 * check them on the sampled rows and columns at opts->eps_end, and, unless
 * both errors are at most check_tol or max_rounds checks were made, run
 * more_iters further coarse iterations from (F, G).  Synchronises once per
 * check.  workspace: fs_sampled_workspace_bytes(nrows, ncols) + 256 bytes.
 * f and g are then a warm start for the fine (block-sparse) solve.
 * coarse_delta in [0, 1): 0 solves the coarse problem on the dense path; a
 * positive value runs the coarse solves in block-sparse form
 * (fs_bs_sinkhorn_solve with that delta; the coarse problem must have been
 * attached with fs_bs_attach), which pays once the centroid clouds are large
 * (the centroids of Morton-ordered cells keep that order's locality). */
fs_status fs_bs_coarse_start(fs_problem* coarse, const fs_solve_opts* opts, int32_t more_iters,
                             float coarse_delta,
                             const float* X, const float* Y, const float* a, const float* b,
                             int64_t n, int64_t m, int32_t d, int32_t cell, float check_tol,
                             int32_t max_rounds, const int32_t* rows, int32_t nrows,
                             const int32_t* cols, int32_t ncols, float* F, float* G, float* f,
                             float* g, void* workspace, size_t workspace_bytes,
                             fs_coarse_info* info, void* stream);

/* Introspection (host): side 0 = the f-update (rows X, keys Y), side 1 = the
 * g-update.  fs_bs_shape: block counts and the row stride of the lists.
 * fs_bs_read_screen (synchronises): the kept-block count of every row block
 * from the last screening of that side, and, if lists is non-NULL, the kept
 * key-block indices (increasing, padded to a multiple of 16 with the index
 * of the sentinel block, ceil(keys_padded / 32)) of the last screening, which
 * must be of that side. */
fs_status fs_bs_shape(const fs_problem* p, int32_t side, int32_t* n_row_blocks,
                      int32_t* n_key_blocks, int32_t* list_stride);
fs_status fs_bs_read_screen(fs_problem* p, int32_t side, int32_t* counts, int32_t* lists,
                            void* stream);

/* ---- Allocation-free set-up + solve ------------------------------------
 * For callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, harnesses that forbid hipMalloc): fs_potentials_init
 * followed by fs_sinkhorn_solve, squared-Euclidean cost, no transport buffers,
 * with the workspace in a static device array of the library instead of
 * caller memory.  The caller passes only the inputs (X, Y, a, b) and the
 * outputs (f, g), as for those two calls; nothing is allocated on the device
 * or the host.
 *
 * The array holds FS_STATIC_SCRATCH_BYTES; a problem whose
 * fs_workspace_bytes(n, m, d, 0, prec) exceeds it returns FS_ERR_WORKSPACE
 * before anything is enqueued (fs_static_scratch_bytes() reports the limit).
 * Every GPU the library is loaded on holds one such array for the lifetime
 * of the process; all calls on one GPU share it and each leaves its contents
 * behind, so calls that overlap on one GPU (two streams, two threads) race
 * and must be serialised by the caller.  opts->time_kernels must be 0 (it
 * would create HIP events).  Errors and results as for the two calls it
 * replaces: the set-up's one synchronisation (its validity flag) and, with
 * tol > 0, the residual checks'. */
#define FS_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
size_t fs_static_scratch_bytes(void);
fs_status fs_sinkhorn_solve_static(const float* X, const float* Y, const float* a,
                                   const float* b, int64_t n, int64_t m, int32_t d,
                                   fs_score_prec prec, const fs_solve_opts* opts, float* f,
                                   float* g, fs_solve_info* info, void* stream);

/* Frees the host handle only (the workspace is the caller's). */
void fs_destroy(fs_problem* p);

/* Static text for a status code. */
const char* fs_status_string(fs_status s);

/* Thread-local detail message of the last failing call on this thread. */
const char* fs_last_error(void);

/* Introspection for tests and benchmarks (host): the score path chosen for the
 * problem (0 = fp32 vector, 1 = fp32 matrix, 2 = bf16 matrix, 3 = fp16
 * matrix, 4 = fp32 matrix for d <= 8, 5 = bf16 matrix with fp16 refinement),
 * its padded dimension, and the split count used for the f- and
 * g-update launches. */
fs_status fs_problem_info(const fs_problem* p, int32_t* path, int32_t* d_pad,
                          int32_t* f_splits, int32_t* g_splits);

#ifdef __cplusplus
}
#endif

#endif /* FS_SINKHORN_H */
