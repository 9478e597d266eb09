// fs_internal.h -- declarations shared by the host library and the kernel
// translation units (launchers and their argument blocks).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fs_sinkhorn.h"

namespace fs {

// Score path of a problem.
// PATH_VALU: d <= 8, scores by vector FMA.  PATH_SMALL: d <= 8, scores (bias
// included) on the fp32 matrix cores.  PATH_MFMA_*: padded d on the matrix
// cores in the named element type.
enum Path : int {
    PATH_VALU = 0,
    PATH_MFMA_F32 = 1,
    PATH_MFMA_BF16 = 2,
    PATH_MFMA_F16 = 3,
    PATH_SMALL = 4
};
// Paths that keep the points as fp32 rows of 4 (d <= 4) or 8 floats.
inline bool small_d_path(int path) { return path == PATH_VALU || path == PATH_SMALL; }

// Rows per workgroup of the matrix-core kernels is 4 waves x 32 x qb; clouds are
// padded to a multiple of this so no kernel ever reads past an operand.
constexpr int kRowPad = 512;
// Keys per streamed tile (one 32-row MFMA operand block).
constexpr int kKeyTile = 32;

// One side of the problem, stored in the caller's workspace.
struct Cloud {
    void* ops;      // centred, converted points [n_pad][dp] (fp32 / bf16 / fp16), zero padded
    float* nrm;     // cost term A(x) or B(y) of the centred split [n]
    float* lw2;     // log2 of the weights [n]
    float* w;       // copy of the weights [n]
    int64_t n;
    int64_t n_pad;
    float* l1max = nullptr;  // small-d matrix path: largest L1 norm of a point (device scalar)
    float* rscale = nullptr; // cosine cost: 1/|p_i| [n] (the solver's points are p_i/|p_i|)
};

// Arguments of one streaming log-sum-exp pass ("half-step"): for every row
// point p_i of one cloud, LSE2_i = log2 sum_j 2^(z2_ij) with
//   z2_ij = c_score * (p~_i . q~_j) + beta_j,
//   beta_j = (pot_j - |q~_j|^2) * c_bias + log2 w_j,
// over the key points q_j of the other cloud.  Outputs (finalize stage):
//   mode 0: out_i = out_scale * LSE2_i + |p~_i|^2      (the new potential)
//   mode 1: out_i = LSE2_i
// and, if cur != nullptr, the residual sum_i w_i |2^((cur_i - out_i) c_bias) - 1|.
struct LseArgs {
    const void* rows;
    const float* row_nrm;
    const float* row_w;
    const void* keys;
    const float* key_pot;
    const float* key_nrm;
    const float* key_lw2;
    int n_rows;
    int n_keys;
    int dp;
    float c_bias;     // log2(e) / eps
    float c_score;    // 2 log2(e) / eps
    float out_scale;  // -eps ln 2
    int n_split;      // key-range splits (1: finalize in the streaming kernel)
    int keys_per_split;
    float2* part;     // [n_split][n_rows] partial (M, s) when n_split > 1
    int mode;
    float* out;
    const float* cur;
    float* resid_part;  // one partial per finalizing block
    float* resid_out;   // 1 float
    // PATH_SMALL (workspace): key records of this pass, fp32 [krec_keys][2*kp]
    // and, for d <= 4, fp16-split [krec_keys][16] and bf16 three-part
    // [krec_keys][32]; two guard words.
    float* krec;
    void* krec16;
    void* krec3;
    void* krec_guard;
    int krec_keys;      // records packed (the key cloud's padded count)
    const float* row_l1;  // largest L1 norm of a row point (device scalar)
    // 1024-wide split-contraction kernel (workspace): key biases in
    // dot-product units of this pass [keys' padded count]
    float* kbias;
    int kbias_keys;
    // block-sparse form (PATH_SMALL, d <= 3; see fs_bsparse.hip): per row
    // block of 256 rows, the kept 32-key blocks [row blocks][bs_cap] padded to
    // whole tiles of 16 with bs_sentinel (the block of -inf records right
    // after the padded keys), and their count.  NULL: the dense pass.  A row
    // block with S splits (bs_nsplit) has its list's tiles s, s + S, s + 2S, ..
    // taken by the workgroup of split s, which writes a partial (M, s) like a
    // key-range split (n_split > 1 then only marks the partial form).
    const int* bs_list;
    const int* bs_count;
    const int* bs_best;  // per row block: the block whose scores set the starting reference
    const float4* bs_org;  // per row block: origin and fp16-format flag (see fs_bsparse.hip)
    // work plan (launch_split_plan): per row block its split count, per
    // workgroup its (row block, split), the number of planned workgroups,
    // and the grid launched (an upper bound; the rest exit at once).  Partials
    // go to part[split][n_rows] and the merge takes bs_nsplit[row / 256].
    const int* bs_nsplit;
    const int* bs_map;
    const int* bs_total;
    int bs_grid;
    int bs_cap;
    int bs_sentinel;
};

// Arguments of the transport application U = P.V (or P.V / a).
// Where the streaming transport kernel takes each row's reference R (its
// weights are 2^(z2 - R)): the exact LSE2 it is given, minus a slack; the
// row potential's value of it (R = (|x~|^2 - f) c_bias - slack, the LSE2 of
// the f-update that produced f), moved up lazily when a tile's scores exceed
// it; or, in the repair pass, the row's score maximum found by the first pass.
enum TransportRef : int { REF_GIVEN = 0, REF_ONLINE = 1, REF_REPAIR = 2 };

constexpr int kTransportMaxSplit = 4;

struct TransportArgs {
    const void* rows;        // X~ [n_pad][dp]
    const float* row_lse2;   // exact LSE2 of each row under the current g (REF_GIVEN)
    const float* row_pot;    // f
    const float* row_nrm;    // rows' cost term (A(x) for X, B(y) for Y)
    const float* row_w;      // a
    const void* keys;        // Y~ [m_pad][dp]
    const float* key_pot;    // g
    const float* key_nrm;    // keys' cost term
    const float* key_lw2;    // log2 b
    const float* V;          // fp32 [m][dv] (vector path)
    const float* v_off;      // nullable [dv]: the product uses V - v_off (row-broadcast)
    const float* v_rscale;   // nullable [keys]: ... and V_j * v_rscale[j] before the offset
    const void* Vt;          // f16 [dv][m_pad] scaled copy (matrix path)
    const float* v_unscale_dev;  // device float 2^-s undoing the copy's scaling
    int n_rows, n_keys, dp, dv;
    float c_bias, c_score;
    int divide_by_a;
    float* U;                // [n][dv]
    // streaming matrix kernel (d_pad <= 512 for 2-byte types)
    const float* key_bias;   // [m_pad] key biases in dot-product units (-inf padding)
    float* U_part;           // [n_split][n][dv] partial products of the key ranges
    int64_t part_stride;     // n * dv
    int n_split;             // key ranges (1: U written directly)
    int keys_per_split;      // multiple of 32 (1024-wide kernel: equal ranges)
    // streaming kernel: range s is key tiles [split_tile[s], split_tile[s+1])
    // (longest first); its work units are (row block, column block) pairs
    int split_tile[kTransportMaxSplit + 1];
    int n_units;
    // second-moment form (Hessian-vector product): direction rows in the
    // score type [n_pad][dp], or NULL for a plain transport
    const void* rows2;
    // streaming kernel's references (NULL: the other kernels, which take
    // row_lse2 as it is): per key range and row, the final reference R, the
    // sum of the weights relative to it and the score maximum (base 2)
    int ref_mode;            // TransportRef
    float* row_ref;          // [n_split][n]
    float* row_sum;          // [n_split][n]
    float* row_max;          // [n_split][n]
    int* row_flag;           // [n] rows the repair pass recomputes
    float* lse_out;          // nullable [n]: each row's LSE2, R + log2(sum)
};

// ---- launchers (each returns the first HIP error, enqueues on `s`) ----
hipError_t launch_zero_flag(int* flag, hipStream_t s);
// xscale / yscale / rscale (nullable): per-point factors applied on reading
// (1/|p| for the cosine cost)
hipError_t launch_inv_norm(const float* P, int64_t n, int d, float* inv, int* flag,
                           hipStream_t s);
hipError_t launch_bbox(const float* X, const float* xscale, int64_t n, const float* Y,
                       const float* yscale, int64_t m, int d, float* part_min, float* part_max,
                       int parts_per_cloud, float* centres, hipStream_t s);
hipError_t launch_convert(const float* P, const float* rscale, int64_t n, int64_t n_pad, int d,
                          int dp, int path, const float* own_centre, const float* other_centre,
                          void* ops, float* nrm, int* flag, hipStream_t s);
// The preparation of a small squared-Euclidean problem with fp32 operands
// (d <= 8) in two launches: both centres, then every row's operand, cost
// term, L1 norm (into xl1 / yl1 when non-null) and weight terms, with the
// same arithmetic as the separate kernels.  Clears the flag and the L1 words.
struct SmallPrepArgs {
    const float *X, *Y, *a, *b;
    int64_t n, m, n_pad, m_pad;
    int d, dp;
    float* centre;  // [2][d]
    float *xops, *yops, *xn, *yn, *xlw, *ylw, *xw, *yw;
    float *f, *g;      // zeroed when non-null
    float *xl1, *yl1;  // nullable
    int* flag;
};
hipError_t launch_prep_small(const SmallPrepArgs& a, hipStream_t s);
hipError_t launch_weights(const float* w, int64_t n, float* lw2, float* wcopy, float* pot,
                          int* flag, hipStream_t s);
hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t s);

// ---- gradient pieces and dual value (fs_grad.hip) ----
// rscale (nullable): cosine cost -- the points are P_i rscale_i, and the
// gradient is taken back through that normalisation
hipError_t launch_grad_finish(const float* P, const float* rscale, const float* c,
                              const float* lse2, const float* pot, const float* nrm,
                              const float* w, float c_bias, int64_t n, int d, float* G,
                              hipStream_t s);
// streaming Hessian-vector product (fs_hvp.hip)
hipError_t launch_marginal(const float* lse2, const float* pot, const float* nrm, const float* w,
                           float c_bias, int64_t n, float* out, hipStream_t s);
hipError_t launch_hvp_rows(const float* X, const float* V, const float* mu, const float* PY,
                           const float* r, int64_t n, int d, float* u, float* W, hipStream_t s);
hipError_t launch_hvp_cols(const float* Y, const float* mu, const float* PtW, int64_t m, int d,
                           float* rhs, hipStream_t s);
hipError_t launch_dot(const float* x, const float* y, int64_t len, double* out, hipStream_t s);
hipError_t launch_axpby(float alpha, const float* x, float beta, float* y, int64_t len,
                        const double* shift, double shift_scale, hipStream_t s);
hipError_t launch_scale_sub(const float* a, const float* x, const float* y, int64_t len,
                            int divide, float* out, hipStream_t s);
hipError_t launch_hvp_dgy(const float* Y, const float* mu, const float* dg, int64_t m, int d,
                          float* V2, hipStream_t s);
hipError_t launch_hvp_outer(const float* Y, const float* mu, int64_t m, int d, int64_t q0, int w,
                            float* V3, hipStream_t s);
hipError_t launch_hvp_moment(const float* T3, const float* V, int64_t n, int d, int64_t q0, int w,
                             float* M, hipStream_t s);
hipError_t launch_hvp_final(const float* V, const float* r, const float* u, const float* W,
                            const float* PY, const float* T, const float* M,
                            const float* m_scale, int64_t n, int d, float inv_eps, float* HV,
                            hipStream_t s);
hipError_t launch_hvp_vconv(int path, const float* V, int64_t n, int64_t n_pad, int d, int dp,
                            void* out, float* inv_sigma, hipStream_t s);
hipError_t launch_dual_value(const float* a, const float* f, int64_t n, const float* b,
                             const float* g, int64_t m, double* out, hipStream_t s);

// ---- throughput probes (fs_probe.hip) ----
int probe_blocks();  // workgroups per probe launch on the current device; 0 on error
double probe_work_per_launch(int kind, int blocks);  // flops or exponentials
hipError_t launch_probe(int kind, int blocks, float* sink, hipStream_t s);

// Streaming LSE pass (+ merge when split).  `path` selects the kernel family,
// `dp` the padded dimension.
// ev_begin/ev_end (may be null) are recorded on `s` right before and after
// the streaming kernel (not around the merge).
hipError_t launch_lse(int path, const LseArgs& a, hipStream_t s, hipEvent_t ev_begin = nullptr,
                      hipEvent_t ev_end = nullptr);
// Rows handled by one workgroup of the streaming kernel (path, dp as passed
// in LseArgs, rows of the pass).
int lse_rows_per_block(int path, int dp, int n_rows);
// Largest key range one workgroup of the streaming kernel may cover (its key
// biases are held in LDS).
int lse_max_keys_per_split(int path, int dp);
// true when the pass runs the split-contraction kernel for 1024-wide two-byte
// rows, which needs LseArgs::kbias (one float per padded key)
bool lse_wide(int path, int dp);
// Key-range granularity of a split (keys per streamed tile).
int lse_split_granule(int path, int dp);

// PATH_SMALL: key-record slot pairs for dimension d, keys per streamed tile,
// rows per workgroup; the streaming kernel (after packing the key records);
// ev_begin is recorded after the packing.
int small_kp(int d);
int small_tile(int d);
int small_rows_per_block();
size_t small_f32_rec_bytes(int d);  // per key
size_t small_f16_rec_bytes(int d);  // per key (0 if d > 4)
size_t small_b3_rec_bytes(int d);   // per key (0 if d > 4)
// Largest L1 norm over the (converted, fp32) points of a cloud into *out.
hipError_t launch_row_l1max(const float* ops, int64_t n, int d, float* out, hipStream_t s);
hipError_t launch_lse_small(const LseArgs& a, hipStream_t s, hipEvent_t ev_begin);
// the block-sparse form (a.bs_list set, d <= 3; the key records must hold the
// sentinel block: a.krec_keys = padded keys + 32; a.part must hold
// a.n_split * n_rows partials when a.n_split > 1)
hipError_t launch_lse_small_sparse(const LseArgs& a, hipStream_t s, hipEvent_t ev_begin);

// ---- block-sparse low-dimensional path (fs_bsparse.hip) ----
// Bits per coordinate of the Morton code (30 / d).
int morton_bits(int d);
size_t morton_workspace_bytes(int64_t n);
// Sorts the n points of X (n x d, d <= 8) by Morton code (ties by index) into
// Xo, gathers w (nullable) into wo, and writes the permutation (Xo[i] =
// X[perm[i]]).  ws: morton_workspace_bytes(n) bytes, 256-aligned.
hipError_t launch_morton_sort(const float* X, const float* w, int64_t n, int d, float* Xo,
                              float* wo, int32_t* perm, void* ws, hipStream_t s);
// dst[perm[i]] = src[i] for rows of `width` floats.
hipError_t launch_unpermute(const float* src, const int32_t* perm, int64_t n, int width,
                            float* dst, hipStream_t s);
// Boxes (lo, hi) of the blocks of gs (32 or 256) consecutive points of a cloud
// stored as centred fp32 rows of 4 (plus its centre).
hipError_t launch_block_boxes(const float* ops, const float* centre, int d, int64_t n, int gs,
                              float4* box, hipStream_t s);
// Per-block linear fits of a potential p and of p - |x|^2 into fit[2*blk]
// and fit[2*blk+1]: rows (gs 256, key false) -> (u, c), keys (gs 32, key
// true) -> (v, G) with G in base 2 (uses lw2 and c_bias).
hipError_t launch_block_fit(const float* ops, const float* centre, int d, int64_t n, int gs,
                            bool key, const float* pot, const float* lw2, float c_bias,
                            float4* fit, hipStream_t s);
// Coarse stage: centroids (weighted means) and weights of runs of `cell`
// points (d <= 8); the lift f[i] = F[i / cell]; the sampled marginal check
// (out2 = relative L1 marginal error over the sampled rows, then columns;
// part: nrows + ncols float2 of scratch).
hipError_t launch_centroids(const float* P, const float* w, int64_t n, int d, int cell,
                            float* C, float* W, hipStream_t s);
hipError_t launch_lift(const float* F, int64_t n, int cell, float* f, hipStream_t s);
hipError_t launch_sampled_marginal(const float* X, const float* Y, const float* a,
                                   const float* b, int64_t n, int64_t m, int d, float c_bias,
                                   const float* f, const float* g, const int32_t* rows,
                                   int nrows, const int32_t* cols, int ncols, float2* part,
                                   float* out2, hipStream_t s);
// Transport U = P.V (dv <= 16) over the kept blocks of a screening (list/
// count/cap of nbR row blocks of 256; rows and keys as fp32 rows of 4).  With
// V == NULL it is the gradient form: U_i = 2 sum_j P_ij (x_i - y_j), dv = d <= 3,
// cR/cK the centres the rows and keys were taken about.
hipError_t launch_bs_transport(const float* rows, const float* row_nrm, const float* row_lw2,
                               const float* row_pot, const float* row_w, int n_rows,
                               const float* keys, const float* key_nrm, const float* key_lw2,
                               const float* key_pot, int n_keys, const float* V, int dv,
                               float c_bias, float c_score, int divide, const int* list,
                               const int* count, int cap, int nbR, const float* cR,
                               const float* cK, float* U, hipStream_t s);
// Work plan of the retained-block pass from the kept counts (see LseArgs).
hipError_t launch_split_plan(const int* count, int nbR, int target, int smax, int* nsplit,
                             int* map, int* total, hipStream_t s);
// Kept key blocks of every row block (threshold thr2 = log2(delta / nbK)),
// their count, and the key block of largest bound.
// Also the row block's origin for shifted fp16 operands and its format flag
// (org[2I], org[2I+1]; cR, cK: the row and key clouds' centres).
// Two-level screening: chunks of kChunkKeys keys (256 key blocks of 32), at
// most kMaxChunks of them (the screening keeps one flag per chunk in LDS).
constexpr int kChunkKeys = 8192;
constexpr int kMaxChunks = 16384;
// Boxes and key-side fits of the chunks of a cloud (n keys, ceil(n /
// kChunkKeys) <= kMaxChunks chunks).
hipError_t launch_chunk_fit(const float* ops, const float* centre, int d, int64_t n,
                            const float* pot, const float* lw2, float c_bias, float4* cbox,
                            float4* cfit, hipStream_t s);
// nbC > 0 (= ceil(nbK / 256)): skip the chunks whose own bound is below the
// threshold before screening the blocks of the others.
hipError_t launch_screen(const float4* rbox, const float4* rfit, int nbR, const float4* kbox,
                         const float4* kfit, int nbK, float c_bias, float thr2, float mag,
                         int* list, int* count, int* best, const float* cR, const float* cK,
                         int d, float4* org, int cap, int sentinel, const float4* cbox,
                         const float4* cfit, int nbC, hipStream_t s);

// Transport: V -> f16 transposed scaled copy, then the streaming product.
// Matrix paths: the streaming transport kernel serves operand rows of up to
// 512 two-byte (or 256 fp32) values and may split the key range into up to
// kTransportMaxSplit parts (kTransportMaxSplit is defined above
// TransportArgs), whose partial products need n * dv floats each.
bool transport_streams(int path, int dp);
// True when launch_transport with these shapes runs the streaming kernel with
// references of its own (REF_ONLINE: no LSE pass needed before it).
bool transport_online(int path, int dp, int dv, int64_t m_pad, bool moment);
// ref_buf: 3 * kTransportMaxSplit * n_rows floats + n_rows ints (streaming
// kernel only).  With a.ref_mode == REF_ONLINE the launch runs the first
// pass, marks the rows whose weights came out too small for their float16
// rounding (all far below the reference: a row potential far from its
// update's), recomputes their row blocks from the score maxima, then merges.
hipError_t launch_transport(int path, const TransportArgs& a, float* vmax_scratch,
                            void* Vt_buf, int64_t m_pad, float* key_bias_buf, float* part_buf,
                            float* ref_buf, hipStream_t s);

// The whole alternating schedule of a small d <= 8 problem in one launch
// (fs_persistent.hip): W <= 64 workgroups, each holding both clouds in LDS,
// exchanging the potentials of each half-step as tagged words.  X, Y: the
// problem's fp32 operand rows (stride floats apart); xn, yn: cost terms A, B;
// xl, yl: log2 weights; f, g: the potentials (g read first, unless g_zero:
// then the first f-update takes g = 0 and g is only written); tf [n], tg [m]:
// zeroed tagged copies of f and g; err: a zeroed word.
constexpr int kPersistentMaxStages = 32;
struct PersistentArgs {
    const float* X;
    const float* Y;
    const float* xn;
    const float* yn;
    const float* xl;
    const float* yl;
    float* f;
    float* g;
    int n, m, d, stride, W, n_stages, iters, g_zero;
    float eps[kPersistentMaxStages];
    unsigned long long* tf;
    unsigned long long* tg;
    int* err;
};
hipError_t launch_solve_persistent(const PersistentArgs& a, hipStream_t s);
// whether an n x m problem in d dimensions fits the persistent solve (both
// clouds within one workgroup's 64 KiB of LDS)
bool persistent_fits(int64_t n, int64_t m, int d);
int persistent_workgroups(int64_t n, int64_t m);

// Sets the thread's fs_last_error() message and returns s.
fs_status report(fs_status s, const char* msg);

// Set-up and alternating solve in one call with every device buffer in
// `workspace` and the problem struct on the stack (fs_api.cpp): the body of
// the allocation-free entry point, which passes its static scratch array.
fs_status solve_in_workspace(const float* X, const float* Y, const float* a, const float* b,
                             int64_t n, int64_t m, int32_t d, fs_score_prec prec,
                             const fs_solve_opts* opts, void* workspace, size_t workspace_bytes,
                             float* f, float* g, fs_solve_info* info, void* stream);

}  // namespace fs
