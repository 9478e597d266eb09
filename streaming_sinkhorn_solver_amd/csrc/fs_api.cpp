// fs_api.cpp -- host side of the C ABI declared in include/fs_sinkhorn.h:
// argument validation, workspace layout, path and launch-shape selection, and
// the alternating solve loop (one stream, no host round trips unless a
// residual stop was asked for).
//
// The iteration follows "FlashSinkhorn: IO-Aware Entropic Optimal Transport
// on GPU" (gist.science explainer), section "Method", part 1 (the f-update and
// its mirror g-update, alternated); the annealing and residual stop are the
// schedule options of fs_solve_opts.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <string>
#include <utility>
#include <vector>

#include "fs_internal.h"
#include "fs_probe.h"
#include "fs_sinkhorn.h"

using namespace fs;

struct fs_problem {
    int device;
    int cost;  // fs_cost
    int path;
    // FS_PREC_BF16_REFINE: the fp16 copies of the operands and their path;
    // RefineScope exchanges them with X.ops, Y.ops and path while a pass
    // that is to run in fp16 is enqueued
    bool refine = false;
    void* xops16 = nullptr;
    void* yops16 = nullptr;
    int path16 = -1;
    int64_t n, m;
    int d;       // true dimension
    int dp;      // operand row stride in elements
    int lse_dp;  // the dp value passed to the LSE/transport launchers
    int dv_max;
    int f_split, f_kps;  // split count / keys per split of the f-update (rows X, keys Y)
    int g_split, g_kps;
    Cloud X, Y;
    float* centre;  // [2][d]: centre of X, then of Y
    float* bbox_min;
    float* bbox_max;
    int* flag;
    float2* part;
    float* resid_part;
    float* scal;      // [0..1] residual outputs, [2..4] transport scale pair and max bits
    float* pot_tmp;   // max(n, m) floats
    void* vt;         // f16 [dv_max][m_pad] (matrix paths with dv_max > 0)
    float* kbias;     // [m_pad] key biases of the streaming transport kernel
    float* lbias;     // [max(n_pad, m_pad) + 256] key seeds of the matrix-core LSE kernels
    unsigned long long* ptag;  // [n + m + 1] single-launch solve (small d): tagged f, g, error
    float* upart;     // [kTransportMaxSplit][n][dv_max] its partial products
    float* uref;      // its row references, weight sums, maxima [3][kTransportMaxSplit][n], flags [n]
    float* krec;      // small-d matrix path: key records of one pass (fp32)
    void* krec16;     //   fp16-split records (d <= 4)
    void* krec3;      //   bf16 three-part records (d <= 4)
    void* kguard;     //   guard words of the packing
    // block-sparse form (fs_bs_attach): side 0 = rows X / keys Y (f-update),
    // side 1 = rows Y / keys X (g-update)
    bool bs_on = false;
    int bs_nbR[2] = {0, 0}, bs_nbK[2] = {0, 0}, bs_cap[2] = {0, 0};
    float4* bs_rbox[2] = {nullptr, nullptr};  // [nbR][2] (lo, hi) of 256-row blocks
    float4* bs_kbox[2] = {nullptr, nullptr};  // [nbK][2] of 32-key blocks
    float4* bs_rfit = nullptr;                // per pass: [2] fits (u, c) of the row blocks
    float4* bs_kfit = nullptr;                // per pass: [2] fits (v, G) of the key blocks
    float4* bs_cbox = nullptr;                // per pass: [2] boxes of the key chunks
    float4* bs_cfit = nullptr;                // per pass: [2] fits (v, G) of the key chunks
    int bs_min_chunks = 64;                   // two-level screening from this many chunks
    int* bs_cnt[2] = {nullptr, nullptr};      // kept blocks per row block, last pass of a side
    int* bs_best = nullptr;                   // per row block: the block of largest bound
    float4* bs_org = nullptr;                 // per row block: [2] origin and format flag
    int* bs_nsplit = nullptr;                 // work plan: splits per row block
    int* bs_map = nullptr;                    //   (row block, split) per workgroup
    int* bs_total = nullptr;                  //   planned workgroups
    int* bs_list = nullptr;                   // kept blocks of the last pass
    float2* bs_part = nullptr;                // [kBsMaxSplit][max(n, m)] partials
    int bs_last_side = -1;
    float bs_mag = 1.f;                       // coordinate magnitude of the rounding margin
};

namespace {

thread_local std::string g_err;

fs_status fail(fs_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

fs_status hip_fail(hipError_t e, const char* where) {
    return fail(FS_ERR_DEVICE, "%s: HIP error %d (%s)", where, (int)e, hipGetErrorString(e));
}

constexpr int kBboxParts = 64;
// preparation in two launches (launch_prep_small) up to this many points in
// both clouds: one workgroup per cloud forms its centre
constexpr int64_t kSmallPrepPoints = 32768;
constexpr size_t kAlign = 256;

size_t up(size_t v, size_t a) { return (v + a - 1) / a * a; }
int64_t pad_rows(int64_t n) { return (n + kRowPad - 1) / kRowPad * kRowPad; }
int next_pow2(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

struct Shape {
    int path = -1;
    int dp = 0;      // stride
    int lse_dp = 0;  // launcher dp
    size_t es = 4;   // element size
    int f_split = 1, f_kps = 0, g_split = 1, g_kps = 0;
    bool refine = false;  // FS_PREC_BF16_REFINE: an fp16 copy of the operands too
};

// Returns FS_OK and fills sh, or an error.
fs_status choose_path(int64_t n, int64_t m, int32_t d, int32_t dv_max, fs_score_prec prec,
                      Shape& sh) {
    if (n < 1 || m < 1 || n > 0x7fffffffLL || m > 0x7fffffffLL)
        return fail(FS_ERR_INVALID_ARG, "n and m must be in [1, 2^31-1] (got n=%lld, m=%lld)",
                    (long long)n, (long long)m);
    if (d < 1 || d > 1024)
        return fail(FS_ERR_INVALID_ARG, "d must be in [1, 1024] (got %d)", d);
    if (dv_max < 0 || dv_max > 4096)
        return fail(FS_ERR_INVALID_ARG, "dv_max must be in [0, 4096] (got %d)", dv_max);
    switch (prec) {
        case FS_PREC_FP32_VALU:
            if (d > 8)
                return fail(FS_ERR_INVALID_ARG, "FS_PREC_FP32_VALU supports d <= 8 (got %d)", d);
            sh.path = PATH_VALU;
            sh.dp = d <= 4 ? 4 : 8;
            sh.lse_dp = d;
            sh.es = 4;
            break;
        case FS_PREC_AUTO:
        case FS_PREC_FP32:
            if (d <= 8) {
                sh.path = PATH_SMALL;
                sh.dp = d <= 4 ? 4 : 8;
                sh.lse_dp = d;
                sh.es = 4;
            } else if (d <= 512) {
                sh.path = PATH_MFMA_F32;
                sh.dp = 8 * next_pow2((d + 7) / 8);
                sh.lse_dp = sh.dp;
                sh.es = 4;
            } else {
                return fail(FS_ERR_INVALID_ARG,
                            "fp32 scores support d <= 512 (got %d); use FS_PREC_BF16 or FS_PREC_FP16",
                            d);
            }
            break;
        case FS_PREC_BF16_REFINE:
            if (d <= 8)
                return fail(FS_ERR_INVALID_ARG,
                            "FS_PREC_BF16_REFINE needs d > 8 (got %d): the d <= 8 paths score "
                            "in fp32", d);
            sh.refine = true;
            [[fallthrough]];
        case FS_PREC_BF16:
        case FS_PREC_FP16:
            sh.path = prec == FS_PREC_FP16 ? PATH_MFMA_F16 : PATH_MFMA_BF16;
            sh.dp = 16 * next_pow2((d + 15) / 16);
            sh.lse_dp = sh.dp;
            sh.es = 2;
            break;
        default:
            return fail(FS_ERR_INVALID_ARG, "unknown fs_score_prec %d", (int)prec);
    }
    return FS_OK;
}

// Key-range split so that (row blocks x splits) fills the GPU in a near-whole
// number of rounds, preferring few splits, with every split no larger than
// the kernel's key-range limit.
void choose_split(int path, int lse_dp, int64_t n_rows, int64_t n_keys, int& S_out,
                  int& kps_out) {
    const int rpb = lse_rows_per_block(path, lse_dp, (int)n_rows);
    const int64_t R = (n_rows + rpb - 1) / rpb;
    const int slots = path == PATH_VALU ? 1024 : path == PATH_SMALL ? 512 : 256;
    const int tile = lse_split_granule(path, lse_dp);
    const int64_t min_keys = small_d_path(path) ? 2048 : 256;
    const int64_t max_keys = lse_max_keys_per_split(path, lse_dp);
    int bestS = -1;
    int64_t bestK = 0;
    double best = -1.0;
    for (int S = 1; S <= 4096; ++S) {
        const int64_t kps = ((n_keys + S - 1) / S + tile - 1) / tile * tile;
        if (kps > max_keys) continue;
        if (S > 1 && kps < min_keys && bestS > 0) break;
        const int64_t Se = (n_keys + kps - 1) / kps;
        if (Se != S) continue;
        const int64_t blocks = R * Se;
        const int64_t rounds = (blocks + slots - 1) / slots;
        const double eff = (double)blocks / (double)(rounds * slots);
        const double score = eff - 0.003 * (double)(Se - 1);
        if (score > best + 1e-12) {
            best = score;
            bestS = (int)Se;
            bestK = kps;
        }
        if (S >= 64 && bestS > 0) break;
    }
    S_out = bestS;
    kps_out = (int)bestK;
}

struct Layout {
    size_t centre, bmin, bmax, flag, xops, yops, xops16, yops16, xn, xl, xw, yn, yl, yw, part, rpart, scal, ptmp,
        vt, kbias, upart, uref, krec, krec16, krec3, kguard, rsx, rsy, lbias, ptag, total;
};

Layout make_layout(int64_t n, int64_t m, int d, int dv_max, const Shape& sh) {
    Layout L{};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = up(o + bytes, kAlign);
        return at;
    };
    const int64_t np = pad_rows(n), mp = pad_rows(m);
    L.centre = take(sizeof(float) * 2 * d);
    L.bmin = take(sizeof(float) * 2 * kBboxParts * d);
    L.bmax = take(sizeof(float) * 2 * kBboxParts * d);
    L.flag = take(sizeof(int) * 4);
    L.xops = take(sh.es * (size_t)np * sh.dp);
    L.yops = take(sh.es * (size_t)mp * sh.dp);
    L.xops16 = take(sh.refine ? sh.es * (size_t)np * sh.dp : 0);
    L.yops16 = take(sh.refine ? sh.es * (size_t)mp * sh.dp : 0);
    L.xn = take(sizeof(float) * n);
    L.xl = take(sizeof(float) * n);
    L.xw = take(sizeof(float) * n);
    L.yn = take(sizeof(float) * m);
    L.yl = take(sizeof(float) * m);
    L.yw = take(sizeof(float) * m);
    const size_t part_elems = std::max((size_t)(sh.f_split > 1 ? sh.f_split * n : 0),
                                       (size_t)(sh.g_split > 1 ? sh.g_split * m : 0));
    L.part = take(sizeof(float2) * (part_elems > 0 ? part_elems : 1));
    L.rpart = take(sizeof(float) * ((std::max(n, m) + 127) / 128 + 64));
    L.scal = take(sizeof(float) * 8);
    L.ptmp = take(sizeof(float) * std::max(n, m));
    const bool vt = dv_max > 0 && !small_d_path(sh.path);
    // transport buffers serve both sides (keys Y for P.V, keys X for P^T.W)
    const size_t kp = (size_t)std::max(np, mp);
    L.vt = take(vt ? (size_t)2 * dv_max * kp : 0);
    const bool streams = vt && transport_streams(sh.path, sh.lse_dp);
    L.kbias = take(streams ? sizeof(float) * kp : 0);
    L.upart = take(streams ? sizeof(float) * kTransportMaxSplit * (size_t)std::max(n, m) * dv_max
                           : 0);
    L.uref = take(streams ? sizeof(float) * (3 * kTransportMaxSplit + 1) * (size_t)std::max(n, m)
                          : 0);
    const bool small = sh.path == PATH_SMALL;
    const size_t kmax = (size_t)std::max(np, mp);
    // (+32 records: the -inf sentinel block of the block-sparse form)
    L.krec = take(small ? small_f32_rec_bytes(d) * (kmax + 32) : 0);
    L.krec16 = take(small ? small_f16_rec_bytes(d) * (kmax + 32) : 0);
    L.krec3 = take(small ? small_b3_rec_bytes(d) * (kmax + 32) : 0);
    L.kguard = take(small ? 32 : 0);  // packing guard [2], cloud L1 maxima [2]
    L.rsx = take(sizeof(float) * n);  // cosine cost: 1/|x_i|
    L.rsy = take(sizeof(float) * m);
    // key seeds of the matrix-core LSE kernels, plus one 256-key slice of
    // padding for the copy of a split's seeds to LDS
    L.lbias = take(!small_d_path(sh.path) ? sizeof(float) * (kmax + 256) : 0);
    // single-launch solve: the tagged potentials of both sides and an error word
    L.ptag = take(small_d_path(sh.path) && persistent_fits(n, m, d)
                      ? sizeof(unsigned long long) * (size_t)(n + m + 1)
                      : 0);
    L.total = o;
    return L;
}

fs_status plan(int64_t n, int64_t m, int32_t d, int32_t dv_max, fs_score_prec prec, Shape& sh,
               Layout& L) {
    fs_status st = choose_path(n, m, d, dv_max, prec, sh);
    if (st != FS_OK) return st;
    choose_split(sh.path, sh.lse_dp, n, m, sh.f_split, sh.f_kps);
    choose_split(sh.path, sh.lse_dp, m, n, sh.g_split, sh.g_kps);
    L = make_layout(n, m, d, dv_max, sh);
    return FS_OK;
}

fs_status check_device(int* dev_out) {
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess || count < 1) return fail(FS_ERR_DEVICE, "no HIP device available");
    int dev = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return hip_fail(e, "hipGetDevice");
    hipDeviceProp_t prop;
    if ((e = hipGetDeviceProperties(&prop, dev)) != hipSuccess)
        return hip_fail(e, "hipGetDeviceProperties");
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(FS_ERR_DEVICE, "device %d is %s; this library is built for gfx950 only", dev,
                    prop.gcnArchName);
    *dev_out = dev;
    return FS_OK;
}

bool finite_pos(float v) { return std::isfinite(v) && v > 0.f; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const char* x = (const char*)a;
    const char* y = (const char*)b;
    return x < y + nb && y < x + na;
}

// While alive (and `on`), passes enqueued on p use the fp16 copies of a
// FS_PREC_BF16_REFINE problem: its operands and path are exchanged with the
// fp16 ones and put back at the end of the scope.  (Handles are not
// thread-safe, and every pass reads these fields when it is enqueued.)
struct RefineScope {
    fs_problem* p;
    bool active;
    RefineScope(fs_problem* p_, bool on = true) : p(p_), active(on && p_ && p_->refine) {
        if (active) swap();
    }
    ~RefineScope() {
        if (active) swap();
    }
    void swap() {
        std::swap(p->X.ops, p->xops16);
        std::swap(p->Y.ops, p->yops16);
        std::swap(p->path, p->path16);
    }
};

LseArgs base_args(const fs_problem* p, bool f_side, float eps) {
    LseArgs a{};
    const Cloud& R = f_side ? p->X : p->Y;
    const Cloud& K = f_side ? p->Y : p->X;
    a.rows = R.ops;
    a.row_nrm = R.nrm;
    a.row_w = R.w;
    a.keys = K.ops;
    a.key_nrm = K.nrm;
    a.key_lw2 = K.lw2;
    a.n_rows = (int)R.n;
    a.n_keys = (int)K.n;
    a.dp = p->lse_dp;
    const double e = (double)eps;
    a.c_bias = (float)(1.4426950408889634 / e);
    a.c_score = (float)(2.8853900817779268 / e);
    a.out_scale = (float)(-e * 0.6931471805599453);
    a.n_split = f_side ? p->f_split : p->g_split;
    a.keys_per_split = f_side ? p->f_kps : p->g_kps;
    a.part = p->part;
    a.resid_part = p->resid_part;
    a.krec = p->krec;
    a.krec16 = p->krec16;
    a.krec3 = p->krec3;
    a.krec_guard = p->kguard;
    a.krec_keys = (int)K.n_pad;
    a.row_l1 = R.l1max;
    a.kbias = p->lbias;
    a.kbias_keys = (int)K.n_pad;
    return a;
}

// Optional HIP-event timing of the streaming kernels of a solve.
struct KernelTimer {
    bool on = false;
    std::vector<hipEvent_t> ev;  // begin/end pairs
    size_t used = 0;
    hipError_t reserve(size_t pairs) {
        on = true;
        ev.assign(2 * pairs, nullptr);
        for (auto& e : ev) {
            hipError_t r = hipEventCreate(&e);
            if (r != hipSuccess) return r;
        }
        return hipSuccess;
    }
    void next(hipEvent_t& b, hipEvent_t& e) {
        b = e = nullptr;
        if (!on || used + 2 > ev.size()) return;
        b = ev[used];
        e = ev[used + 1];
        used += 2;
    }
    ~KernelTimer() {
        for (auto& e : ev)
            if (e) (void)hipEventDestroy(e);
    }
};

// One half-step: out = update(other potential); optional residual of (cur, other).
fs_status half_step(fs_problem* p, bool f_side, float eps, const float* other, float* out,
                    const float* cur, float* resid, int mode, hipStream_t s,
                    KernelTimer* timer = nullptr) {
    LseArgs a = base_args(p, f_side, eps);
    a.key_pot = other;
    a.out = out;
    a.mode = mode;
    a.cur = cur;
    a.resid_out = resid;
    hipEvent_t eb = nullptr, ee = nullptr;
    if (timer) timer->next(eb, ee);
    hipError_t e = launch_lse(p->path, a, s, eb, ee);
    if (e != hipSuccess) return hip_fail(e, f_side ? "f-update launch" : "g-update launch");
    return FS_OK;
}

bool eps_ok(float eps) { return std::isfinite(eps) && eps > 0.f; }

// One transport application.  f_side: U_i = sum_j P_ij (V_j - voff) over the
// keys Y (U: n x dv, V: m x dv); otherwise U_j = sum_i P_ij (V_i - voff) over
// the keys X (U: m x dv, V: n x dv).  divide_by_w divides by a_i (b_j).
// lse2: the rows' exact LSE2 under these potentials, when the caller holds
// it.  Otherwise the streaming kernel takes its references from the row
// potential (no LSE pass) and the other kernels get an LSE pass first; with
// need_lse the rows' LSE2 is left in pot_tmp either way.
fs_status transport_side(fs_problem* p, bool f_side, float eps, const float* f, const float* g,
                         const float* V, int32_t dv, float* U, int32_t divide_by_w,
                         const float* voff, const float* vrs, hipStream_t s,
                         const float* lse2 = nullptr, const void* rows2 = nullptr,
                         bool need_lse = false) {
    if (!p || !f || !g || !V || !U) return fail(FS_ERR_INVALID_ARG, "NULL argument");
    if (!eps_ok(eps)) return fail(FS_ERR_INVALID_ARG, "eps must be finite and > 0");
    if (dv < 1 || dv > p->dv_max)
        return fail(FS_ERR_INVALID_ARG, "dv must be in [1, dv_max=%d] (got %d)", p->dv_max, dv);
    const Cloud& R = f_side ? p->X : p->Y;
    const Cloud& K = f_side ? p->Y : p->X;
    if (overlaps(U, (size_t)4 * R.n * dv, V, (size_t)4 * K.n * dv))
        return fail(FS_ERR_INVALID_ARG, "U overlaps V");
    const float* row_pot = f_side ? f : g;
    const float* key_pot = f_side ? g : f;
    const bool online = !lse2 && p->uref &&
                        transport_online(p->path, p->lse_dp, dv, K.n_pad, rows2 != nullptr);
    // exact row LSE (base 2) of this side's update scores, unless the caller
    // holds it for these potentials or the kernel needs none
    if (!lse2 && !online) {
        fs_status st = half_step(p, f_side, eps, key_pot, p->pot_tmp, nullptr, nullptr, 1, s);
        if (st != FS_OK) return st;
    }
    TransportArgs t{};
    t.ref_mode = online ? REF_ONLINE : REF_GIVEN;
    t.lse_out = online && need_lse ? p->pot_tmp : nullptr;
    t.rows = R.ops;
    t.row_lse2 = lse2 ? lse2 : p->pot_tmp;
    t.row_pot = row_pot;
    t.row_nrm = R.nrm;
    t.row_w = R.w;
    t.keys = K.ops;
    t.key_pot = key_pot;
    t.key_nrm = K.nrm;
    t.key_lw2 = K.lw2;
    t.V = V;
    t.v_off = voff;
    t.v_rscale = vrs;
    t.Vt = p->vt;
    t.v_unscale_dev = nullptr;
    t.n_rows = (int)R.n;
    t.n_keys = (int)K.n;
    t.dp = p->lse_dp;
    t.dv = dv;
    t.c_bias = (float)(1.4426950408889634 / (double)eps);
    t.c_score = (float)(2.8853900817779268 / (double)eps);
    t.divide_by_a = divide_by_w ? 1 : 0;
    t.U = U;
    t.rows2 = rows2;
    hipError_t e = launch_transport(p->path, t, p->scal + 2, p->vt, K.n_pad, p->kbias, p->upart,
                                    p->uref, s);
    if (e != hipSuccess) return hip_fail(e, "transport launch");
    return FS_OK;
}

}  // namespace

namespace {

// fs_potentials_init_cost into a problem struct the caller provides (host
// memory it owns); on failure *p is left unusable and nothing needs freeing.
fs_status init_problem(fs_problem* p, const float* X, const float* Y, const float* a,
                       const float* b, int64_t n, int64_t m, int32_t d, int32_t dv_max,
                       fs_score_prec prec, fs_cost cost, void* workspace,
                       size_t workspace_bytes, float* f, float* g, void* stream) {
    if (cost != FS_COST_SQEUCLIDEAN && cost != FS_COST_COSINE)
        return fail(FS_ERR_INVALID_ARG, "unknown fs_cost %d", (int)cost);
    if (!X || !Y || !a || !b) return fail(FS_ERR_INVALID_ARG, "X, Y, a and b must be non-NULL");
    Shape sh;
    Layout L;
    fs_status st = plan(n, m, d, dv_max, prec, sh, L);
    if (st != FS_OK) return st;
    if (!workspace) return fail(FS_ERR_WORKSPACE, "workspace is NULL");
    if ((uintptr_t)workspace % kAlign)
        return fail(FS_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
    if (workspace_bytes < L.total)
        return fail(FS_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                    L.total);
    int dev = 0;
    if ((st = check_device(&dev)) != FS_OK) return st;

    *p = fs_problem();
    char* w = (char*)workspace;
    p->device = dev;
    p->cost = (int)cost;
    p->path = sh.path;
    p->refine = sh.refine;
    if (sh.refine) {
        p->xops16 = w + L.xops16;
        p->yops16 = w + L.yops16;
        p->path16 = PATH_MFMA_F16;
    }
    p->n = n;
    p->m = m;
    p->d = d;
    p->dp = sh.dp;
    p->lse_dp = sh.lse_dp;
    p->dv_max = dv_max;
    p->f_split = sh.f_split;
    p->f_kps = sh.f_kps;
    p->g_split = sh.g_split;
    p->g_kps = sh.g_kps;
    p->centre = (float*)(w + L.centre);
    p->bbox_min = (float*)(w + L.bmin);
    p->bbox_max = (float*)(w + L.bmax);
    p->flag = (int*)(w + L.flag);
    p->X = Cloud{w + L.xops, (float*)(w + L.xn), (float*)(w + L.xl), (float*)(w + L.xw), n,
                 pad_rows(n)};
    p->Y = Cloud{w + L.yops, (float*)(w + L.yn), (float*)(w + L.yl), (float*)(w + L.yw), m,
                 pad_rows(m)};
    p->part = (float2*)(w + L.part);
    p->resid_part = (float*)(w + L.rpart);
    p->scal = (float*)(w + L.scal);
    p->pot_tmp = (float*)(w + L.ptmp);
    p->vt = (dv_max > 0 && !small_d_path(sh.path)) ? (void*)(w + L.vt) : nullptr;
    {
        const bool streams = p->vt && transport_streams(sh.path, sh.lse_dp);
        p->kbias = streams ? (float*)(w + L.kbias) : nullptr;
        p->upart = streams ? (float*)(w + L.upart) : nullptr;
        p->uref = streams ? (float*)(w + L.uref) : nullptr;
    }
    p->lbias = !small_d_path(sh.path) ? (float*)(w + L.lbias) : nullptr;
    p->ptag = small_d_path(sh.path) && persistent_fits(n, m, d)
                  ? (unsigned long long*)(w + L.ptag)
                  : nullptr;
    p->krec = sh.path == PATH_SMALL ? (float*)(w + L.krec) : nullptr;
    p->krec16 = sh.path == PATH_SMALL ? (void*)(w + L.krec16) : nullptr;
    p->krec3 = sh.path == PATH_SMALL && small_b3_rec_bytes(d) ? (void*)(w + L.krec3) : nullptr;
    p->kguard = sh.path == PATH_SMALL ? (void*)(w + L.kguard) : nullptr;
    if (sh.path == PATH_SMALL) {
        p->X.l1max = (float*)(w + L.kguard) + 2;
        p->Y.l1max = (float*)(w + L.kguard) + 3;
    }
    if (cost == FS_COST_COSINE) {
        p->X.rscale = (float*)(w + L.rsx);
        p->Y.rscale = (float*)(w + L.rsy);
    }

    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (cost == FS_COST_SQEUCLIDEAN && small_d_path(p->path) && n + m <= kSmallPrepPoints) {
        // small problems: the same preparation in two launches
        SmallPrepArgs sp{};
        sp.X = X;
        sp.Y = Y;
        sp.a = a;
        sp.b = b;
        sp.n = n;
        sp.m = m;
        sp.n_pad = p->X.n_pad;
        sp.m_pad = p->Y.n_pad;
        sp.d = d;
        sp.dp = p->dp;
        sp.centre = p->centre;
        sp.xops = (float*)p->X.ops;
        sp.yops = (float*)p->Y.ops;
        sp.xn = p->X.nrm;
        sp.yn = p->Y.nrm;
        sp.xlw = p->X.lw2;
        sp.ylw = p->Y.lw2;
        sp.xw = p->X.w;
        sp.yw = p->Y.w;
        sp.f = f;
        sp.g = g;
        sp.xl1 = p->path == PATH_SMALL ? p->X.l1max : nullptr;
        sp.yl1 = p->path == PATH_SMALL ? p->Y.l1max : nullptr;
        sp.flag = p->flag;
        if ((e = launch_prep_small(sp, s)) != hipSuccess) goto hip_error;
        goto check_flag;
    }
    if ((e = launch_zero_flag(p->flag, s)) != hipSuccess) goto hip_error;
    if (cost == FS_COST_COSINE &&
        ((e = launch_inv_norm(X, n, d, p->X.rscale, p->flag, s)) != hipSuccess ||
         (e = launch_inv_norm(Y, m, d, p->Y.rscale, p->flag, s)) != hipSuccess))
        goto hip_error;
    if ((e = launch_bbox(X, p->X.rscale, n, Y, p->Y.rscale, m, d, p->bbox_min, p->bbox_max,
                         kBboxParts, p->centre, s)) != hipSuccess)
        goto hip_error;
    if ((e = launch_convert(X, p->X.rscale, n, p->X.n_pad, d, p->dp, p->path, p->centre,
                            p->centre + d, p->X.ops, p->X.nrm, p->flag, s)) != hipSuccess)
        goto hip_error;
    if ((e = launch_convert(Y, p->Y.rscale, m, p->Y.n_pad, d, p->dp, p->path, p->centre + d,
                            p->centre, p->Y.ops, p->Y.nrm, p->flag, s)) != hipSuccess)
        goto hip_error;
    // the fp16 copies (the cost terms are written again, with the same values)
    if (p->refine &&
        ((e = launch_convert(X, p->X.rscale, n, p->X.n_pad, d, p->dp, p->path16, p->centre,
                             p->centre + d, p->xops16, p->X.nrm, p->flag, s)) != hipSuccess ||
         (e = launch_convert(Y, p->Y.rscale, m, p->Y.n_pad, d, p->dp, p->path16, p->centre + d,
                             p->centre, p->yops16, p->Y.nrm, p->flag, s)) != hipSuccess))
        goto hip_error;
    if (p->path == PATH_SMALL &&
        ((e = launch_row_l1max((const float*)p->X.ops, n, d, p->X.l1max, s)) != hipSuccess ||
         (e = launch_row_l1max((const float*)p->Y.ops, m, d, p->Y.l1max, s)) != hipSuccess))
        goto hip_error;
    if ((e = launch_weights(a, n, p->X.lw2, p->X.w, f, p->flag, s)) != hipSuccess) goto hip_error;
    if ((e = launch_weights(b, m, p->Y.lw2, p->Y.w, g, p->flag, s)) != hipSuccess) goto hip_error;
check_flag:
    {
        int flag = 0;
        if ((e = hipMemcpyAsync(&flag, p->flag, sizeof(int), hipMemcpyDeviceToHost, s)) !=
            hipSuccess)
            goto hip_error;
        if ((e = hipStreamSynchronize(s)) != hipSuccess) goto hip_error;
        if (flag) {
            if (flag & 1) return fail(FS_ERR_NONFINITE, "X or Y holds a NaN or Inf");
            if (flag & 2) return fail(FS_ERR_NONFINITE, "a weight is <= 0, subnormal, NaN or Inf");
            if (flag & 8)
                return fail(FS_ERR_INVALID_ARG,
                            "cosine cost: a point has zero (or non-finite) length");
            return fail(FS_ERR_INVALID_ARG,
                        "a centred coordinate overflows the fp16 range; scale the points "
                        "(and eps by the square of the scale) or use FS_PREC_BF16");
        }
    }
    return FS_OK;
hip_error:
    return hip_fail(e, "fs_potentials_init");
}

}  // namespace

extern "C" {

size_t fs_workspace_bytes(int64_t n, int64_t m, int32_t d, int32_t dv_max, fs_score_prec prec) {
    Shape sh;
    Layout L;
    if (plan(n, m, d, dv_max, prec, sh, L) != FS_OK) return 0;
    return L.total;
}

fs_status fs_potentials_init(const float* X, const float* Y, const float* a, const float* b,
                             int64_t n, int64_t m, int32_t d, int32_t dv_max, fs_score_prec prec,
                             void* workspace, size_t workspace_bytes, float* f, float* g,
                             void* stream, fs_problem** out) {
    return fs_potentials_init_cost(X, Y, a, b, n, m, d, dv_max, prec, FS_COST_SQEUCLIDEAN,
                                   workspace, workspace_bytes, f, g, stream, out);
}


fs_status fs_potentials_init_cost(const float* X, const float* Y, const float* a,
                                  const float* b, int64_t n, int64_t m, int32_t d,
                                  int32_t dv_max, fs_score_prec prec, fs_cost cost,
                                  void* workspace, size_t workspace_bytes, float* f, float* g,
                                  void* stream, fs_problem** out) {
    if (!out) return fail(FS_ERR_INVALID_ARG, "out handle pointer is NULL");
    *out = nullptr;
    fs_problem* p = new (std::nothrow) fs_problem();
    if (!p) return fail(FS_ERR_DEVICE, "host allocation failed");
    const fs_status st = init_problem(p, X, Y, a, b, n, m, d, dv_max, prec, cost, workspace,
                                      workspace_bytes, f, g, stream);
    if (st != FS_OK) {
        delete p;
        return st;
    }
    *out = p;
    return FS_OK;
}


fs_status fs_lse_update_f(fs_problem* p, float eps, const float* g, float* f_out,
                          const float* f_cur, float* row_resid, void* stream) {
    if (!p || !g || !f_out) return fail(FS_ERR_INVALID_ARG, "NULL handle, g or f_out");
    if (!eps_ok(eps)) return fail(FS_ERR_INVALID_ARG, "eps must be finite and > 0");
    if (row_resid && !f_cur) return fail(FS_ERR_INVALID_ARG, "row_resid needs f_cur");
    if (row_resid && overlaps(f_out, 4 * p->n, f_cur, 4 * p->n))
        return fail(FS_ERR_INVALID_ARG, "f_out may not overlap f_cur when a residual is asked");
    if (overlaps(f_out, 4 * p->n, g, 4 * p->m))
        return fail(FS_ERR_INVALID_ARG, "f_out overlaps g");
    return half_step(p, true, eps, g, f_out, row_resid ? f_cur : nullptr, row_resid, 0,
                     (hipStream_t)stream);
}

fs_status fs_lse_update_g(fs_problem* p, float eps, const float* f, float* g_out,
                          const float* g_cur, float* col_resid, void* stream) {
    if (!p || !f || !g_out) return fail(FS_ERR_INVALID_ARG, "NULL handle, f or g_out");
    if (!eps_ok(eps)) return fail(FS_ERR_INVALID_ARG, "eps must be finite and > 0");
    if (col_resid && !g_cur) return fail(FS_ERR_INVALID_ARG, "col_resid needs g_cur");
    if (col_resid && overlaps(g_out, 4 * p->m, g_cur, 4 * p->m))
        return fail(FS_ERR_INVALID_ARG, "g_out may not overlap g_cur when a residual is asked");
    if (overlaps(g_out, 4 * p->m, f, 4 * p->n))
        return fail(FS_ERR_INVALID_ARG, "g_out overlaps f");
    return half_step(p, false, eps, f, g_out, col_resid ? g_cur : nullptr, col_resid, 0,
                     (hipStream_t)stream);
}

fs_status fs_marginal_residual(fs_problem* p, float eps, const float* f, const float* g,
                               float* out2, void* stream) {
    if (!p || !f || !g || !out2) return fail(FS_ERR_INVALID_ARG, "NULL argument");
    if (!eps_ok(eps)) return fail(FS_ERR_INVALID_ARG, "eps must be finite and > 0");
    RefineScope fp16_passes(p);
    hipStream_t s = (hipStream_t)stream;
    fs_status st = half_step(p, true, eps, g, p->pot_tmp, f, out2, 0, s);
    if (st != FS_OK) return st;
    return half_step(p, false, eps, f, p->pot_tmp, g, out2 + 1, 0, s);
}

fs_status fs_sinkhorn_solve(fs_problem* p, const fs_solve_opts* o, float* f, float* g,
                            fs_solve_info* info, void* stream) {
    if (!p || !o || !f || !g) return fail(FS_ERR_INVALID_ARG, "NULL handle, opts, f or g");
    if (o->n_stages < 1) return fail(FS_ERR_INVALID_ARG, "n_stages must be >= 1");
    if (o->iters_per_stage < 0) return fail(FS_ERR_INVALID_ARG, "iters_per_stage must be >= 0");
    if (o->refine_iters < 0) return fail(FS_ERR_INVALID_ARG, "refine_iters must be >= 0");
    if (!eps_ok(o->eps_end) || (o->n_stages > 1 && !eps_ok(o->eps_start)))
        return fail(FS_ERR_INVALID_ARG, "eps_start/eps_end must be finite and > 0");
    if (!std::isfinite(o->tol)) return fail(FS_ERR_INVALID_ARG, "tol must be finite");
    if (o->tol > 0.f && o->check_every < 1)
        return fail(FS_ERR_INVALID_ARG, "check_every must be >= 1 when tol > 0");
    if (overlaps(f, 4 * p->n, g, 4 * p->m)) return fail(FS_ERR_INVALID_ARG, "f overlaps g");
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    const bool use_tol = o->tol > 0.f;
    // the whole schedule as one launch (small d <= 8 problems, fixed count)
    const bool sl_allowed = !use_tol && small_d_path(p->path) && !p->refine &&
                            o->n_stages <= kPersistentMaxStages && o->iters_per_stage > 0 &&
                            2 * (int64_t)o->n_stages * o->iters_per_stage < (int64_t)0xffffffff &&
                            p->ptag != nullptr;
    const bool single =
        sl_allowed && (o->single_launch == 1 ||
                       (o->single_launch == 0 && p->n * p->m <= ((int64_t)1 << 19)));
    KernelTimer timer;
    if (o->time_kernels) {
        // one begin/end pair per streaming launch (one for the single launch)
        const size_t pairs =
            single ? 1 : 2 * (size_t)o->n_stages * (size_t)o->iters_per_stage + 8;
        if ((e = timer.reserve(pairs)) != hipSuccess) return hip_fail(e, "hipEventCreate");
    }
    KernelTimer* tp = o->time_kernels ? &timer : nullptr;
    // the single launch starts from g = 0 by itself and writes f and g
    if (!o->warm_start && !single) {
        if ((e = launch_fill(g, p->m, 0.f, s)) != hipSuccess) return hip_fail(e, "fill g");
        if ((e = launch_fill(f, p->n, 0.f, s)) != hipSuccess) return hip_fail(e, "fill f");
    }
    if (single) {
        PersistentArgs pa{};
        pa.g_zero = o->warm_start ? 0 : 1;
        pa.X = (const float*)p->X.ops;
        pa.Y = (const float*)p->Y.ops;
        pa.xn = p->X.nrm;
        pa.yn = p->Y.nrm;
        pa.xl = p->X.lw2;
        pa.yl = p->Y.lw2;
        pa.f = f;
        pa.g = g;
        pa.n = (int)p->n;
        pa.m = (int)p->m;
        pa.d = p->d;
        pa.stride = p->dp;
        pa.W = persistent_workgroups(p->n, p->m);
        pa.n_stages = o->n_stages;
        pa.iters = o->iters_per_stage;
        for (int st_i = 0; st_i < o->n_stages; ++st_i)
            pa.eps[st_i] = o->n_stages == 1
                               ? o->eps_end
                               : (float)((double)o->eps_start *
                                         std::pow((double)o->eps_end / (double)o->eps_start,
                                                  (double)st_i / (double)(o->n_stages - 1)));
        pa.tf = p->ptag;
        pa.tg = p->ptag + p->n;
        pa.err = (int*)(p->ptag + p->n + p->m);
        hipEvent_t eb = nullptr, ee = nullptr;
        if (tp) tp->next(eb, ee);
        if ((e = launch_fill((float*)p->ptag, 2 * (p->n + p->m + 1), 0.f, s)) != hipSuccess)
            return hip_fail(e, "fill");
        if (eb && (e = hipEventRecord(eb, s)) != hipSuccess) return hip_fail(e, "event");
        if ((e = launch_solve_persistent(pa, s)) != hipSuccess)
            return hip_fail(e, "single-launch solve");
        if (ee && (e = hipEventRecord(ee, s)) != hipSuccess) return hip_fail(e, "event");
        float ms = 0.f;
        if (tp) {
            if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(e, "timing sync");
            if ((e = hipEventElapsedTime(&ms, eb, ee)) != hipSuccess)
                return hip_fail(e, "hipEventElapsedTime");
        }
        if (info) {
            info->iters_done = o->n_stages * o->iters_per_stage;
            info->final_eps = pa.eps[o->n_stages - 1];
            info->residual = -1.f;
            // one launch: reported as its half-steps, each the launch's mean share
            info->lse_launches = tp ? 2 * info->iters_done : 0;
            info->lse_ms = ms;
            info->single_launch = 1;
        }
        return FS_OK;
    }
    int done = 0;
    float resid = -1.f;
    float eps = o->eps_end;
    bool converged = false;
    const int64_t total_iters = (int64_t)o->n_stages * o->iters_per_stage;
    const int refine_iters = o->refine_iters > 0 ? o->refine_iters : 1;
    bool have_next_f = false;  // pot_tmp already holds the next f-update (same eps)
    fs_status st;
    auto check = [&](float eps_c, bool& reusable_next) -> fs_status {
        // Both terms of the L1 residual of (f, g) from dry-run updates: the
        // column term (a g-update of f into pot_tmp, against g) first, then
        // the row term (an f-update of g into pot_tmp, against f), whose
        // output is the next iteration's f-update and is kept for it.
        fs_status s2 = half_step(p, false, eps_c, f, p->pot_tmp, g, p->scal + 1, 0, s);
        if (s2 == FS_OK) s2 = half_step(p, true, eps_c, g, p->pot_tmp, f, p->scal, 0, s);
        if (s2 != FS_OK) return s2;
        float h[2] = {0.f, 0.f};
        hipError_t e2 = hipMemcpyAsync(h, p->scal, sizeof(h), hipMemcpyDeviceToHost, s);
        if (e2 == hipSuccess) e2 = hipStreamSynchronize(s);
        if (e2 != hipSuccess) return hip_fail(e2, "residual readback");
        resid = h[0] + h[1];
        reusable_next = true;
        return FS_OK;
    };
    for (int st_i = 0; st_i < o->n_stages && !converged; ++st_i) {
        if (o->n_stages == 1)
            eps = o->eps_end;
        else
            eps = (float)((double)o->eps_start *
                          std::pow((double)o->eps_end / (double)o->eps_start,
                                   (double)st_i / (double)(o->n_stages - 1)));
        if (have_next_f) have_next_f = false;  // new stage: eps changed
        for (int it = 0; it < o->iters_per_stage; ++it) {
            // the last refine_iters iterations of a fixed-count schedule run
            // on the fp16 copies of a FS_PREC_BF16_REFINE problem
            RefineScope last(p, !use_tol && (int64_t)st_i * o->iters_per_stage + it >=
                                                total_iters - refine_iters);
            if (have_next_f) {
                if ((e = hipMemcpyAsync(f, p->pot_tmp, sizeof(float) * p->n,
                                        hipMemcpyDeviceToDevice, s)) != hipSuccess)
                    return hip_fail(e, "copy f");
                have_next_f = false;
            } else if ((st = half_step(p, true, eps, g, f, nullptr, nullptr, 0, s, tp)) != FS_OK) {
                return st;
            }
            if ((st = half_step(p, false, eps, f, g, nullptr, nullptr, 0, s, tp)) != FS_OK)
                return st;
            ++done;
            if (use_tol && done % o->check_every == 0) {
                bool reusable = false;
                if ((st = check(eps, reusable)) != FS_OK) return st;
                if (resid <= o->tol) {
                    converged = true;
                    break;
                }
                have_next_f = reusable;
            }
        }
    }
    if (use_tol && !converged && (done == 0 || done % o->check_every != 0)) {
        bool dummy = false;
        if ((st = check(eps, dummy)) != FS_OK) return st;
        converged = resid <= o->tol;
    }
    if (use_tol && p->refine) {
        // FS_PREC_BF16_REFINE with a residual stop: the checks measure the
        // bf16 iterations themselves; refine_iters iterations on the fp16
        // copies follow the stop
        RefineScope fp16_passes(p);
        for (int r = 0; r < refine_iters; ++r) {
            if ((st = half_step(p, true, eps, g, f, nullptr, nullptr, 0, s, tp)) != FS_OK)
                return st;
            if ((st = half_step(p, false, eps, f, g, nullptr, nullptr, 0, s, tp)) != FS_OK)
                return st;
            ++done;
        }
    }
    float lse_ms = 0.f;
    int lse_n = 0;
    if (tp) {
        if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(e, "timing sync");
        for (size_t k = 0; k + 1 < timer.used; k += 2) {
            float ms = 0.f;
            if ((e = hipEventElapsedTime(&ms, timer.ev[k], timer.ev[k + 1])) != hipSuccess)
                return hip_fail(e, "hipEventElapsedTime");
            lse_ms += ms;
            ++lse_n;
        }
    }
    if (info) {
        info->iters_done = done;
        info->final_eps = eps;
        info->residual = use_tol ? resid : -1.f;
        info->lse_launches = lse_n;
        info->lse_ms = lse_ms;
        info->single_launch = 0;
    }
    if (use_tol && !converged)
        return fail(FS_ERR_NOT_CONVERGED, "residual %g above tol %g after %d iterations",
                    (double)resid, (double)o->tol, done);
    return FS_OK;
}

fs_status fs_apply_transport(fs_problem* p, float eps, const float* f, const float* g,
                             const float* V, int32_t dv, float* U, int32_t divide_by_a,
                             void* stream) {
    RefineScope fp16_passes(p);
    return transport_side(p, true, eps, f, g, V, dv, U, divide_by_a, nullptr, nullptr,
                          (hipStream_t)stream);
}

fs_status fs_apply_transport_t(fs_problem* p, float eps, const float* f, const float* g,
                               const float* W, int32_t dv, float* U, int32_t divide_by_b,
                               void* stream) {
    RefineScope fp16_passes(p);
    return transport_side(p, false, eps, f, g, W, dv, U, divide_by_b, nullptr, nullptr,
                          (hipStream_t)stream);
}

fs_status fs_gradient(fs_problem* p, float eps, const float* f, const float* g, const float* X,
                      const float* Y, float* grad_x, float* grad_y, void* stream) {
    if (!p || !f || !g || !X || !Y) return fail(FS_ERR_INVALID_ARG, "NULL argument");
    RefineScope fp16_passes(p);
    if (p->dv_max < p->d)
        return fail(FS_ERR_INVALID_ARG,
                    "the gradient needs dv_max >= d at init (dv_max=%d, d=%d)", p->dv_max, p->d);
    if (grad_x && (overlaps(grad_x, (size_t)4 * p->n * p->d, X, (size_t)4 * p->n * p->d) ||
                   overlaps(grad_x, (size_t)4 * p->n * p->d, Y, (size_t)4 * p->m * p->d)))
        return fail(FS_ERR_INVALID_ARG, "grad_x overlaps X or Y");
    if (grad_y && (overlaps(grad_y, (size_t)4 * p->m * p->d, X, (size_t)4 * p->n * p->d) ||
                   overlaps(grad_y, (size_t)4 * p->m * p->d, Y, (size_t)4 * p->m * p->d)))
        return fail(FS_ERR_INVALID_ARG, "grad_y overlaps X or Y");
    hipStream_t s = (hipStream_t)stream;
    const float c_bias = (float)(1.4426950408889634 / (double)eps);
    const float* nu = p->centre;          // centre of X
    const float* mu = p->centre + p->d;   // centre of Y
    if (grad_x) {
        // grad_x <- sum_j P_ij (y_j - mu), then 2 (r_i (x_i - mu) - that)
        fs_status st = transport_side(p, true, eps, f, g, Y, p->d, grad_x, 0, mu, p->Y.rscale, s,
                                      nullptr, nullptr, true);
        if (st != FS_OK) return st;
        hipError_t e = launch_grad_finish(X, p->X.rscale, mu, p->pot_tmp, f, p->X.nrm, p->X.w,
                                          c_bias, p->n, p->d, grad_x, s);
        if (e != hipSuccess) return hip_fail(e, "gradient launch");
    }
    if (grad_y) {
        fs_status st = transport_side(p, false, eps, f, g, X, p->d, grad_y, 0, nu, p->X.rscale, s,
                                      nullptr, nullptr, true);
        if (st != FS_OK) return st;
        hipError_t e = launch_grad_finish(Y, p->Y.rscale, nu, p->pot_tmp, g, p->Y.nrm, p->Y.w,
                                          c_bias, p->m, p->d, grad_y, s);
        if (e != hipSuccess) return hip_fail(e, "gradient launch");
    }
    return FS_OK;
}

fs_status fs_dual_value(fs_problem* p, const float* f, const float* g, double* out,
                        void* stream) {
    if (!p || !f || !g || !out) return fail(FS_ERR_INVALID_ARG, "NULL argument");
    hipError_t e = launch_dual_value(p->X.w, f, p->n, p->Y.w, g, p->m, out, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "dual value launch");
    return FS_OK;
}

}  // extern "C"

namespace {

// Device scratch of fs_hvp, carved from the caller's workspace (floats, each
// array 256-byte aligned; CH = second-moment columns per transport pass).
struct HvpLayout {
    size_t lse_r, lse_c, r, c, PY, W, PtW, u, rhs, dg, res, pd, Ap, Pp, Ptq, V2, T, M, V3, T3, dots,
        vops, vsig, total;
    int ch;
    bool fused;  // second moment by the one-pass kernel (else d*d columns in passes)
};

// The one-pass second-moment kernel serves two-byte scores at d_pad 64..512.
bool hvp_fused(const fs_problem* p) {
    return (p->path == PATH_MFMA_BF16 || p->path == PATH_MFMA_F16) && p->lse_dp >= 64 &&
           p->lse_dp <= 512 && p->d <= 512 &&
           (int64_t)p->d * std::max(p->X.n_pad, p->Y.n_pad) * 2 < ((int64_t)1 << 32);
}

HvpLayout hvp_layout(const fs_problem* p) {
    HvpLayout L{};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = up(o + bytes, kAlign);
        return at;
    };
    // either cloud can be the differentiated one: size both roles for the
    // larger
    const size_t n = (size_t)std::max(p->n, p->m), m = n, d = (size_t)p->d;
    L.fused = hvp_fused(p);
    L.ch = L.fused ? 0 : (int)std::min<int64_t>((int64_t)p->dv_max, (int64_t)d * d);
    L.lse_r = take(4 * n);
    L.lse_c = take(4 * m);
    L.r = take(4 * n);
    L.c = take(4 * m);
    L.PY = take(4 * n * d);
    L.W = take(4 * n * (d + 2));
    L.PtW = take(4 * m * (d + 2));
    L.u = take(4 * n);
    L.rhs = take(4 * m);
    L.dg = take(4 * m);
    L.res = take(4 * m);
    L.pd = take(4 * m);
    L.Ap = take(4 * m);
    L.Pp = take(4 * n);
    L.Ptq = take(4 * m);
    L.V2 = take(4 * m * (d + 1));
    L.T = take(4 * n * (d + 1));
    L.M = take(4 * n * d);
    L.V3 = take(4 * m * (size_t)L.ch);
    L.T3 = take(4 * n * (size_t)L.ch);
    L.dots = take(sizeof(double) * 4);
    L.vops = take(L.fused ? (size_t)2 * (size_t)std::max(p->X.n_pad, p->Y.n_pad) *
                                (size_t)p->lse_dp
                          : 0);
    L.vsig = take(L.fused ? 4 * n : 0);
    L.total = o;
    return L;
}

// (x.y, sum x, x.x) on the host (one workgroup reduction, then a synchronous
// copy)
fs_status host_dots(const float* x, const float* y, int64_t len, double* dev, double out[3],
                    hipStream_t s) {
    hipError_t e = launch_dot(x, y, len, dev, s);
    if (e == hipSuccess) e = hipMemcpyAsync(out, dev, 3 * sizeof(double), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return e == hipSuccess ? FS_OK : hip_fail(e, "HVP reduction");
}

}  // namespace

extern "C" {

size_t fs_hvp_workspace_bytes(const fs_problem* p) { return p ? hvp_layout(p).total : 0; }

fs_status fs_hvp(fs_problem* p, float eps, const float* f, const float* g, const float* X,
                 const float* Y, int32_t wrt, const float* V, float* HV, float cg_tol,
                 int32_t cg_max_iter, void* workspace, size_t workspace_bytes, fs_hvp_info* info,
                 void* stream) {
    RefineScope fp16_passes(p);
    if (!p || !f || !g || !X || !Y || !V || !HV || !workspace)
        return fail(FS_ERR_INVALID_ARG, "NULL argument");
    if (wrt != 0 && wrt != 1) return fail(FS_ERR_INVALID_ARG, "wrt must be 0 (X) or 1 (Y)");
    if (!eps_ok(eps)) return fail(FS_ERR_INVALID_ARG, "eps must be finite and > 0");
    if (p->cost != FS_COST_SQEUCLIDEAN)
        return fail(FS_ERR_INVALID_ARG, "the HVP supports the squared-Euclidean cost only");
    if (p->dv_max < p->d + 2)
        return fail(FS_ERR_INVALID_ARG, "the HVP needs dv_max >= d + 2 at init (dv_max=%d, d=%d)",
                    p->dv_max, p->d);
    if (!(cg_tol >= 0.f) || cg_max_iter < 0)
        return fail(FS_ERR_INVALID_ARG, "cg_tol must be >= 0 and cg_max_iter >= 0");
    const HvpLayout L = hvp_layout(p);
    if (workspace_bytes < L.total)
        return fail(FS_ERR_WORKSPACE, "HVP workspace too small: %zu < %zu bytes", workspace_bytes,
                    L.total);
    // The differentiated cloud R ("rows") and the other one K ("keys"): X
    // and Y, or exchanged.  Every formula below is written for R = X.
    const bool xs = wrt == 0;
    const int64_t n = xs ? p->n : p->m, m = xs ? p->m : p->n;
    const float* Rp = xs ? X : Y;
    const float* Kp = xs ? Y : X;
    const float* fr = xs ? f : g;
    const float* fk = xs ? g : f;
    const Cloud& RC = xs ? p->X : p->Y;
    const Cloud& KC = xs ? p->Y : p->X;
    const size_t nd = (size_t)4 * n * p->d;
    if (overlaps(HV, nd, V, nd) || overlaps(HV, nd, X, (size_t)4 * p->n * p->d) ||
        overlaps(HV, nd, workspace, workspace_bytes) ||
        overlaps(HV, nd, Y, (size_t)4 * p->m * p->d))
        return fail(FS_ERR_INVALID_ARG, "HV overlaps an input or the workspace");
    hipStream_t s = (hipStream_t)stream;
    char* w = (char*)workspace;
    auto F = [&](size_t off) { return (float*)(w + off); };
    double* dots = (double*)(w + L.dots);
    const int d = p->d;
    const float c_bias = (float)(1.4426950408889634 / (double)eps);
    // centre of K: every point is taken relative to it
    const float* mu = xs ? p->centre + d : p->centre;
    fs_status st;
    hipError_t e;
#define FS_HIP(call, what)                     \
    do {                                       \
        if ((e = (call)) != hipSuccess) return hip_fail(e, what); \
    } while (0)
    // exact row and column LSEs (reused by every transport below), marginals
    if ((st = half_step(p, xs, eps, fk, F(L.lse_r), nullptr, nullptr, 1, s)) != FS_OK) return st;
    if ((st = half_step(p, !xs, eps, fr, F(L.lse_c), nullptr, nullptr, 1, s)) != FS_OK) return st;
    FS_HIP(launch_marginal(F(L.lse_r), fr, RC.nrm, RC.w, c_bias, n, F(L.r), s), "HVP marginal");
    FS_HIP(launch_marginal(F(L.lse_c), fk, KC.nrm, KC.w, c_bias, m, F(L.c), s), "HVP marginal");
    // PY = P (K - mu); u, W = [V | s | u/r]; PtW = P^T W; rhs = w - P^T (u/r)
    if ((st = transport_side(p, xs, eps, f, g, Kp, d, F(L.PY), 0, mu, nullptr, s, F(L.lse_r))) !=
        FS_OK)
        return st;
    FS_HIP(launch_hvp_rows(Rp, V, mu, F(L.PY), F(L.r), n, d, F(L.u), F(L.W), s), "HVP rows");
    if ((st = transport_side(p, !xs, eps, f, g, F(L.W), d + 2, F(L.PtW), 0, nullptr, nullptr, s,
                             F(L.lse_c))) != FS_OK)
        return st;
    FS_HIP(launch_hvp_cols(Kp, mu, F(L.PtW), m, d, F(L.rhs), s), "HVP columns");
    // Preconditioned CG (M = diag(c), the diagonal of K's first term) for
    // K dg = rhs on the complement of the constant vector,
    // K = diag(c) - P^T diag(1/r) P.  The residual is kept mean-free (K's
    // range); dg's own constant does not change dP.  Stops when the plain
    // residual norm falls to cg_tol of its start.
    double h[3];
    if ((st = host_dots(F(L.rhs), F(L.rhs), m, dots, h, s)) != FS_OK) return st;
    FS_HIP(launch_axpby(0.f, F(L.rhs), 1.f, F(L.rhs), m, dots + 1, 1.0 / (double)m, s),
           "HVP projection");
    const double rr0 = std::max(h[2] - h[1] * h[1] / (double)m, 0.0);
    FS_HIP(launch_fill(F(L.dg), m, 0.f, s), "HVP fill");
    FS_HIP(launch_axpby(1.f, F(L.rhs), 0.f, F(L.res), m, nullptr, 0.0, s), "HVP copy");
    FS_HIP(launch_scale_sub(F(L.c), F(L.res), nullptr, m, 1, F(L.pd), s), "HVP precondition");
    if ((st = host_dots(F(L.res), F(L.pd), m, dots, h, s)) != FS_OK) return st;
    double rz = h[0], rel = rr0 > 0.0 ? 1.0 : 0.0;
    int it = 0;
    while (rr0 > 0.0 && it < cg_max_iter && rel > (double)cg_tol) {
        // Ap = c pd - P^T ((P pd) / r)
        if ((st = transport_side(p, xs, eps, f, g, F(L.pd), 1, F(L.Pp), 0, nullptr, nullptr, s,
                                 F(L.lse_r))) != FS_OK)
            return st;
        FS_HIP(launch_scale_sub(F(L.r), F(L.Pp), nullptr, n, 1, F(L.Pp), s), "HVP scale");
        if ((st = transport_side(p, !xs, eps, f, g, F(L.Pp), 1, F(L.Ptq), 0, nullptr, nullptr, s,
                                 F(L.lse_c))) != FS_OK)
            return st;
        FS_HIP(launch_scale_sub(F(L.c), F(L.pd), F(L.Ptq), m, 0, F(L.Ap), s), "HVP scale");
        if ((st = host_dots(F(L.pd), F(L.Ap), m, dots, h, s)) != FS_OK) return st;
        if (!(h[0] > 0.0)) break;  // no descent left (rounding): stop at the current dg
        const double alpha = rz / h[0];
        FS_HIP(launch_axpby((float)alpha, F(L.pd), 1.f, F(L.dg), m, nullptr, 0.0, s), "HVP update");
        FS_HIP(launch_axpby((float)-alpha, F(L.Ap), 1.f, F(L.res), m, nullptr, 0.0, s),
               "HVP update");
        // res <- res - mean(res); z = res / c (into Ap, free now); r.z and |res|^2
        if ((st = host_dots(F(L.res), F(L.res), m, dots, h, s)) != FS_OK) return st;
        FS_HIP(launch_axpby(0.f, F(L.res), 1.f, F(L.res), m, dots + 1, 1.0 / (double)m, s),
               "HVP projection");
        const double rr_new = std::max(h[2] - h[1] * h[1] / (double)m, 0.0);
        ++it;
        rel = std::sqrt(rr_new / rr0);
        if (rel <= (double)cg_tol) break;
        FS_HIP(launch_scale_sub(F(L.c), F(L.res), nullptr, m, 1, F(L.Ap), s), "HVP precondition");
        if ((st = host_dots(F(L.res), F(L.Ap), m, dots, h, s)) != FS_OK) return st;
        const double rz_new = h[0];
        FS_HIP(launch_axpby(1.f, F(L.Ap), (float)(rz_new / rz), F(L.pd), m, nullptr, 0.0, s),
               "HVP update");
        rz = rz_new;
    }
    // T = P [dg (Y - mu) | dg]
    FS_HIP(launch_hvp_dgy(Kp, mu, F(L.dg), m, d, F(L.V2), s), "HVP dg columns");
    if ((st = transport_side(p, xs, eps, f, g, F(L.V2), d + 1, F(L.T), 0, nullptr, nullptr, s,
                             F(L.lse_r))) != FS_OK)
        return st;
    // M_i = sum_j P_ij ((y_j - mu).v_i) (y_j - mu)
    if (L.fused) {
        // one pass: the direction rows (scaled per row into the score type)
        // as a second resident block, weights P_ij (v_i sigma_i).y~_j
        FS_HIP(launch_hvp_vconv(p->path, V, n, RC.n_pad, d, p->lse_dp, w + L.vops, F(L.vsig), s),
               "HVP direction rows");
        if ((st = transport_side(p, xs, eps, f, g, Kp, d, F(L.M), 0, mu, nullptr, s, F(L.lse_r),
                                 w + L.vops)) != FS_OK)
            return st;
    } else {
        // from the d*d outer-product columns in passes of L.ch
        FS_HIP(launch_fill(F(L.M), n * d, 0.f, s), "HVP fill");
        for (int64_t q0 = 0; q0 < (int64_t)d * d; q0 += L.ch) {
            const int wq = (int)std::min<int64_t>(L.ch, (int64_t)d * d - q0);
            FS_HIP(launch_hvp_outer(Kp, mu, m, d, q0, wq, F(L.V3), s), "HVP outer products");
            if ((st = transport_side(p, xs, eps, f, g, F(L.V3), wq, F(L.T3), 0, nullptr, nullptr,
                                     s, F(L.lse_r))) != FS_OK)
                return st;
            FS_HIP(launch_hvp_moment(F(L.T3), V, n, d, q0, wq, F(L.M), s), "HVP moment");
        }
    }
    FS_HIP(launch_hvp_final(V, F(L.r), F(L.u), F(L.W), F(L.PY), F(L.T), F(L.M),
                            L.fused ? F(L.vsig) : nullptr, n, d, (float)(1.0 / (double)eps), HV, s),
           "HVP assembly");
#undef FS_HIP
    if (info) {
        info->cg_iters = it;
        info->cg_residual = (float)rel;
    }
    return FS_OK;
}

void fs_destroy(fs_problem* p) { delete p; }

const char* fs_status_string(fs_status s) {
    switch (s) {
        case FS_OK: return "FS_OK";
        case FS_ERR_INVALID_ARG: return "FS_ERR_INVALID_ARG";
        case FS_ERR_WORKSPACE: return "FS_ERR_WORKSPACE";
        case FS_ERR_DEVICE: return "FS_ERR_DEVICE";
        case FS_ERR_NONFINITE: return "FS_ERR_NONFINITE";
        case FS_ERR_NOT_CONVERGED: return "FS_ERR_NOT_CONVERGED";
    }
    return "FS_ERR_UNKNOWN";
}

const char* fs_last_error(void) { return g_err.c_str(); }

fs_status fs_probe_peak(fs_probe_kind kind, float* sink, int32_t reps, void* stream,
                        double* rate) {
    if (kind < FS_PROBE_MFMA_BF16 || kind > FS_PROBE_EXP)
        return fail(FS_ERR_INVALID_ARG, "unknown fs_probe_kind %d", (int)kind);
    if (reps < 1 || reps > 64) return fail(FS_ERR_INVALID_ARG, "reps must be in [1, 64]");
    if (!sink || !rate) return fail(FS_ERR_INVALID_ARG, "NULL sink or rate");
    const int blocks = probe_blocks();
    if (blocks <= 0) return fail(FS_ERR_DEVICE, "no usable device for the probe");
    hipStream_t s = (hipStream_t)stream;
    std::vector<hipEvent_t> ev(2 * reps, nullptr);
    std::vector<double> r;
    hipError_t e = hipSuccess;
    for (auto& x : ev)
        if ((e = hipEventCreate(&x)) != hipSuccess) break;
    if (e == hipSuccess) e = launch_probe((int)kind, blocks, sink, s);  // untimed
    for (int i = 0; e == hipSuccess && i < reps; ++i) {
        if ((e = hipEventRecord(ev[2 * i], s)) != hipSuccess) break;
        if ((e = launch_probe((int)kind, blocks, sink, s)) != hipSuccess) break;
        e = hipEventRecord(ev[2 * i + 1], s);
    }
    if (e == hipSuccess) e = hipEventSynchronize(ev[2 * reps - 1]);
    for (int i = 0; e == hipSuccess && i < reps; ++i) {
        float ms = 0.f;
        if ((e = hipEventElapsedTime(&ms, ev[2 * i], ev[2 * i + 1])) != hipSuccess) break;
        r.push_back(probe_work_per_launch((int)kind, blocks) / (ms * 1e-3));
    }
    for (auto x : ev)
        if (x) (void)hipEventDestroy(x);
    if (e != hipSuccess) return hip_fail(e, "fs_probe_peak");
    std::sort(r.begin(), r.end());
    *rate = r.size() % 2 ? r[r.size() / 2] : 0.5 * (r[r.size() / 2 - 1] + r[r.size() / 2]);
    return FS_OK;
}

fs_status fs_problem_info(const fs_problem* p, int32_t* path, int32_t* d_pad, int32_t* f_splits,
                          int32_t* g_splits) {
    if (!p) return fail(FS_ERR_INVALID_ARG, "NULL handle");
    if (path) *path = p->refine ? 5 : p->path;
    if (d_pad) *d_pad = p->dp;
    if (f_splits) *f_splits = p->f_split;
    if (g_splits) *g_splits = p->g_split;
    return FS_OK;
}

}  // extern "C"

namespace {

// ---------------------------------------------------------------------------
// Block-sparse low-dimensional form ("FlashSinkhorn 2" explainer, sections on
// cutting space and on guaranteeing the skip; see fs_bsparse.hip).

// Work plan of the block-sparse pass: the kept tiles are dealt so that about
// kBsTarget workgroups share them evenly (a row block's list to at most
// kBsMaxSplit of them); the kernel is launched with row blocks + kBsTarget
// workgroups, the plan's upper bound.
constexpr int kBsTarget = 4096;
constexpr int kBsMaxSplit = 16;

// Chunks of kChunkKeys keys in a key cloud of n points (0 above the LDS flag
// limit of the screening).
int bs_chunks_of(int64_t n) {
    const int64_t c = (n + kChunkKeys - 1) / kChunkKeys;
    return c <= kMaxChunks ? (int)c : 0;
}

// The chunks the screening uses for a key cloud of n points: the two-level
// form from min_chunks chunks on (below that, its one-workgroup-per-chunk fit
// costs more latency than the first level saves), else 0.
int bs_chunks(int64_t n, int min_chunks) {
    const int c = bs_chunks_of(n);
    return c >= std::max(min_chunks, 2) ? c : 0;
}

// The per-block fits of the row side's potential `cur` and the key side's
// `other`, then the screening of side 0 (rows X, keys Y) or 1 (rows Y, keys
// X) into the problem's list buffer.
fs_status bs_screen_side(fs_problem* p, bool f_side, float eps, float delta, const float* cur,
                         const float* other, hipStream_t s) {
    const int side = f_side ? 0 : 1;
    const Cloud& R = f_side ? p->X : p->Y;
    const Cloud& K = f_side ? p->Y : p->X;
    const float* cR = p->centre + (f_side ? 0 : p->d);
    const float* cK = p->centre + (f_side ? p->d : 0);
    const int nbR = p->bs_nbR[side], nbK = p->bs_nbK[side];
    const float c_bias = (float)(1.4426950408889634 / (double)eps);
    hipError_t e;
    if ((e = launch_block_fit((const float*)R.ops, cR, p->d, R.n, 256, false, cur, nullptr, c_bias,
                              p->bs_rfit, s)) != hipSuccess ||
        (e = launch_block_fit((const float*)K.ops, cK, p->d, K.n, 32, true, other, K.lw2, c_bias,
                              p->bs_kfit, s)) != hipSuccess)
        return hip_fail(e, "block fit launch");
    const float thr2 = delta > 0.f ? (float)std::log2((double)delta / (double)nbK) : -INFINITY;
    const int sentinel = (int)(K.n_pad / 32);
    // the two-level form once there are at least 4 chunks of 256 key blocks
    const int nbC = bs_chunks(K.n, p->bs_min_chunks);
    if (nbC > 0 && (e = launch_chunk_fit((const float*)K.ops, cK, p->d, K.n, other, K.lw2,
                                         c_bias, p->bs_cbox, p->bs_cfit, s)) != hipSuccess)
        return hip_fail(e, "chunk fit launch");
    if ((e = launch_screen(p->bs_rbox[side], p->bs_rfit, nbR, p->bs_kbox[side], p->bs_kfit, nbK,
                           c_bias, thr2, p->bs_mag, p->bs_list, p->bs_cnt[side], p->bs_best,
                           cR, cK, p->d, p->bs_org, p->bs_cap[side], sentinel, p->bs_cbox,
                           p->bs_cfit, nbC, s)) != hipSuccess)
        return hip_fail(e, "screening launch");
    p->bs_last_side = side;
    return FS_OK;
}

fs_status fs_bs_half_step(fs_problem* p, bool f_side, float eps, float delta, const float* cur,
                          const float* other, float* out, float* resid, hipStream_t s,
                          hipEvent_t eb, hipEvent_t ee) {
    const int side = f_side ? 0 : 1;
    const Cloud& K = f_side ? p->Y : p->X;
    const int nbR = p->bs_nbR[side];
    const int sentinel = (int)(K.n_pad / 32);
    fs_status st = bs_screen_side(p, f_side, eps, delta, cur, other, s);
    if (st != FS_OK) return st;
    hipError_t e;
    if ((e = launch_split_plan(p->bs_cnt[side], nbR, kBsTarget, kBsMaxSplit, p->bs_nsplit,
                               p->bs_map, p->bs_total, s)) != hipSuccess)
        return hip_fail(e, "split plan launch");
    LseArgs a = base_args(p, f_side, eps);
    a.key_pot = other;
    a.out = out;
    a.mode = 0;
    a.cur = resid ? cur : nullptr;
    a.resid_out = resid;
    a.n_split = kBsMaxSplit;  // the partial form; the splits are planned per row block
    a.part = p->bs_part;
    a.bs_nsplit = p->bs_nsplit;
    a.bs_map = p->bs_map;
    a.bs_total = p->bs_total;
    a.bs_grid = nbR + kBsTarget;
    a.keys_per_split = (int)K.n_pad;
    a.krec_keys = (int)K.n_pad + 32;
    a.bs_list = p->bs_list;
    a.bs_count = p->bs_cnt[side];
    a.bs_best = p->bs_best;
    a.bs_org = p->bs_org;
    a.bs_cap = p->bs_cap[side];
    a.bs_sentinel = sentinel;
    if ((e = launch_lse(p->path, a, s, eb, ee)) != hipSuccess)
        return hip_fail(e, f_side ? "block-sparse f-update launch" : "block-sparse g-update launch");
    return FS_OK;
}

struct BsLayout {
    size_t rbox[2], kbox[2], rfit, kfit, cbox, cfit, cnt[2], best, org, nsplit, map, ptotal, list,
        part, total;
};

BsLayout bs_layout(const fs_problem* p) {
    BsLayout L{};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = up(o + bytes, kAlign);
        return at;
    };
    const int64_t n = p->n, m = p->m;
    const int64_t nbR[2] = {(n + 255) / 256, (m + 255) / 256};
    const int64_t nbK[2] = {(m + 31) / 32, (n + 31) / 32};
    for (int q = 0; q < 2; ++q) {
        L.rbox[q] = take(sizeof(float4) * 2 * nbR[q]);
        L.kbox[q] = take(sizeof(float4) * 2 * nbK[q]);
        L.cnt[q] = take(sizeof(int) * nbR[q]);
    }
    L.rfit = take(sizeof(float4) * 2 * std::max(nbR[0], nbR[1]));
    L.best = take(sizeof(int) * std::max(nbR[0], nbR[1]));
    L.org = take(sizeof(float4) * 2 * std::max(nbR[0], nbR[1]));
    L.nsplit = take(sizeof(int) * std::max(nbR[0], nbR[1]));
    L.map = take(sizeof(int) * 2 * (std::max(nbR[0], nbR[1]) + kBsTarget));
    L.ptotal = take(sizeof(int) * 4);
    L.kfit = take(sizeof(float4) * 2 * std::max(nbK[0], nbK[1]));
    const int64_t nbC = std::max<int64_t>(1, std::max(bs_chunks_of(m), bs_chunks_of(n)));
    L.cbox = take(sizeof(float4) * 2 * nbC);
    L.cfit = take(sizeof(float4) * 2 * nbC);
    const int64_t cap0 = (nbK[0] + 15) / 16 * 16, cap1 = (nbK[1] + 15) / 16 * 16;
    L.list = take(sizeof(int) * (size_t)std::max(nbR[0] * cap0, nbR[1] * cap1));
    L.part = take(sizeof(float2) * kBsMaxSplit * (size_t)std::max(n, m));
    L.total = o;
    return L;
}

fs_status bs_check(const fs_problem* p) {
    if (!p) return fail(FS_ERR_INVALID_ARG, "NULL handle");
    if (p->path != PATH_SMALL || p->d > 3 || p->cost != FS_COST_SQEUCLIDEAN)
        return fail(FS_ERR_INVALID_ARG,
                    "the block-sparse form needs d <= 3, fp32 matrix-core scores (FS_PREC_AUTO or "
                    "FS_PREC_FP32) and the squared-Euclidean cost");
    // the kernel addresses records with 32-bit offsets: (padded keys + 32) x 32 bytes
    if ((std::max(p->X.n_pad, p->Y.n_pad) + 32) * 32 > ((int64_t)1 << 32))
        return fail(FS_ERR_INVALID_ARG, "the block-sparse form supports up to 2^27 - 544 points");
    if (small_rows_per_block() != 256) return fail(FS_ERR_DEVICE, "row block mismatch");
    return FS_OK;
}

}  // namespace

extern "C" {

size_t fs_morton_workspace_bytes(int64_t n, int32_t d) {
    if (n < 1 || n > 0x7fffffffLL || d < 1 || d > 8) return 0;
    return morton_workspace_bytes(n);
}

fs_status fs_morton_sort(const float* X, const float* w, int64_t n, int32_t d, float* X_sorted,
                         float* w_sorted, int32_t* perm, void* workspace, size_t workspace_bytes,
                         void* stream) {
    if (!X || !X_sorted || !perm) return fail(FS_ERR_INVALID_ARG, "X, X_sorted and perm must be non-NULL");
    if ((w == nullptr) != (w_sorted == nullptr))
        return fail(FS_ERR_INVALID_ARG, "w and w_sorted must both be given or both be NULL");
    if (n < 1 || n > 0x7fffffffLL) return fail(FS_ERR_INVALID_ARG, "n must be in [1, 2^31-1]");
    if (d < 1 || d > 8) return fail(FS_ERR_INVALID_ARG, "Morton order supports 1 <= d <= 8");
    if (overlaps(X, 4 * (size_t)n * d, X_sorted, 4 * (size_t)n * d) ||
        (w && overlaps(w, 4 * (size_t)n, w_sorted, 4 * (size_t)n)))
        return fail(FS_ERR_INVALID_ARG, "outputs may not overlap inputs");
    if (!workspace || (uintptr_t)workspace % kAlign)
        return fail(FS_ERR_WORKSPACE, "workspace must be non-NULL and %zu-byte aligned", kAlign);
    if (workspace_bytes < morton_workspace_bytes(n))
        return fail(FS_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                    morton_workspace_bytes(n));
    int dev = 0;
    fs_status st = check_device(&dev);
    if (st != FS_OK) return st;
    hipError_t e = launch_morton_sort(X, w, n, d, X_sorted, w_sorted, perm, workspace,
                                      (hipStream_t)stream);
    return e == hipSuccess ? FS_OK : hip_fail(e, "fs_morton_sort");
}

fs_status fs_unpermute(const float* src, const int32_t* perm, int64_t n, int32_t width, float* dst,
                       void* stream) {
    if (!src || !perm || !dst) return fail(FS_ERR_INVALID_ARG, "NULL argument");
    if (n < 1 || n > 0x7fffffffLL || width < 1 || width > 65536)
        return fail(FS_ERR_INVALID_ARG, "n must be in [1, 2^31-1] and width in [1, 65536]");
    if (overlaps(src, 4 * (size_t)n * width, dst, 4 * (size_t)n * width))
        return fail(FS_ERR_INVALID_ARG, "dst overlaps src");
    hipError_t e = launch_unpermute(src, perm, n, width, dst, (hipStream_t)stream);
    return e == hipSuccess ? FS_OK : hip_fail(e, "fs_unpermute");
}

size_t fs_bs_workspace_bytes(const fs_problem* p) {
    if (!p || p->path != PATH_SMALL || p->d > 3) return 0;
    return bs_layout(p).total;
}

fs_status fs_bs_attach(fs_problem* p, void* workspace, size_t workspace_bytes, void* stream) {
    fs_status st = bs_check(p);
    if (st != FS_OK) return st;
    const BsLayout L = bs_layout(p);
    if (!workspace || (uintptr_t)workspace % kAlign)
        return fail(FS_ERR_WORKSPACE, "workspace must be non-NULL and %zu-byte aligned", kAlign);
    if (workspace_bytes < L.total)
        return fail(FS_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                    L.total);
    char* w = (char*)workspace;
    const Cloud* rows[2] = {&p->X, &p->Y};
    const Cloud* keys[2] = {&p->Y, &p->X};
    for (int q = 0; q < 2; ++q) {
        p->bs_nbR[q] = (int)((rows[q]->n + 255) / 256);
        p->bs_nbK[q] = (int)((keys[q]->n + 31) / 32);
        p->bs_cap[q] = (p->bs_nbK[q] + 15) / 16 * 16;
        p->bs_rbox[q] = (float4*)(w + L.rbox[q]);
        p->bs_kbox[q] = (float4*)(w + L.kbox[q]);
        p->bs_cnt[q] = (int*)(w + L.cnt[q]);
    }
    p->bs_rfit = (float4*)(w + L.rfit);
    p->bs_kfit = (float4*)(w + L.kfit);
    p->bs_cbox = (float4*)(w + L.cbox);
    p->bs_cfit = (float4*)(w + L.cfit);
    {
        const char* env = std::getenv("FS_BS_MIN_CHUNKS");
        const long v = env ? std::strtol(env, nullptr, 10) : 64;
        p->bs_min_chunks = v >= 2 && v <= kMaxChunks ? (int)v : 64;
    }
    p->bs_list = (int*)(w + L.list);
    p->bs_part = (float2*)(w + L.part);
    p->bs_best = (int*)(w + L.best);
    p->bs_org = (float4*)(w + L.org);
    p->bs_nsplit = (int*)(w + L.nsplit);
    p->bs_map = (int*)(w + L.map);
    p->bs_total = (int*)(w + L.ptotal);
    p->bs_last_side = -1;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    const float* cx = p->centre;
    const float* cy = p->centre + p->d;
    if ((e = launch_block_boxes((const float*)p->X.ops, cx, p->d, p->n, 256, p->bs_rbox[0], s)) !=
            hipSuccess ||
        (e = launch_block_boxes((const float*)p->Y.ops, cy, p->d, p->m, 32, p->bs_kbox[0], s)) !=
            hipSuccess ||
        (e = launch_block_boxes((const float*)p->Y.ops, cy, p->d, p->m, 256, p->bs_rbox[1], s)) !=
            hipSuccess ||
        (e = launch_block_boxes((const float*)p->X.ops, cx, p->d, p->n, 32, p->bs_kbox[1], s)) !=
            hipSuccess)
        return hip_fail(e, "block boxes");
    // coordinate magnitude for the screening's rounding margin (read back once)
    std::vector<float4> hb(2 * (size_t)std::max(p->bs_nbR[0], p->bs_nbR[1]));
    double M[3] = {0, 0, 0};
    for (int q = 0; q < 2; ++q) {
        const size_t cnt = 2 * (size_t)p->bs_nbR[q];
        if ((e = hipMemcpyAsync(hb.data(), p->bs_rbox[q], sizeof(float4) * cnt,
                                hipMemcpyDeviceToHost, s)) != hipSuccess ||
            (e = hipStreamSynchronize(s)) != hipSuccess)
            return hip_fail(e, "box readback");
        for (size_t k = 0; k < cnt; ++k) {
            M[0] = std::max(M[0], (double)std::fabs(hb[k].x));
            M[1] = std::max(M[1], (double)std::fabs(hb[k].y));
            M[2] = std::max(M[2], (double)std::fabs(hb[k].z));
        }
    }
    p->bs_mag = (float)(1.0 + 4.0 * (M[0] * M[0] + M[1] * M[1] + M[2] * M[2]));
    p->bs_on = true;
    return FS_OK;
}

fs_status fs_bs_lse_update_f(fs_problem* p, float eps, float delta, const float* g,
                             const float* f_cur, float* f_out, float* row_resid, void* stream) {
    fs_status st = bs_check(p);
    if (st != FS_OK) return st;
    if (!p->bs_on) return fail(FS_ERR_INVALID_ARG, "call fs_bs_attach first");
    if (!g || !f_cur || !f_out) return fail(FS_ERR_INVALID_ARG, "NULL g, f_cur or f_out");
    if (!eps_ok(eps)) return fail(FS_ERR_INVALID_ARG, "eps must be finite and > 0");
    if (!(delta >= 0.f && delta < 1.f)) return fail(FS_ERR_INVALID_ARG, "delta must be in [0, 1)");
    if (row_resid && overlaps(f_out, 4 * p->n, f_cur, 4 * p->n))
        return fail(FS_ERR_INVALID_ARG, "f_out may not overlap f_cur when a residual is asked");
    if (overlaps(f_out, 4 * p->n, g, 4 * p->m)) return fail(FS_ERR_INVALID_ARG, "f_out overlaps g");
    return fs_bs_half_step(p, true, eps, delta, f_cur, g, f_out, row_resid, (hipStream_t)stream,
                           nullptr, nullptr);
}

fs_status fs_bs_lse_update_g(fs_problem* p, float eps, float delta, const float* f,
                             const float* g_cur, float* g_out, float* col_resid, void* stream) {
    fs_status st = bs_check(p);
    if (st != FS_OK) return st;
    if (!p->bs_on) return fail(FS_ERR_INVALID_ARG, "call fs_bs_attach first");
    if (!f || !g_cur || !g_out) return fail(FS_ERR_INVALID_ARG, "NULL f, g_cur or g_out");
    if (!eps_ok(eps)) return fail(FS_ERR_INVALID_ARG, "eps must be finite and > 0");
    if (!(delta >= 0.f && delta < 1.f)) return fail(FS_ERR_INVALID_ARG, "delta must be in [0, 1)");
    if (col_resid && overlaps(g_out, 4 * p->m, g_cur, 4 * p->m))
        return fail(FS_ERR_INVALID_ARG, "g_out may not overlap g_cur when a residual is asked");
    if (overlaps(g_out, 4 * p->m, f, 4 * p->n)) return fail(FS_ERR_INVALID_ARG, "g_out overlaps f");
    return fs_bs_half_step(p, false, eps, delta, g_cur, f, g_out, col_resid, (hipStream_t)stream,
                           nullptr, nullptr);
}

fs_status fs_bs_sinkhorn_solve(fs_problem* p, const fs_solve_opts* o, float delta, float* f,
                               float* g, fs_solve_info* info, void* stream) {
    fs_status st = bs_check(p);
    if (st != FS_OK) return st;
    if (!p->bs_on) return fail(FS_ERR_INVALID_ARG, "call fs_bs_attach first");
    if (!o || !f || !g) return fail(FS_ERR_INVALID_ARG, "NULL opts, f or g");
    if (o->n_stages < 1) return fail(FS_ERR_INVALID_ARG, "n_stages must be >= 1");
    if (o->iters_per_stage < 0) return fail(FS_ERR_INVALID_ARG, "iters_per_stage must be >= 0");
    if (o->refine_iters < 0) return fail(FS_ERR_INVALID_ARG, "refine_iters must be >= 0");
    if (!eps_ok(o->eps_end) || (o->n_stages > 1 && !eps_ok(o->eps_start)))
        return fail(FS_ERR_INVALID_ARG, "eps_start/eps_end must be finite and > 0");
    if (!std::isfinite(o->tol)) return fail(FS_ERR_INVALID_ARG, "tol must be finite");
    if (o->tol > 0.f && o->check_every < 1)
        return fail(FS_ERR_INVALID_ARG, "check_every must be >= 1 when tol > 0");
    if (!(delta >= 0.f && delta < 1.f)) return fail(FS_ERR_INVALID_ARG, "delta must be in [0, 1)");
    if (overlaps(f, 4 * p->n, g, 4 * p->m)) return fail(FS_ERR_INVALID_ARG, "f overlaps g");
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    KernelTimer timer;
    if (o->time_kernels) {
        const size_t half_steps = 2 * (size_t)o->n_stages * (size_t)o->iters_per_stage + 8;
        if ((e = timer.reserve(half_steps)) != hipSuccess) return hip_fail(e, "hipEventCreate");
    }
    const bool use_tol = o->tol > 0.f;
    int done = 0;
    float resid = -1.f, eps = o->eps_end;
    bool converged = false;
    auto check = [&](float eps_c) -> fs_status {
        // both terms of the residual of (f, g) (of the plan on the kept
        // blocks) from dry-run updates into pot_tmp: the column term, then
        // the row term
        fs_status s2 = fs_bs_half_step(p, false, eps_c, delta, g, f, p->pot_tmp, p->scal + 1, s,
                                       nullptr, nullptr);
        if (s2 == FS_OK)
            s2 = fs_bs_half_step(p, true, eps_c, delta, f, g, p->pot_tmp, p->scal, s, nullptr,
                                 nullptr);
        if (s2 != FS_OK) return s2;
        float h[2] = {0.f, 0.f};
        hipError_t e2 = hipMemcpyAsync(h, p->scal, sizeof(h), hipMemcpyDeviceToHost, s);
        if (e2 == hipSuccess) e2 = hipStreamSynchronize(s);
        if (e2 != hipSuccess) return hip_fail(e2, "residual readback");
        resid = h[0] + h[1];
        return FS_OK;
    };
    for (int si = 0; si < o->n_stages && !converged; ++si) {
        eps = o->n_stages == 1
                  ? o->eps_end
                  : (float)((double)o->eps_start *
                            std::pow((double)o->eps_end / (double)o->eps_start,
                                     (double)si / (double)(o->n_stages - 1)));
        for (int it = 0; it < o->iters_per_stage; ++it) {
            hipEvent_t eb = nullptr, ee = nullptr;
            if (o->time_kernels) timer.next(eb, ee);
            if ((st = fs_bs_half_step(p, true, eps, delta, f, g, f, nullptr, s, eb, ee)) != FS_OK)
                return st;
            if (o->time_kernels) timer.next(eb, ee);
            if ((st = fs_bs_half_step(p, false, eps, delta, g, f, g, nullptr, s, eb, ee)) != FS_OK)
                return st;
            ++done;
            if (use_tol && done % o->check_every == 0) {
                if ((st = check(eps)) != FS_OK) return st;
                if (resid <= o->tol) {
                    converged = true;
                    break;
                }
            }
        }
    }
    if (use_tol && !converged && (done == 0 || done % o->check_every != 0)) {
        if ((st = check(eps)) != FS_OK) return st;
        converged = resid <= o->tol;
    }
    float lse_ms = 0.f;
    int lse_n = 0;
    if (o->time_kernels) {
        if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(e, "timing sync");
        for (size_t k = 0; k + 1 < timer.used; k += 2) {
            float ms = 0.f;
            if ((e = hipEventElapsedTime(&ms, timer.ev[k], timer.ev[k + 1])) != hipSuccess)
                return hip_fail(e, "hipEventElapsedTime");
            lse_ms += ms;
            ++lse_n;
        }
    }
    if (info) {
        info->iters_done = done;
        info->final_eps = eps;
        info->residual = use_tol ? resid : -1.f;
        info->lse_launches = lse_n;
        info->lse_ms = lse_ms;
        info->single_launch = 0;
    }
    if (use_tol && !converged)
        return fail(FS_ERR_NOT_CONVERGED, "residual %g above tol %g after %d iterations",
                    (double)resid, (double)o->tol, done);
    return FS_OK;
}

}  // extern "C"

namespace {

// Block-sparse transport or gradient of one side: screening of that side at
// (f, g), then one launch over its kept blocks.  Side 0: rows X (potential
// f), keys Y (g), V [m][dv] -> U [n][dv]; side 1 the roles swapped.  V == NULL
// asks for the gradient 2 sum_j P_ij (x_i - y_j) (dv = d).
fs_status bs_transport_side(fs_problem* p, bool f_side, float eps, float delta, const float* f,
                            const float* g, const float* V, int32_t dv, float* U, int divide,
                            hipStream_t s) {
    const int side = f_side ? 0 : 1;
    const Cloud& R = f_side ? p->X : p->Y;
    const Cloud& K = f_side ? p->Y : p->X;
    const float* rpot = f_side ? f : g;
    const float* kpot = f_side ? g : f;
    fs_status st = bs_screen_side(p, f_side, eps, delta, rpot, kpot, s);
    if (st != FS_OK) return st;
    const float c_bias = (float)(1.4426950408889634 / (double)eps);
    const float c_score = (float)(2.8853900817779268 / (double)eps);
    hipError_t e = launch_bs_transport(
        (const float*)R.ops, R.nrm, R.lw2, rpot, R.w, (int)R.n, (const float*)K.ops, K.nrm, K.lw2,
        kpot, (int)K.n, V, dv, c_bias, c_score, divide, p->bs_list, p->bs_cnt[side],
        p->bs_cap[side], p->bs_nbR[side], p->centre + (f_side ? 0 : p->d),
        p->centre + (f_side ? p->d : 0), U, s);
    if (e != hipSuccess) return hip_fail(e, "block-sparse transport launch");
    return FS_OK;
}

fs_status bs_transport_check(fs_problem* p, float eps, float delta, const float* f,
                             const float* g) {
    fs_status st = bs_check(p);
    if (st != FS_OK) return st;
    if (!p->bs_on) return fail(FS_ERR_INVALID_ARG, "call fs_bs_attach first");
    if (!f || !g) return fail(FS_ERR_INVALID_ARG, "NULL f or g");
    if (!eps_ok(eps)) return fail(FS_ERR_INVALID_ARG, "eps must be finite and > 0");
    if (!(delta >= 0.f && delta < 1.f)) return fail(FS_ERR_INVALID_ARG, "delta must be in [0, 1)");
    return FS_OK;
}

}  // namespace

extern "C" {

fs_status fs_bs_apply_transport(fs_problem* p, float eps, float delta, const float* f,
                               const float* g, const float* V, int32_t dv, float* U,
                               int32_t divide_by_a, void* stream) {
    fs_status st = bs_transport_check(p, eps, delta, f, g);
    if (st != FS_OK) return st;
    if (!V || !U) return fail(FS_ERR_INVALID_ARG, "NULL V or U");
    if (dv < 1 || dv > 16) return fail(FS_ERR_INVALID_ARG, "dv must be in [1, 16] (got %d)", dv);
    if (overlaps(U, 4 * (size_t)p->n * dv, V, 4 * (size_t)p->m * dv) ||
        overlaps(U, 4 * (size_t)p->n * dv, f, 4 * (size_t)p->n) ||
        overlaps(U, 4 * (size_t)p->n * dv, g, 4 * (size_t)p->m))
        return fail(FS_ERR_INVALID_ARG, "U overlaps an input");
    return bs_transport_side(p, true, eps, delta, f, g, V, dv, U, divide_by_a ? 1 : 0,
                             (hipStream_t)stream);
}

fs_status fs_bs_apply_transport_t(fs_problem* p, float eps, float delta, const float* f,
                                 const float* g, const float* W, int32_t dv, float* U,
                                 int32_t divide_by_b, void* stream) {
    fs_status st = bs_transport_check(p, eps, delta, f, g);
    if (st != FS_OK) return st;
    if (!W || !U) return fail(FS_ERR_INVALID_ARG, "NULL W or U");
    if (dv < 1 || dv > 16) return fail(FS_ERR_INVALID_ARG, "dv must be in [1, 16] (got %d)", dv);
    if (overlaps(U, 4 * (size_t)p->m * dv, W, 4 * (size_t)p->n * dv) ||
        overlaps(U, 4 * (size_t)p->m * dv, f, 4 * (size_t)p->n) ||
        overlaps(U, 4 * (size_t)p->m * dv, g, 4 * (size_t)p->m))
        return fail(FS_ERR_INVALID_ARG, "U overlaps an input");
    return bs_transport_side(p, false, eps, delta, f, g, W, dv, U, divide_by_b ? 1 : 0,
                             (hipStream_t)stream);
}

fs_status fs_bs_gradient(fs_problem* p, float eps, float delta, const float* f, const float* g,
                         float* grad_x, float* grad_y, void* stream) {
    fs_status st = bs_transport_check(p, eps, delta, f, g);
    if (st != FS_OK) return st;
    const size_t bx = 4 * (size_t)p->n * p->d, by = 4 * (size_t)p->m * p->d;
    if (grad_x && (overlaps(grad_x, bx, f, 4 * (size_t)p->n) ||
                   overlaps(grad_x, bx, g, 4 * (size_t)p->m)))
        return fail(FS_ERR_INVALID_ARG, "grad_x overlaps f or g");
    if (grad_y && (overlaps(grad_y, by, f, 4 * (size_t)p->n) ||
                   overlaps(grad_y, by, g, 4 * (size_t)p->m) ||
                   (grad_x && overlaps(grad_y, by, grad_x, bx))))
        return fail(FS_ERR_INVALID_ARG, "grad_y overlaps f, g or grad_x");
    hipStream_t s = (hipStream_t)stream;
    if (grad_x && (st = bs_transport_side(p, true, eps, delta, f, g, nullptr, p->d, grad_x, 0,
                                          s)) != FS_OK)
        return st;
    if (grad_y && (st = bs_transport_side(p, false, eps, delta, f, g, nullptr, p->d, grad_y, 0,
                                          s)) != FS_OK)
        return st;
    return FS_OK;
}

fs_status fs_centroids(const float* P, const float* w, int64_t n, int32_t d, int32_t cell,
                       float* C, float* W, void* stream) {
    if (!P || !w || !C || !W) return fail(FS_ERR_INVALID_ARG, "NULL argument");
    if (n < 1 || n > 0x7fffffffLL || d < 1 || d > 8 || cell < 1)
        return fail(FS_ERR_INVALID_ARG, "need 1 <= n <= 2^31-1, 1 <= d <= 8, cell >= 1");
    const int64_t nc = (n + cell - 1) / cell;
    if (overlaps(C, 4 * (size_t)nc * d, P, 4 * (size_t)n * d) ||
        overlaps(W, 4 * (size_t)nc, w, 4 * (size_t)n))
        return fail(FS_ERR_INVALID_ARG, "outputs may not overlap inputs");
    hipError_t e = launch_centroids(P, w, n, d, cell, C, W, (hipStream_t)stream);
    return e == hipSuccess ? FS_OK : hip_fail(e, "fs_centroids");
}

fs_status fs_lift(const float* F, int64_t n, int32_t cell, float* f, void* stream) {
    if (!F || !f) return fail(FS_ERR_INVALID_ARG, "NULL argument");
    if (n < 1 || n > 0x7fffffffLL || cell < 1)
        return fail(FS_ERR_INVALID_ARG, "need 1 <= n <= 2^31-1 and cell >= 1");
    if (overlaps(F, 4 * (size_t)((n + cell - 1) / cell), f, 4 * (size_t)n))
        return fail(FS_ERR_INVALID_ARG, "f overlaps F");
    hipError_t e = launch_lift(F, n, cell, f, (hipStream_t)stream);
    return e == hipSuccess ? FS_OK : hip_fail(e, "fs_lift");
}

size_t fs_sampled_workspace_bytes(int32_t nrows, int32_t ncols) {
    if (nrows < 0 || ncols < 0) return 0;
    return up(sizeof(float2) * ((size_t)nrows + ncols + 1), kAlign);
}

fs_status fs_sampled_marginal_error(const float* X, const float* Y, const float* a,
                                    const float* b, int64_t n, int64_t m, int32_t d, float eps,
                                    const float* f, const float* g, const int32_t* rows,
                                    int32_t nrows, const int32_t* cols, int32_t ncols,
                                    float* out2, void* workspace, size_t workspace_bytes,
                                    void* stream) {
    if (!X || !Y || !a || !b || !f || !g || !out2 || (nrows > 0 && !rows) || (ncols > 0 && !cols))
        return fail(FS_ERR_INVALID_ARG, "NULL argument");
    if (n < 1 || m < 1 || n > 0x7fffffffLL || m > 0x7fffffffLL || d < 1 || d > 8)
        return fail(FS_ERR_INVALID_ARG, "need 1 <= n, m <= 2^31-1 and 1 <= d <= 8");
    if (nrows < 0 || ncols < 0 || nrows > 1 << 20 || ncols > 1 << 20)
        return fail(FS_ERR_INVALID_ARG, "sample counts must be in [0, 2^20]");
    if (!eps_ok(eps)) return fail(FS_ERR_INVALID_ARG, "eps must be finite and > 0");
    if (!workspace || (uintptr_t)workspace % kAlign ||
        workspace_bytes < fs_sampled_workspace_bytes(nrows, ncols))
        return fail(FS_ERR_WORKSPACE, "workspace must be 256-byte aligned and hold %zu bytes",
                    fs_sampled_workspace_bytes(nrows, ncols));
    const float c_bias = (float)(1.4426950408889634 / (double)eps);
    hipError_t e = launch_sampled_marginal(X, Y, a, b, n, m, d, c_bias, f, g, rows, nrows, cols,
                                           ncols, (float2*)workspace, out2, (hipStream_t)stream);
    return e == hipSuccess ? FS_OK : hip_fail(e, "fs_sampled_marginal_error");
}

fs_status fs_bs_coarse_start(fs_problem* coarse, const fs_solve_opts* opts, int32_t more_iters,
                             float coarse_delta, const float* X, const float* Y, const float* a, const float* b,
                             int64_t n, int64_t m, int32_t d, int32_t cell, float check_tol,
                             int32_t max_rounds, const int32_t* rows, int32_t nrows,
                             const int32_t* cols, int32_t ncols, float* F, float* G, float* f,
                             float* g, void* workspace, size_t workspace_bytes,
                             fs_coarse_info* info, void* stream) {
    if (!coarse || !opts || !F || !G || !f || !g) return fail(FS_ERR_INVALID_ARG, "NULL argument");
    if (cell < 1 || max_rounds < 1 || more_iters < 0 || !(check_tol >= 0.f))
        return fail(FS_ERR_INVALID_ARG, "need cell >= 1, max_rounds >= 1, more_iters >= 0, "
                                        "check_tol >= 0");
    if (coarse->n != (n + cell - 1) / cell || coarse->m != (m + cell - 1) / cell ||
        coarse->d != d)
        return fail(FS_ERR_INVALID_ARG, "the coarse problem must hold the centroids of cells "
                                        "of %d points of both clouds", cell);
    if (!(coarse_delta >= 0.f && coarse_delta < 1.f))
        return fail(FS_ERR_INVALID_ARG, "coarse_delta must be in [0, 1)");
    if (coarse_delta > 0.f && !coarse->bs_on)
        return fail(FS_ERR_INVALID_ARG, "coarse_delta > 0 needs fs_bs_attach on the coarse problem");
    if (workspace_bytes < fs_sampled_workspace_bytes(nrows, ncols) + kAlign)
        return fail(FS_ERR_WORKSPACE, "workspace must hold %zu bytes",
                    fs_sampled_workspace_bytes(nrows, ncols) + kAlign);
    hipStream_t s = (hipStream_t)stream;
    // the coarse solves: dense, or block-sparse with coarse_delta
    auto coarse_solve = [&](const fs_solve_opts* o) {
        return coarse_delta > 0.f ? fs_bs_sinkhorn_solve(coarse, o, coarse_delta, F, G, nullptr,
                                                         stream)
                                  : fs_sinkhorn_solve(coarse, o, F, G, nullptr, stream);
    };
    fs_status st = coarse_solve(opts);
    if (st != FS_OK && st != FS_ERR_NOT_CONVERGED) return st;
    float* out2 = (float*)((char*)workspace + fs_sampled_workspace_bytes(nrows, ncols));
    fs_solve_opts more{};
    more.n_stages = 1;
    more.eps_end = opts->eps_end;
    more.eps_start = opts->eps_end;
    more.iters_per_stage = more_iters;
    more.warm_start = 1;
    float err[2] = {0.f, 0.f};
    int k = 0;
    bool ok = false;
    for (;;) {
        hipError_t e;
        if ((e = launch_lift(F, n, cell, f, s)) != hipSuccess ||
            (e = launch_lift(G, m, cell, g, s)) != hipSuccess)
            return hip_fail(e, "lift");
        if ((st = fs_sampled_marginal_error(X, Y, a, b, n, m, d, opts->eps_end, f, g, rows, nrows,
                                            cols, ncols, out2, workspace, workspace_bytes,
                                            stream)) != FS_OK)
            return st;
        if ((e = hipMemcpyAsync(err, out2, sizeof(err), hipMemcpyDeviceToHost, s)) != hipSuccess ||
            (e = hipStreamSynchronize(s)) != hipSuccess)
            return hip_fail(e, "check readback");
        ++k;
        ok = err[0] <= check_tol && err[1] <= check_tol;
        if (ok || k >= max_rounds) break;
        if ((st = coarse_solve(&more)) != FS_OK) return st;
    }
    if (info) {
        info->rounds = k;
        info->accepted = ok ? 1 : 0;
        info->err_rows = err[0];
        info->err_cols = err[1];
    }
    return FS_OK;
}

fs_status fs_bs_shape(const fs_problem* p, int32_t side, int32_t* n_row_blocks,
                      int32_t* n_key_blocks, int32_t* list_stride) {
    if (!p || !p->bs_on) return fail(FS_ERR_INVALID_ARG, "NULL handle or fs_bs_attach not called");
    if (side != 0 && side != 1) return fail(FS_ERR_INVALID_ARG, "side must be 0 or 1");
    if (n_row_blocks) *n_row_blocks = p->bs_nbR[side];
    if (n_key_blocks) *n_key_blocks = p->bs_nbK[side];
    if (list_stride) *list_stride = p->bs_cap[side];
    return FS_OK;
}

fs_status fs_bs_read_screen(fs_problem* p, int32_t side, int32_t* counts, int32_t* lists,
                            void* stream) {
    if (!p || !p->bs_on) return fail(FS_ERR_INVALID_ARG, "NULL handle or fs_bs_attach not called");
    if (side != 0 && side != 1) return fail(FS_ERR_INVALID_ARG, "side must be 0 or 1");
    if (!counts) return fail(FS_ERR_INVALID_ARG, "counts is NULL");
    if (lists && p->bs_last_side != side)
        return fail(FS_ERR_INVALID_ARG, "the lists held are those of side %d", p->bs_last_side);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync(counts, p->bs_cnt[side], sizeof(int) * p->bs_nbR[side],
                                  hipMemcpyDeviceToHost, s);
    if (e == hipSuccess && lists)
        e = hipMemcpyAsync(lists, p->bs_list,
                           sizeof(int) * (size_t)p->bs_nbR[side] * p->bs_cap[side],
                           hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return e == hipSuccess ? FS_OK : hip_fail(e, "fs_bs_read_screen");
}

}  // extern "C"

namespace fs {

fs_status report(fs_status s, const char* msg) { return fail(s, "%s", msg); }

// Set-up and solve in one call, with the problem struct on this stack frame
// and every device buffer in `workspace`: nothing is allocated, on the host
// or the device.  The allocation-free entry point passes its static scratch
// array here.
fs_status solve_in_workspace(const float* X, const float* Y, const float* a, const float* b,
                             int64_t n, int64_t m, int32_t d, fs_score_prec prec,
                             const fs_solve_opts* opts, void* workspace, size_t workspace_bytes,
                             float* f, float* g, fs_solve_info* info, void* stream) {
    if (!opts) return fail(FS_ERR_INVALID_ARG, "NULL opts");
    if (opts->time_kernels)
        return fail(FS_ERR_INVALID_ARG, "time_kernels creates HIP events; not available here");
    fs_problem p;
    fs_status st = init_problem(&p, X, Y, a, b, n, m, d, 0, prec, FS_COST_SQEUCLIDEAN,
                                workspace, workspace_bytes, f, g, stream);
    if (st != FS_OK) return st;
    return fs_sinkhorn_solve(&p, opts, f, g, info, stream);
}

}  // namespace fs
