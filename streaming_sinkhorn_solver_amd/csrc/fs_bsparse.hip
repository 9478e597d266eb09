// fs_bsparse.hip -- the block-sparse pieces of the low-dimensional path:
// Morton ordering of a cloud, per-block linear fits of the potentials, and
// the screening that lists, for every block of rows, the key blocks whose
// contribution can exceed the skipping threshold.
//
// "FlashSinkhorn 2: block-sparse entropic optimal transport" (patty.io
// explainer).  Section on cutting space: sorting the points along a Z-order
// (Morton) curve puts spatial neighbours next to each other in memory, so a
// block of consecutive points is a compact group and a block of the cost
// matrix pairs two groups.  Section on guaranteeing the skip: each block is
// judged by a bound on its mass, and the threshold caps the error that
// skipped blocks can leave in every row and every column at every iteration.
// The page gives no formula; the bound used here:
//
//   f_i <= c_I + u_I.x_i on the row block I (u_I a least-squares slope of f
//   over the block, c_I the exact maximum of f_i - u_I.x_i), and
//   G_J = log2 sum_{j in J} b_j 2^((g_j - v_J.y_j) c_bias) on the key block J,
//   H(I, J) = max_{x in box I, y in box J} (u_I.x + v_J.y - |x - y|^2)
//           = sum over coordinates of a 1-D maximum over a rectangle, found
//             on one of its four edges at a clipped stationary point,
//   beta(I, J) = (c_I + H(I, J)) c_bias + G_J   (base 2),
//
// so that for every row i of I the mass of J relative to the row's target,
// sum_{j in J} b_j exp((f_i + g_j - C_ij)/eps), is at most 2^beta.  A second
// bound of the same kind comes from the dot-product split of the exponent,
// f_i + g_j - C_ij = phi_i + psi_j + 2 x_i.y_j (phi = f - |x|^2, psi =
// g - |y|^2): the fits taken of phi and psi, and H2 = max over the boxes of
// u2.x + v2.y + 2 x.y, bilinear per coordinate, at a corner.  The first is
// tight where f is nearly linear over a block, the second where phi is (a map
// that concentrates mass); beta is the smaller.  J is kept for I when
// beta >= log2(delta / N_J) (less a rounding margin), so the skipped mass of
// a row stays below delta * a_i.
//
// Layout: row blocks are the 256 rows of one workgroup of the streaming
// kernel, key blocks the 32 keys of one matrix-core block.  Per-block boxes
// are fixed for a problem (computed once); fits, bounds and lists are redone
// for every half-step, since they depend on the potentials.  The list of a
// row block holds the kept key-block indices in increasing order, padded to a
// whole tile of 16 blocks with a sentinel block of -inf records.
#include <algorithm>

#include "fs_device.hpp"
#include "fs_internal.h"

namespace fs {

namespace {

constexpr int kSortTile = 4096;  // keys per tile of a radix pass (256 threads x 16)
constexpr int kSortThreads = 256;
constexpr int kBoxParts = 256;

// ---------------------------------------------------------------- Morton order

__global__ __launch_bounds__(256) void mbox_partial_kernel(const float* __restrict__ X, int64_t n,
                                                           int d, float* pmin, float* pmax) {
    __shared__ float smin[8][256], smax[8][256];
    float lo[8], hi[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        lo[c] = INFINITY;
        hi[c] = -INFINITY;
    }
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        for (int c = 0; c < d; ++c) {
            const float v = X[i * d + c];
            lo[c] = fminf(lo[c], v);
            hi[c] = fmaxf(hi[c], v);
        }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        smin[c][threadIdx.x] = lo[c];
        smax[c][threadIdx.x] = hi[c];
    }
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
        if ((int)threadIdx.x < w)
            for (int c = 0; c < d; ++c) {
                smin[c][threadIdx.x] = fminf(smin[c][threadIdx.x], smin[c][threadIdx.x + w]);
                smax[c][threadIdx.x] = fmaxf(smax[c][threadIdx.x], smax[c][threadIdx.x + w]);
            }
        __syncthreads();
    }
    if ((int)threadIdx.x < d) {
        pmin[blockIdx.x * 8 + threadIdx.x] = smin[threadIdx.x][0];
        pmax[blockIdx.x * 8 + threadIdx.x] = smax[threadIdx.x][0];
    }
}

// lo_c and scale_c = 2^B / (hi_c - lo_c) (0 for a flat axis), each one
// correctly rounded float32 operation.
__global__ void mbox_final_kernel(const float* __restrict__ pmin, const float* __restrict__ pmax,
                                  int parts, int d, int bits, float* lo_out, float* scale_out) {
    const int c = threadIdx.x;
    if (c >= d) return;
    float lo = INFINITY, hi = -INFINITY;
    for (int p = 0; p < parts; ++p) {
        lo = fminf(lo, pmin[p * 8 + c]);
        hi = fmaxf(hi, pmax[p * 8 + c]);
    }
    const float span = __fsub_rn(hi, lo);
    lo_out[c] = lo;
    scale_out[c] = span > 0.f ? __fdiv_rn((float)(1u << bits), span) : 0.f;
}

__global__ __launch_bounds__(256) void mcode_kernel(const float* __restrict__ X, int64_t n, int d,
                                                    int bits, const float* __restrict__ lo,
                                                    const float* __restrict__ scale,
                                                    uint32_t* __restrict__ code,
                                                    int32_t* __restrict__ idx) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const uint32_t top = (1u << bits) - 1u;
    uint32_t k = 0;
    for (int c = 0; c < d; ++c) {
        const float t = __fmul_rn(__fsub_rn(X[i * d + c], lo[c]), scale[c]);
        const float fl = floorf(t);
        const uint32_t q = fl >= (float)top ? top : (uint32_t)fl;  // t >= 0
        for (int b = 0; b < bits; ++b) k |= ((q >> b) & 1u) << (b * d + c);
    }
    code[i] = k;
    idx[i] = (int32_t)i;
}

// Radix sort, 8 bits per pass, stable.  Pass: digit histogram per tile
// (digit-major), one exclusive scan, then a stable scatter: inside a tile the
// keys are ranked round by round (256 consecutive keys per round), inside a
// round by wave and lane, using ballots over the digit bits.
__global__ __launch_bounds__(kSortThreads) void rs_hist_kernel(const uint32_t* __restrict__ keys,
                                                               int64_t n, int shift, int tiles,
                                                               uint32_t* __restrict__ hist) {
    __shared__ uint32_t cnt[256];
    cnt[threadIdx.x] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kSortTile;
    for (int r = 0; r < kSortTile / kSortThreads; ++r) {
        const int64_t i = base + r * kSortThreads + threadIdx.x;
        if (i < n) atomicAdd(&cnt[(keys[i] >> shift) & 255u], 1u);
    }
    __syncthreads();
    hist[(int64_t)threadIdx.x * tiles + blockIdx.x] = cnt[threadIdx.x];
}

// Exclusive scan of len counts in place, one workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void rs_scan_kernel(uint32_t* __restrict__ v, int64_t len) {
    __shared__ uint32_t wsum[16];
    __shared__ uint32_t carry_s;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    if (tid == 0) carry_s = 0;
    __syncthreads();
    for (int64_t base = 0; base < len; base += 4096) {
        uint32_t x[4];
        uint32_t s = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t i = base + tid * 4 + k;
            x[k] = i < len ? v[i] : 0u;
            s += x[k];
        }
        // inclusive wave scan of s
        uint32_t inc = s;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t t = __shfl_up(inc, o, 64);
            if (lane >= o) inc += t;
        }
        if (lane == 63) wsum[wid] = inc;
        __syncthreads();
        uint32_t wpre = 0, total = 0;
        for (int w = 0; w < 16; ++w) {
            if (w < wid) wpre += wsum[w];
            total += wsum[w];
        }
        uint32_t run = carry_s + wpre + inc - s;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t i = base + tid * 4 + k;
            if (i < len) v[i] = run;
            run += x[k];
        }
        __syncthreads();
        if (tid == 0) carry_s += total;
        __syncthreads();
    }
}

__global__ __launch_bounds__(kSortThreads) void rs_scatter_kernel(
    const uint32_t* __restrict__ kin, const int32_t* __restrict__ vin, uint32_t* __restrict__ kout,
    int32_t* __restrict__ vout, int64_t n, int shift, int tiles, const uint32_t* __restrict__ offs) {
    __shared__ uint32_t base[256];
    __shared__ uint32_t wc[4][256];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    base[tid] = offs[(int64_t)tid * tiles + blockIdx.x];
#pragma unroll
    for (int q = 0; q < 4; ++q) wc[q][tid] = 0;
    const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    for (int r = 0; r < kSortTile / kSortThreads; ++r) {
        __syncthreads();
        const int64_t i = (int64_t)blockIdx.x * kSortTile + r * kSortThreads + tid;
        const bool valid = i < n;
        const uint32_t k = valid ? kin[i] : 0u;
        const int32_t val = valid ? vin[i] : 0;
        const uint32_t dg = (k >> shift) & 255u;
        uint64_t m = __builtin_amdgcn_ballot_w64(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const bool bit = (dg >> b) & 1u;
            const uint64_t bb = __builtin_amdgcn_ballot_w64(bit);
            m &= bit ? bb : ~bb;
        }
        const uint32_t rank = (uint32_t)__popcll(m & lt);
        if (valid && rank == 0) wc[w][dg] = (uint32_t)__popcll(m);
        __syncthreads();
        if (valid) {
            uint32_t pos = base[dg] + rank;
            for (int q = 0; q < w; ++q) pos += wc[q][dg];
            kout[pos] = k;
            vout[pos] = val;
        }
        __syncthreads();
        base[tid] += wc[0][tid] + wc[1][tid] + wc[2][tid] + wc[3][tid];
#pragma unroll
        for (int q = 0; q < 4; ++q) wc[q][tid] = 0;
    }
}

__global__ __launch_bounds__(256) void mgather_kernel(const float* __restrict__ X,
                                                      const float* __restrict__ wt, int64_t n,
                                                      int d, const int32_t* __restrict__ perm,
                                                      float* __restrict__ Xo,
                                                      float* __restrict__ wo,
                                                      int32_t* __restrict__ perm_out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int64_t s = perm[i];
    for (int c = 0; c < d; ++c) Xo[i * d + c] = X[s * d + c];
    if (wo) wo[i] = wt[s];
    perm_out[i] = (int32_t)s;
}

__global__ __launch_bounds__(256) void unpermute_kernel(const float* __restrict__ src,
                                                        const int32_t* __restrict__ perm, int64_t n,
                                                        int width, float* __restrict__ dst) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= n * width) return;
    const int64_t i = t / width;
    const int c = (int)(t - i * width);
    dst[(int64_t)perm[i] * width + c] = src[t];
}

// ---------------------------------------------------------------- block fits

// Point i of a cloud in the caller's frame: the stored centred fp32 row
// (stride 4, d <= 3) plus the cloud's centre.
__device__ __forceinline__ void load_point(const float* __restrict__ ops,
                                           const float* __restrict__ centre, int d, int64_t i,
                                           float (&x)[3]) {
    const float4 p = *(const float4*)(ops + i * 4);
    x[0] = d > 0 ? p.x + centre[0] : 0.f;
    x[1] = d > 1 ? p.y + centre[1] : 0.f;
    x[2] = d > 2 ? p.z + centre[2] : 0.f;
}

// Sum over the GS consecutive threads of a group (GS = 32: a half wave;
// GS = 256: the workgroup, via `red`, which holds 4 x 16 floats).  Fixed
// order; every thread of the group gets the total.
template <int GS, int N>
__device__ __forceinline__ void group_sum(float (&v)[N], float* red) {
#pragma unroll
    for (int q = 0; q < N; ++q) {
        float t = v[q];
#pragma unroll
        for (int o = (GS >= 64 ? 32 : GS / 2); o >= 1; o >>= 1) t += __shfl_xor(t, o, 64);
        v[q] = t;
    }
    if constexpr (GS > 64) {
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
        __syncthreads();
        if (lane == 0)
#pragma unroll
            for (int q = 0; q < N; ++q) red[w * 16 + q] = v[q];
        __syncthreads();
#pragma unroll
        for (int q = 0; q < N; ++q) v[q] = red[q] + red[16 + q] + red[32 + q] + red[48 + q];
    }
}

template <int GS>
__device__ __forceinline__ float group_max(float v, float* red) {
#pragma unroll
    for (int o = (GS >= 64 ? 32 : GS / 2); o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    if constexpr (GS > 64) {
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
        __syncthreads();
        if (lane == 0) red[w * 16] = v;
        __syncthreads();
        v = fmaxf(fmaxf(red[0], red[16]), fmaxf(red[32], red[48]));
    }
    return v;
}

// Least-squares slope of values over points from centred sums (S_xx: xx, yy,
// zz, xy, xz, yz; S_xf), regularised by 1e-6 trace (+1e-30), in double.
__device__ __forceinline__ void solve_slope(const float (&S)[9], float (&u)[3]) {
    const double lam = 1e-6 * ((double)S[0] + S[1] + S[2]) + 1e-30;
    const double a = S[0] + lam, b = S[3], c = S[4];
    const double e = S[1] + lam, f = S[5];
    const double i = S[2] + lam;
    const double r0 = S[6], r1 = S[7], r2 = S[8];
    // symmetric [[a b c] [b e f] [c f i]]
    const double A = e * i - f * f, B = c * f - b * i, C = b * f - c * e;
    const double det = a * A + b * B + c * C;
    if (!(det > 0.0) || !isfinite(det)) {
        u[0] = u[1] = u[2] = 0.f;
        return;
    }
    const double E = a * i - c * c, F = b * c - a * f, I = a * e - b * b;
    const double x0 = (A * r0 + B * r1 + C * r2) / det;
    const double x1 = (B * r0 + E * r1 + F * r2) / det;
    const double x2 = (C * r0 + F * r1 + I * r2) / det;
    u[0] = isfinite(x0) ? (float)x0 : 0.f;
    u[1] = isfinite(x1) ? (float)x1 : 0.f;
    u[2] = isfinite(x2) ? (float)x2 : 0.f;
}

// Boxes of the blocks of GS consecutive points: box[2*blk] = lo, box[2*blk+1]
// = hi (x, y, z, 0).
template <int GS>
__global__ __launch_bounds__(256) void block_box_kernel(const float* __restrict__ ops,
                                                        const float* __restrict__ centre, int d,
                                                        int64_t n, int nb, float4* __restrict__ box) {
    __shared__ float red[64];
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int blk = (int)(i / GS);
    float x[3] = {0.f, 0.f, 0.f};
    const bool valid = i < n;
    if (valid) load_point(ops, centre, d, i, x);
    float lo[3], hi[3];
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        hi[c] = group_max<GS>(valid ? x[c] : -INFINITY, red);
        lo[c] = -group_max<GS>(valid ? -x[c] : -INFINITY, red);
    }
    if ((threadIdx.x % GS) == 0 && blk < nb) {
        box[2 * blk] = make_float4(lo[0], lo[1], lo[2], 0.f);
        box[2 * blk + 1] = make_float4(hi[0], hi[1], hi[2], 0.f);
    }
}

// Per-block fits of a potential p and of p - |x|^2 (the two forms of the
// bound), written as fit[2*blk] and fit[2*blk+1].  Row side (KEY = false):
// (u, c) with c the maximum of value_i - u.x_i.  Key side (KEY = true):
// (v, G) with G the base-2 log-sum of lw2_j + (value_j - v.y_j) c_bias.
template <int GS, bool KEY>
__global__ __launch_bounds__(256) void block_fit_kernel(const float* __restrict__ ops,
                                                        const float* __restrict__ centre, int d,
                                                        int64_t n, const float* __restrict__ pot,
                                                        const float* __restrict__ lw2,
                                                        float c_bias, int nb,
                                                        float4* __restrict__ fit) {
    __shared__ float red[64];
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int blk = (int)(i / GS);
    const bool valid = i < n;
    float x[3] = {0.f, 0.f, 0.f};
    float p = 0.f;
    if (valid) {
        load_point(ops, centre, d, i, x);
        p = pot[i];
    }
    const float q = p - (x[0] * x[0] + x[1] * x[1] + x[2] * x[2]);  // p - |x|^2
    float s1[6] = {valid ? x[0] : 0.f, valid ? x[1] : 0.f, valid ? x[2] : 0.f,
                   valid ? p : 0.f,    valid ? q : 0.f,    valid ? 1.f : 0.f};
    group_sum<GS>(s1, red);
    const float inv = s1[5] > 0.f ? 1.f / s1[5] : 0.f;
    const float cx = x[0] - s1[0] * inv, cy = x[1] - s1[1] * inv, cz = x[2] - s1[2] * inv;
    const float cp = p - s1[3] * inv, cq = q - s1[4] * inv;
    float S[12] = {cx * cx, cy * cy, cz * cz, cx * cy, cx * cz, cy * cz,
                   cx * cp, cy * cp, cz * cp, cx * cq, cy * cq, cz * cq};
    if (!valid)
#pragma unroll
        for (int k = 0; k < 12; ++k) S[k] = 0.f;
    group_sum<GS>(S, red);
#pragma unroll
    for (int form = 0; form < 2; ++form) {
        const float Sf[9] = {S[0], S[1], S[2], S[3], S[4], S[5], S[6 + 3 * form],
                             S[7 + 3 * form], S[8 + 3 * form]};
        float u[3];
        solve_slope(Sf, u);
        const float r = (form ? q : p) - (u[0] * x[0] + u[1] * x[1] + u[2] * x[2]);
        float out;
        if constexpr (!KEY) {
            out = group_max<GS>(valid ? r : -INFINITY, red);
        } else {
            const float z = valid ? fmaf(r, c_bias, lw2[i]) : -INFINITY;
            const float M = group_max<GS>(z, red);
            float e[1] = {M > -INFINITY ? ex2(z - M) : 0.f};
            group_sum<GS>(e, red);
            out = M > -INFINITY ? M + lg2(e[0]) : -INFINITY;
        }
        if ((threadIdx.x % GS) == 0 && blk < nb)
            fit[2 * blk + form] = make_float4(u[0], u[1], u[2], out);
    }
}

// Box and key-side fits (both forms, as block_fit_kernel with KEY = true) of
// chunks of kChunkKeys consecutive keys, one workgroup per chunk, each thread
// taking every 256th key of it: cbox[2C], cbox[2C+1] = lo, hi; cfit[2C + form].
__global__ __launch_bounds__(256) void chunk_fit_kernel(const float* __restrict__ ops,
                                                        const float* __restrict__ centre, int d,
                                                        int64_t n, const float* __restrict__ pot,
                                                        const float* __restrict__ lw2,
                                                        float c_bias, float4* __restrict__ cbox,
                                                        float4* __restrict__ cfit) {
    __shared__ float red[64];
    constexpr int PER = kChunkKeys / 256;
    const int C = blockIdx.x;
    const int64_t i0 = (int64_t)C * kChunkKeys + threadIdx.x;
    float s1[6] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float lo[3] = {INFINITY, INFINITY, INFINITY}, hi[3] = {-INFINITY, -INFINITY, -INFINITY};
    auto point = [&](int k, float (&x)[3], float& p, float& q) {
        const int64_t i = i0 + (int64_t)k * 256;
        if (i >= n) return false;
        load_point(ops, centre, d, i, x);
        p = pot[i];
        q = p - (x[0] * x[0] + x[1] * x[1] + x[2] * x[2]);
        return true;
    };
    for (int k = 0; k < PER; ++k) {
        float x[3], p, q;
        if (!point(k, x, p, q)) break;
        s1[0] += x[0];
        s1[1] += x[1];
        s1[2] += x[2];
        s1[3] += p;
        s1[4] += q;
        s1[5] += 1.f;
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            lo[c] = fminf(lo[c], x[c]);
            hi[c] = fmaxf(hi[c], x[c]);
        }
    }
    group_sum<256>(s1, red);
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        hi[c] = group_max<256>(hi[c], red);
        lo[c] = -group_max<256>(-lo[c], red);
    }
    const float inv = s1[5] > 0.f ? 1.f / s1[5] : 0.f;
    float S[12] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < PER; ++k) {
        float x[3], p, q;
        if (!point(k, x, p, q)) break;
        const float cx = x[0] - s1[0] * inv, cy = x[1] - s1[1] * inv, cz = x[2] - s1[2] * inv;
        const float cp = p - s1[3] * inv, cq = q - s1[4] * inv;
        S[0] += cx * cx;
        S[1] += cy * cy;
        S[2] += cz * cz;
        S[3] += cx * cy;
        S[4] += cx * cz;
        S[5] += cy * cz;
        S[6] += cx * cp;
        S[7] += cy * cp;
        S[8] += cz * cp;
        S[9] += cx * cq;
        S[10] += cy * cq;
        S[11] += cz * cq;
    }
    group_sum<256>(S, red);
    if (threadIdx.x == 0) {
        cbox[2 * C] = make_float4(lo[0], lo[1], lo[2], 0.f);
        cbox[2 * C + 1] = make_float4(hi[0], hi[1], hi[2], 0.f);
    }
#pragma unroll
    for (int form = 0; form < 2; ++form) {
        const float Sf[9] = {S[0], S[1], S[2], S[3], S[4], S[5], S[6 + 3 * form],
                             S[7 + 3 * form], S[8 + 3 * form]};
        float u[3];
        solve_slope(Sf, u);
        // base-2 log-sum of lw2_j + (value_j - u.y_j) c_bias over the chunk
        float M = -INFINITY;
        for (int k = 0; k < PER; ++k) {
            float x[3], p, q;
            if (!point(k, x, p, q)) break;
            const float r = (form ? q : p) - (u[0] * x[0] + u[1] * x[1] + u[2] * x[2]);
            M = fmaxf(M, fmaf(r, c_bias, lw2[i0 + (int64_t)k * 256]));
        }
        M = group_max<256>(M, red);
        float e[1] = {0.f};
        if (M > -INFINITY)
            for (int k = 0; k < PER; ++k) {
                float x[3], p, q;
                if (!point(k, x, p, q)) break;
                const float r = (form ? q : p) - (u[0] * x[0] + u[1] * x[1] + u[2] * x[2]);
                e[0] += ex2(fmaf(r, c_bias, lw2[i0 + (int64_t)k * 256]) - M);
            }
        group_sum<256>(e, red);
        if (threadIdx.x == 0)
            cfit[2 * C + form] =
                make_float4(u[0], u[1], u[2], M > -INFINITY ? M + lg2(e[0]) : -INFINITY);
    }
}

// ---------------------------------------------------------------- screening

__device__ __forceinline__ float hq(float u, float v, float x, float y) {
    const float t = x - y;
    return fmaf(u, x, fmaf(v, y, -t * t));
}

// max of u x + v y - (x - y)^2 over x in [a1, b1], y in [a2, b2]
__device__ __forceinline__ float hmax1(float u, float v, float a1, float b1, float a2, float b2) {
    const float y1 = fminf(fmaxf(fmaf(0.5f, v, a1), a2), b2);
    const float y2 = fminf(fmaxf(fmaf(0.5f, v, b1), a2), b2);
    const float x3 = fminf(fmaxf(fmaf(0.5f, u, a2), a1), b1);
    const float x4 = fminf(fmaxf(fmaf(0.5f, u, b2), a1), b1);
    return fmaxf(fmaxf(hq(u, v, a1, y1), hq(u, v, b1, y2)),
                 fmaxf(hq(u, v, x3, a2), hq(u, v, x4, b2)));
}

// max of u x + v y + 2 x y over x in [a1, b1], y in [a2, b2] (a corner)
__device__ __forceinline__ float bmax1(float u, float v, float a1, float b1, float a2, float b2) {
    auto h = [&](float x, float y) { return fmaf(u, x, fmaf(v, y, 2.f * x * y)); };
    return fmaxf(fmaxf(h(a1, a2), h(a1, b2)), fmaxf(h(b1, a2), h(b1, b2)));
}

struct ScreenArgs {
    const float4* rbox;  // [nbR][2]
    const float4* rfit;  // [nbR][2]: (u, c) of f and of f - |x|^2
    const float4* kbox;  // [nbK][2]
    const float4* kfit;  // [nbK][2]: (v, G) of g and of g - |y|^2
    int nbR, nbK;
    float c_bias;
    float thr2;          // log2(delta / nbK), -inf for delta = 0
    float margin_rel;    // rounding margin per unit of c_bias * magnitude
    float mag;           // magnitude of the coordinates (1 + max |coordinate|^2 sum)
    int* list;           // [nbR][cap]
    int* count;          // [nbR]
    int* best;           // [nbR]: the key block of largest bound
    // origin of each row block for the streaming kernel's shifted fp16
    // operands: org[2I] = (O - row cloud centre, format flag), org[2I+1] =
    // (O - key cloud centre, 0), O the centre of the row block's box
    const float* cR;
    const float* cK;
    int d;
    float4* org;
    int cap;
    int sentinel;
    // two-level form (nbC > 0): boxes and fits of chunks of 256 key blocks
    const float4* cbox;  // [nbC][2]
    const float4* cfit;  // [nbC][2]
    int nbC;
};

__global__ __launch_bounds__(256) void screen_kernel(ScreenArgs a) {
    __shared__ int wcnt[4];
    __shared__ float bred[4];
    __shared__ int jred[4];
    __shared__ unsigned char clive[kMaxChunks];
    const int I = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const float4 rlo = a.rbox[2 * I], rhi = a.rbox[2 * I + 1];
    const float4 rf = a.rfit[2 * I], rq = a.rfit[2 * I + 1];
    const float base2 = rf.w * a.c_bias, baseq = rq.w * a.c_bias;
    const float thr =
        a.thr2 - a.margin_rel * a.c_bias * (a.mag + fmaxf(fabsf(rf.w), fabsf(rq.w)));
    int* __restrict__ out = a.list + (int64_t)I * a.cap;
    const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    int count = 0;
    float best = -INFINITY;
    int bestJ = 0;
    // box centre O and the largest |y - O| over the kept key blocks' boxes
    const float O[3] = {0.5f * (rlo.x + rhi.x), 0.5f * (rlo.y + rhi.y), 0.5f * (rlo.z + rhi.z)};
    auto reach = [&](int J) {
        const float4 klo = a.kbox[2 * J], khi = a.kbox[2 * J + 1];
        return fmaxf(fmaxf(fmaxf(fabsf(klo.x - O[0]), fabsf(khi.x - O[0])),
                           fmaxf(fabsf(klo.y - O[1]), fabsf(khi.y - O[1]))),
                     fmaxf(fabsf(klo.z - O[2]), fabsf(khi.z - O[2])));
    };
    // log2 bound of the mass a key group (box klo..khi, fits kf, kq) can hold
    // in any row of this row block
    auto bound = [&](float4 kf, float4 kq, float4 klo, float4 khi) {
        const float H = hmax1(rf.x, kf.x, rlo.x, rhi.x, klo.x, khi.x) +
                        hmax1(rf.y, kf.y, rlo.y, rhi.y, klo.y, khi.y) +
                        hmax1(rf.z, kf.z, rlo.z, rhi.z, klo.z, khi.z);
        const float H2 = bmax1(rq.x, kq.x, rlo.x, rhi.x, klo.x, khi.x) +
                         bmax1(rq.y, kq.y, rlo.y, rhi.y, klo.y, khi.y) +
                         bmax1(rq.z, kq.z, rlo.z, rhi.z, klo.z, khi.z);
        return fminf(fmaf(H, a.c_bias, base2) + kf.w, fmaf(H2, a.c_bias, baseq) + kq.w);
    };
    if (a.nbC > 0) {
        // first level: a chunk below the threshold holds less than that mass in
        // every one of its blocks; the chunk of largest bound is always opened
        float cb = -INFINITY;
        int cj = 0;
        for (int C = tid; C < a.nbC; C += 256) {
            const float beta =
                bound(a.cfit[2 * C], a.cfit[2 * C + 1], a.cbox[2 * C], a.cbox[2 * C + 1]);
            clive[C] = beta >= thr ? 1 : 0;
            if (beta > cb) {
                cb = beta;
                cj = C;
            }
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const float b2 = __shfl_xor(cb, o, 64);
            const int j2 = __shfl_xor(cj, o, 64);
            if (b2 > cb || (b2 == cb && j2 < cj)) {
                cb = b2;
                cj = j2;
            }
        }
        if (lane == 0) {
            bred[w] = cb;
            jred[w] = cj;
        }
        __syncthreads();
        if (tid == 0) {
            float bb = bred[0];
            int jj = jred[0];
            for (int q = 1; q < 4; ++q)
                if (bred[q] > bb || (bred[q] == bb && jred[q] < jj)) {
                    bb = bred[q];
                    jj = jred[q];
                }
            clive[jj] = 1;
        }
        __syncthreads();
    }
    float wmax = 0.f;
    for (int J0 = 0; J0 < a.nbK; J0 += 256) {
        if (a.nbC > 0 && !clive[J0 >> 8]) continue;  // uniform: J0 is the same in every thread
        const int J = J0 + tid;
        bool keep = false;
        if (J < a.nbK) {
            const float beta =
                bound(a.kfit[2 * J], a.kfit[2 * J + 1], a.kbox[2 * J], a.kbox[2 * J + 1]);
            keep = beta >= thr;
            if (beta > best) {
                best = beta;
                bestJ = J;
            }
        }
        const uint64_t m = __builtin_amdgcn_ballot_w64(keep);
        if (lane == 0) wcnt[w] = (int)__popcll(m);
        __syncthreads();
        int pre = 0, tot = 0;
        for (int q = 0; q < 4; ++q) {
            if (q < w) pre += wcnt[q];
            tot += wcnt[q];
        }
        if (keep) {
            out[count + pre + (int)__popcll(m & lt)] = J;
            wmax = fmaxf(wmax, reach(J));
        }
        count += tot;
        __syncthreads();
    }
    {
        // the block of largest bound (first on ties): where the streaming
        // kernel takes its rows' starting reference; kept if nothing else is
        float b = best;
        int j = bestJ;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const float b2 = __shfl_xor(b, o, 64);
            const int j2 = __shfl_xor(j, o, 64);
            if (b2 > b || (b2 == b && j2 < j)) {
                b = b2;
                j = j2;
            }
        }
        if (lane == 0) {
            bred[w] = b;
            jred[w] = j;
        }
        __syncthreads();
        if (tid == 0) {
            float bb = bred[0];
            int jj = jred[0];
            for (int q = 1; q < 4; ++q)
                if (bred[q] > bb || (bred[q] == bb && jred[q] < jj)) {
                    bb = bred[q];
                    jj = jred[q];
                }
            a.best[I] = jj;
            if (count == 0) {
                out[0] = jj;
                wmax = reach(jj);
            }
        }
        if (count == 0) count = 1;
    }
    // origin and fp16 format flag of the row block (the same bounds as the
    // dense kernel's fp16 format, on the shifted magnitudes: rows within the
    // box's half extents of O, kept keys within wmax)
    {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) wmax = fmaxf(wmax, __shfl_xor(wmax, o, 64));
        __syncthreads();
        if (lane == 0) bred[w] = wmax;
        __syncthreads();
        if (tid == 0) {
            const float wm = fmaxf(fmaxf(bred[0], bred[1]), fmaxf(bred[2], bred[3]));
            const float cs = 2.f * a.c_bias;
            float half = 0.f, l1o = 0.f, ox[3] = {0.f, 0.f, 0.f}, oy[3] = {0.f, 0.f, 0.f};
            const float hx[3] = {0.5f * (rhi.x - rlo.x), 0.5f * (rhi.y - rlo.y),
                                 0.5f * (rhi.z - rlo.z)};
            for (int c = 0; c < a.d; ++c) {
                ox[c] = O[c] - a.cR[c];
                oy[c] = O[c] - a.cK[c];
                half += hx[c];
                l1o += fabsf(ox[c]);
            }
            const bool ok = cs * half * wm <= 500.f && cs * l1o * wm <= 16384.f &&
                            cs * half <= 16384.f && wm <= 16384.f;
            a.org[2 * I] = make_float4(ox[0], ox[1], ox[2], ok ? 1.f : 0.f);
            a.org[2 * I + 1] = make_float4(oy[0], oy[1], oy[2], 0.f);
        }
    }
    const int padded = (count + 15) / 16 * 16;
    for (int k = count + tid; k < padded; k += 256) out[k] = a.sentinel;
    if (tid == 0) a.count[I] = count;
}

// Work plan of the retained-block pass: row block I's list of tiles_I =
// ceil(count_I / 16) tiles is dealt to S_I = min(smax, ceil(tiles_I / T))
// workgroups, T = ceil(total tiles / target), so that long and short lists
// take about the same time; map[2k], map[2k+1] = (row block, split) of
// workgroup k, total[0] = sum of S_I (<= nbR + target).  One workgroup.
__global__ __launch_bounds__(1024) void split_plan_kernel(const int* __restrict__ count, int nbR,
                                                          int target, int smax,
                                                          int* __restrict__ nsplit,
                                                          int* __restrict__ map,
                                                          int* __restrict__ total) {
    __shared__ int red[16];
    __shared__ int carry_s;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    // total tiles (fixed-order sum)
    int t = 0;
    for (int I = tid; I < nbR; I += 1024) t += (count[I] + 15) / 16;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) t += __shfl_xor(t, o, 64);
    if (lane == 0) red[wid] = t;
    if (tid == 0) carry_s = 0;
    __syncthreads();
    int all = 0;
    for (int w = 0; w < 16; ++w) all += red[w];
    const int T = max(1, (all + target - 1) / target);
    __syncthreads();
    for (int base = 0; base < nbR; base += 1024) {
        const int I = base + tid;
        const int tiles = I < nbR ? (count[I] + 15) / 16 : 0;
        const int S = I < nbR ? min(smax, max(1, (tiles + T - 1) / T)) : 0;
        int inc = S;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(inc, o, 64);
            if (lane >= o) inc += v;
        }
        if (lane == 63) red[wid] = inc;
        __syncthreads();
        int pre = 0, tot = 0;
        for (int w = 0; w < 16; ++w) {
            if (w < wid) pre += red[w];
            tot += red[w];
        }
        const int off = carry_s + pre + inc - S;
        if (I < nbR) {
            nsplit[I] = S;
            for (int q = 0; q < S; ++q) {
                map[2 * (off + q)] = I;
                map[2 * (off + q) + 1] = q;
            }
        }
        __syncthreads();
        if (tid == 0) carry_s += tot;
        __syncthreads();
    }
    if (tid == 0) total[0] = carry_s;
}

// ---------------------------------------------------------------- coarse stage
// "FlashSinkhorn 2" explainer, solving at a coarse resolution first: cells
// are runs of `cell` consecutive (Morton-ordered) points; a cell's centroid
// is the weighted mean of its points (fp64 sums, fixed order), its weight
// their sum.
__global__ __launch_bounds__(256) void centroid_kernel(const float* __restrict__ P,
                                                       const float* __restrict__ w, int64_t n,
                                                       int d, int cell, int64_t nc,
                                                       float* __restrict__ C,
                                                       float* __restrict__ W) {
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k >= nc) return;
    const int64_t i0 = k * cell, i1 = min(n, i0 + cell);
    double sw = 0.0, sx[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int64_t i = i0; i < i1; ++i) {
        const double wi = w[i];
        sw += wi;
        for (int c = 0; c < d; ++c) sx[c] += wi * (double)P[i * d + c];
    }
    W[k] = (float)sw;
    for (int c = 0; c < d; ++c) C[k * d + c] = (float)(sx[c] / sw);
}

// The lift: every point takes its cell's potential.
__global__ __launch_bounds__(256) void lift_kernel(const float* __restrict__ F, int64_t n,
                                                   int cell, float* __restrict__ f) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) f[i] = F[i / cell];
}

// The sampled marginal check (trusting the lifted solution): for sampled
// point q of one side (one workgroup each), its exact marginal under (f, g)
// against every point of the other side, as the pair (|r_q - w_q|, w_q):
//   r_q / w_q = 2^(pot_q c_bias + LSE2_j (log2 w'_j + (pot'_j - C_qj) c_bias)).
__global__ __launch_bounds__(256) void sampled_marginal_kernel(
    const float* __restrict__ P, const float* __restrict__ w, const float* __restrict__ pot,
    int64_t np_, const int32_t* __restrict__ idx, const float* __restrict__ Q,
    const float* __restrict__ wq, const float* __restrict__ potq, int64_t mq, int d,
    float c_bias, float2* __restrict__ out) {
    __shared__ float smax[256], ssum[256];
    // (an index outside [0, np_) is clamped into it)
    const int64_t i = min((int64_t)max(idx[blockIdx.x], 0), np_ - 1);
    float x[8];
    for (int c = 0; c < 8; ++c) x[c] = c < d ? P[i * d + c] : 0.f;
    float M = -INFINITY, S = 0.f;
    for (int64_t j = threadIdx.x; j < mq; j += 256) {
        float cost = 0.f;
        for (int c = 0; c < d; ++c) {
            const float t = x[c] - Q[j * d + c];
            cost = fmaf(t, t, cost);
        }
        const float z = __log2f(wq[j]) + (potq[j] - cost) * c_bias;
        lse_merge(M, S, z, 1.f);
    }
    smax[threadIdx.x] = M;
    ssum[threadIdx.x] = S;
    __syncthreads();
    for (int o = 128; o >= 1; o >>= 1) {
        if ((int)threadIdx.x < o) {
            float m1 = smax[threadIdx.x], s1 = ssum[threadIdx.x];
            lse_merge(m1, s1, smax[threadIdx.x + o], ssum[threadIdx.x + o]);
            smax[threadIdx.x] = m1;
            ssum[threadIdx.x] = s1;
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const float z = pot[i] * c_bias + smax[0] + lg2(ssum[0]);
        out[blockIdx.x] = make_float2(w[i] * fabsf(ex2(z) - 1.f), w[i]);
    }
}

// (sum |r - w|) / (sum w) over the samples of each side, fixed order.
__global__ __launch_bounds__(256) void sampled_reduce_kernel(const float2* __restrict__ part,
                                                             int nrows, int ncols,
                                                             float* __restrict__ out2) {
    __shared__ double se[256], sw[256];
    for (int side = 0; side < 2; ++side) {
        const int base = side ? nrows : 0, cnt = side ? ncols : nrows;
        double e = 0.0, ww = 0.0;
        for (int k = threadIdx.x; k < cnt; k += 256) {
            e += part[base + k].x;
            ww += part[base + k].y;
        }
        se[threadIdx.x] = e;
        sw[threadIdx.x] = ww;
        __syncthreads();
        for (int o = 128; o >= 1; o >>= 1) {
            if ((int)threadIdx.x < o) {
                se[threadIdx.x] += se[threadIdx.x + o];
                sw[threadIdx.x] += sw[threadIdx.x + o];
            }
            __syncthreads();
        }
        if (threadIdx.x == 0) out2[side] = sw[0] > 0.0 ? (float)(se[0] / sw[0]) : 0.f;
        __syncthreads();
    }
}

// ---------------------------------------------------------------- transport
// The transport U = P.V over the kept blocks of the f-side screening (the
// skipped mass of every row is below delta * a_i, so each component of U
// moves by less than delta a_i max |V|): one workgroup per 256-row block,
// one row per thread, stages of 8 listed key blocks (256 keys) through LDS;
//   log2 P_ij = lw2_i + (f_i - A_i) c_bias + c_score x~_i.y~_j + lw2_j + (g_j - B_j) c_bias.
struct BsTransportArgs {
    const float* rows;  // x~ [n_pad][4]
    const float* row_nrm;
    const float* row_lw2;
    const float* row_pot;
    const float* row_w;
    const float* keys;  // y~ [m_pad][4]
    const float* key_nrm;
    const float* key_lw2;
    const float* key_pot;
    const float* V;  // [m][dv] (unused by the gradient form)
    int dv, n_rows, n_keys;
    float c_bias, c_score;
    int divide;
    const int* list;
    const int* count;
    int cap;
    const float* cR;  // centres of the row and key clouds (gradient form)
    const float* cK;
    float* U;  // [n][dv]
};

// Row block I (one workgroup, a row per thread) against its kept key blocks,
// eight at a time (256 keys staged in LDS).  Transport form: U_i = sum_j
// P_ij V_j (/ a_i).  Gradient form (GRAD, dv = d <= 3): with the centred
// coordinates x' = x - cR, y' = y - cK it accumulates S_i = sum_j P_ij y'_j and
// r_i = sum_j P_ij, and writes 2 (r_i (x'_i + cR - cK) - S_i), which is
// 2 sum_j P_ij (x_i - y_j).
template <int DV, bool GRAD>
__global__ __launch_bounds__(256) void bs_transport_kernel(BsTransportArgs a) {
    __shared__ float4 ky[256];
    __shared__ float kv[GRAD ? 1 : 256][DV];
    const int I = blockIdx.x, tid = threadIdx.x;
    const int64_t i = (int64_t)I * 256 + tid;
    const bool live = i < a.n_rows;
    float xr[3] = {0.f, 0.f, 0.f};
    float rt = -INFINITY;
    if (live) {
        const float4 r = *(const float4*)(a.rows + i * 4);
        xr[0] = r.x;
        xr[1] = r.y;
        xr[2] = r.z;
        rt = fmaf(a.row_pot[i] - a.row_nrm[i], a.c_bias, a.row_lw2[i]);
    }
    const float x0 = xr[0] * a.c_score, x1 = xr[1] * a.c_score, x2 = xr[2] * a.c_score;
    float acc[DV];
#pragma unroll
    for (int c = 0; c < DV; ++c) acc[c] = 0.f;
    const int cnt = a.count[I];
    const int* __restrict__ lst = a.list + (int64_t)I * a.cap;
    for (int k0 = 0; k0 < cnt; k0 += 8) {
        // 8 listed blocks (entries past the count are the -inf sentinel)
        __syncthreads();
        {
            const int J = lst[k0 + (tid >> 5)];
            const int64_t j = (int64_t)J * 32 + (tid & 31);
            if (j < a.n_keys) {
                const float4 y = *(const float4*)(a.keys + j * 4);
                ky[tid] = make_float4(y.x, y.y, y.z,
                                      fmaf(a.key_pot[j] - a.key_nrm[j], a.c_bias, a.key_lw2[j]));
            } else {
                ky[tid] = make_float4(0.f, 0.f, 0.f, -INFINITY);
            }
            if constexpr (!GRAD)
                for (int c = 0; c < DV; ++c)
                    kv[tid][c] = (j < a.n_keys && c < a.dv) ? a.V[j * a.dv + c] : 0.f;
        }
        __syncthreads();
        for (int kk = 0; kk < 256; ++kk) {
            const float4 y = ky[kk];
            const float z = fmaf(x0, y.x, fmaf(x1, y.y, fmaf(x2, y.z, y.w + rt)));
            const float p = ex2(z);
            if constexpr (GRAD) {
                acc[0] = fmaf(p, y.x, acc[0]);
                acc[1] = fmaf(p, y.y, acc[1]);
                acc[2] = fmaf(p, y.z, acc[2]);
                acc[3] += p;
            } else {
#pragma unroll
                for (int c = 0; c < DV; ++c) acc[c] = fmaf(p, kv[kk][c], acc[c]);
            }
        }
    }
    if (!live) return;
    if constexpr (GRAD) {
        for (int c = 0; c < a.dv; ++c)
            a.U[i * a.dv + c] = 2.f * (acc[3] * (xr[c] + (a.cR[c] - a.cK[c])) - acc[c]);
    } else {
        const float inv = a.divide ? 1.f / a.row_w[i] : 1.f;
        for (int c = 0; c < a.dv; ++c) a.U[i * a.dv + c] = acc[c] * inv;
    }
}

}  // namespace

// ---------------------------------------------------------------- launchers

hipError_t launch_bs_transport(const float* rows, const float* row_nrm, const float* row_lw2,
                               const float* row_pot, const float* row_w, int n_rows,
                               const float* keys, const float* key_nrm, const float* key_lw2,
                               const float* key_pot, int n_keys, const float* V, int dv,
                               float c_bias, float c_score, int divide, const int* list,
                               const int* count, int cap, int nbR, const float* cR,
                               const float* cK, float* U, hipStream_t s) {
    BsTransportArgs a{rows, row_nrm, row_lw2, row_pot, row_w, keys, key_nrm, key_lw2, key_pot,
                      V, dv, n_rows, n_keys, c_bias, c_score, divide, list, count, cap, cR, cK, U};
    if (!V) {  // the gradient form
        if (dv > 3 || !cR || !cK) return hipErrorInvalidValue;
        bs_transport_kernel<4, true><<<nbR, 256, 0, s>>>(a);
    } else if (dv <= 4) {
        bs_transport_kernel<4, false><<<nbR, 256, 0, s>>>(a);
    } else if (dv <= 8) {
        bs_transport_kernel<8, false><<<nbR, 256, 0, s>>>(a);
    } else if (dv <= 16) {
        bs_transport_kernel<16, false><<<nbR, 256, 0, s>>>(a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_centroids(const float* P, const float* w, int64_t n, int d, int cell,
                            float* C, float* W, hipStream_t s) {
    const int64_t nc = (n + cell - 1) / cell;
    centroid_kernel<<<(unsigned)((nc + 255) / 256), 256, 0, s>>>(P, w, n, d, cell, nc, C, W);
    return hipGetLastError();
}

hipError_t launch_lift(const float* F, int64_t n, int cell, float* f, hipStream_t s) {
    lift_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(F, n, cell, f);
    return hipGetLastError();
}

hipError_t launch_sampled_marginal(const float* X, const float* Y, const float* a,
                                   const float* b, int64_t n, int64_t m, int d, float c_bias,
                                   const float* f, const float* g, const int32_t* rows,
                                   int nrows, const int32_t* cols, int ncols, float2* part,
                                   float* out2, hipStream_t s) {
    hipError_t e;
    if (nrows > 0) {
        sampled_marginal_kernel<<<nrows, 256, 0, s>>>(X, a, f, n, rows, Y, b, g, m, d, c_bias,
                                                      part);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (ncols > 0) {
        sampled_marginal_kernel<<<ncols, 256, 0, s>>>(Y, b, g, m, cols, X, a, f, n, d, c_bias,
                                                      part + nrows);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    sampled_reduce_kernel<<<1, 256, 0, s>>>(part, nrows, ncols, out2);
    return hipGetLastError();
}

hipError_t launch_split_plan(const int* count, int nbR, int target, int smax, int* nsplit,
                             int* map, int* total, hipStream_t s) {
    split_plan_kernel<<<1, 1024, 0, s>>>(count, nbR, target, smax, nsplit, map, total);
    return hipGetLastError();
}

int morton_bits(int d) { return 30 / d; }

size_t morton_workspace_bytes(int64_t n) {
    const int64_t tiles = (n + kSortTile - 1) / kSortTile;
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    return 4 * up(4 * (size_t)n) + up(4 * 256 * (size_t)tiles) + 2 * up(4 * 8 * kBoxParts) +
           2 * up(4 * 8);
}

hipError_t launch_morton_sort(const float* X, const float* w, int64_t n, int d, float* Xo,
                              float* wo, int32_t* perm, void* ws, hipStream_t s) {
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    const int64_t tiles = (n + kSortTile - 1) / kSortTile;
    char* p = (char*)ws;
    uint32_t* k0 = (uint32_t*)p;
    p += up(4 * (size_t)n);
    uint32_t* k1 = (uint32_t*)p;
    p += up(4 * (size_t)n);
    int32_t* v0 = (int32_t*)p;
    p += up(4 * (size_t)n);
    int32_t* v1 = (int32_t*)p;
    p += up(4 * (size_t)n);
    uint32_t* hist = (uint32_t*)p;
    p += up(4 * 256 * (size_t)tiles);
    float* pmin = (float*)p;
    p += up(4 * 8 * kBoxParts);
    float* pmax = (float*)p;
    p += up(4 * 8 * kBoxParts);
    float* lo = (float*)p;
    p += up(4 * 8);
    float* scale = (float*)p;
    hipError_t e;
    const int bits = morton_bits(d);
    const int parts = (int)std::min<int64_t>(kBoxParts, (n + 255) / 256);
    mbox_partial_kernel<<<parts, 256, 0, s>>>(X, n, d, pmin, pmax);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    mbox_final_kernel<<<1, 64, 0, s>>>(pmin, pmax, parts, d, bits, lo, scale);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const unsigned g = (unsigned)((n + 255) / 256);
    mcode_kernel<<<g, 256, 0, s>>>(X, n, d, bits, lo, scale, k0, v0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int passes = (bits * d + 7) / 8;
    const int64_t hlen = 256 * tiles;
    for (int q = 0; q < passes; ++q) {
        const uint32_t* kin = q & 1 ? k1 : k0;
        const int32_t* vin = q & 1 ? v1 : v0;
        uint32_t* kout = q & 1 ? k0 : k1;
        int32_t* vout = q & 1 ? v0 : v1;
        rs_hist_kernel<<<(unsigned)tiles, kSortThreads, 0, s>>>(kin, n, 8 * q, (int)tiles, hist);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        rs_scan_kernel<<<1, 1024, 0, s>>>(hist, hlen);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        rs_scatter_kernel<<<(unsigned)tiles, kSortThreads, 0, s>>>(kin, vin, kout, vout, n, 8 * q,
                                                                   (int)tiles, hist);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int32_t* sorted = passes & 1 ? v1 : v0;
    mgather_kernel<<<g, 256, 0, s>>>(X, w, n, d, sorted, Xo, wo, perm);
    return hipGetLastError();
}

hipError_t launch_unpermute(const float* src, const int32_t* perm, int64_t n, int width,
                            float* dst, hipStream_t s) {
    const int64_t total = n * width;
    unpermute_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(src, perm, n, width, dst);
    return hipGetLastError();
}

hipError_t launch_block_boxes(const float* ops, const float* centre, int d, int64_t n, int gs,
                              float4* box, hipStream_t s) {
    const unsigned g = (unsigned)((n + 255) / 256);
    const int nb = (int)((n + gs - 1) / gs);
    if (gs == 32)
        block_box_kernel<32><<<g, 256, 0, s>>>(ops, centre, d, n, nb, box);
    else if (gs == 256)
        block_box_kernel<256><<<g, 256, 0, s>>>(ops, centre, d, n, nb, box);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_block_fit(const float* ops, const float* centre, int d, int64_t n, int gs,
                            bool key, const float* pot, const float* lw2, float c_bias,
                            float4* fit, hipStream_t s) {
    const unsigned g = (unsigned)((n + 255) / 256);
    const int nb = (int)((n + gs - 1) / gs);
    if (gs == 32 && key)
        block_fit_kernel<32, true><<<g, 256, 0, s>>>(ops, centre, d, n, pot, lw2, c_bias, nb, fit);
    else if (gs == 256 && !key)
        block_fit_kernel<256, false><<<g, 256, 0, s>>>(ops, centre, d, n, pot, lw2, c_bias, nb,
                                                       fit);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_chunk_fit(const float* ops, const float* centre, int d, int64_t n,
                            const float* pot, const float* lw2, float c_bias, float4* cbox,
                            float4* cfit, hipStream_t s) {
    const int64_t nbC = (n + kChunkKeys - 1) / kChunkKeys;
    if (nbC < 1 || nbC > kMaxChunks) return hipErrorInvalidValue;
    chunk_fit_kernel<<<(unsigned)nbC, 256, 0, s>>>(ops, centre, d, n, pot, lw2, c_bias, cbox,
                                                   cfit);
    return hipGetLastError();
}

hipError_t launch_screen(const float4* rbox, const float4* rfit, int nbR, const float4* kbox,
                         const float4* kfit, int nbK, float c_bias, float thr2, float mag,
                         int* list, int* count, int* best, const float* cR, const float* cK,
                         int d, float4* org, int cap, int sentinel, const float4* cbox,
                         const float4* cfit, int nbC, hipStream_t s) {
    if (nbC < 0 || nbC > kMaxChunks || (nbC > 0 && nbC != (nbK + 255) / 256))
        return hipErrorInvalidValue;
    ScreenArgs a;
    a.rbox = rbox;
    a.rfit = rfit;
    a.kbox = kbox;
    a.kfit = kfit;
    a.nbR = nbR;
    a.nbK = nbK;
    a.c_bias = c_bias;
    a.thr2 = thr2;
    a.margin_rel = 0x1p-16f;
    a.mag = mag;
    a.list = list;
    a.count = count;
    a.best = best;
    a.cR = cR;
    a.cK = cK;
    a.d = d;
    a.org = org;
    a.cap = cap;
    a.sentinel = sentinel;
    a.cbox = cbox;
    a.cfit = cfit;
    a.nbC = nbC;
    screen_kernel<<<nbR, 256, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace fs
