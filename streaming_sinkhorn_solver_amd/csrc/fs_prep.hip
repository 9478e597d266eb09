// fs_prep.hip -- one-time preparation of a problem: centring of each cloud,
// conversion to the score element type, the per-point terms of the expanded
// cost, log-weights and input validation.
//
// The pages ("FlashSinkhorn" explainer, "Method" part 1) call the bias terms
// of the attention form "precomputed log-weight biases"; this pass computes
// everything of that kind that does not depend on the potentials, once.
//
// Centring.  With nu the centre of X, mu the centre of Y, x' = x - nu,
// y' = y - mu and delta = nu - mu, the cost splits exactly as
//   |x - y|^2 = A(x) + B(y) - 2 x'.y',
//   A(x) = |x - mu|^2 - |delta|^2 / 2,   B(y) = |y - nu|^2 - |delta|^2 / 2
// (expand |x' - y' + delta|^2).  The streaming kernels contract x'.y' on the
// matrix cores and take A, B (fp32, from the unrounded points) as row and key
// terms.  Centring each cloud on its own keeps the contracted operands as
// small as the clouds' spreads allow, so the rounding of x', y' to bf16/fp16
// and the fp32 accumulation move the score by as little as possible; a shift
// common to both clouds would leave the offset between them (a cluster of Y
// displaced from X, say) in the operands, where it multiplies the rounding
// error.  Each centre is the midpoint of its cloud's bounding box: min and max
// are exact, so (min + max) * 0.5 is reproducible bit for bit by any IEEE
// implementation.
#include "fs_device.hpp"
#include "fs_internal.h"

namespace fs {

namespace {

enum : int { FLAG_NONFINITE_POINT = 1, FLAG_BAD_WEIGHT = 2, FLAG_RANGE = 4, FLAG_ZERO_NORM = 8 };

__global__ void zero_flag_kernel(int* flag) {
    if (threadIdx.x == 0) flag[0] = 0;
}

// Per-coordinate min/max of one row chunk.  grid = (ceil(d/64), parts):
// 64 coordinates per workgroup, its four waves taking every fourth row of
// the chunk (each wave reads 64 consecutive floats of a row), then the four
// partial results combined through LDS.  rscale (nullable): the points are
// P[r] * rscale[r] (unit rows for the cosine cost).
__global__ __launch_bounds__(256) void bbox_partial_kernel(const float* __restrict__ P,
                                                           const float* __restrict__ rscale,
                                                           int64_t n, int d, int parts,
                                                           float* __restrict__ pmin,
                                                           float* __restrict__ pmax) {
    __shared__ float smn[4][64], smx[4][64];
    const int c = threadIdx.x & 63, rg = threadIdx.x >> 6;
    const int k = blockIdx.x * 64 + c;
    const int part = blockIdx.y;
    const int64_t chunk = (n + parts - 1) / parts;
    const int64_t r0 = part * chunk;
    const int64_t r1 = r0 + chunk < n ? r0 + chunk : n;
    float mn = INFINITY, mx = -INFINITY;
    if (k < d) {
#pragma unroll 8
        for (int64_t r = r0 + rg; r < r1; r += 4) {
            const float v = rscale ? P[r * d + k] * rscale[r] : P[r * d + k];
            mn = fminf(mn, v);
            mx = fmaxf(mx, v);
        }
    }
    smn[rg][c] = mn;
    smx[rg][c] = mx;
    __syncthreads();
    if (rg == 0 && k < d) {
        mn = fminf(fminf(smn[0][c], smn[1][c]), fminf(smn[2][c], smn[3][c]));
        mx = fmaxf(fmaxf(smx[0][c], smx[1][c]), fmaxf(smx[2][c], smx[3][c]));
        pmin[(int64_t)part * d + k] = mn;
        pmax[(int64_t)part * d + k] = mx;
    }
}

// Centre of one cloud from its parts' boxes.  grid = (ceil(d/256), 2): y-block
// 0 reduces X's parts into centre[0..d), 1 Y's parts into centre[d..2d).
__global__ __launch_bounds__(256) void bbox_final_kernel(const float* __restrict__ pmin,
                                                         const float* __restrict__ pmax,
                                                         int parts, int d,
                                                         float* __restrict__ centre) {
    const int k = blockIdx.x * 256 + threadIdx.x;
    if (k >= d) return;
    const int64_t base = (int64_t)blockIdx.y * parts * d;
    float mn = INFINITY, mx = -INFINITY;
    for (int p = 0; p < parts; ++p) {
        mn = fminf(mn, pmin[base + (int64_t)p * d + k]);
        mx = fmaxf(mx, pmax[base + (int64_t)p * d + k]);
    }
    // Midpoint of the bounding box; 0 if the coordinate is all-NaN or
    // unbounded (the convert pass reports the NaN / Inf).
    float c = (mn + mx) * 0.5f;
    if (!(fabsf(c) <= 3.402823466e38f)) c = 0.f;
    centre[(int64_t)blockIdx.y * d + k] = c;
}

template <typename T>
__device__ __forceinline__ T to_elem(float v);
template <>
__device__ __forceinline__ float to_elem<float>(float v) { return v; }
template <>
__device__ __forceinline__ __bf16 to_elem<__bf16>(float v) { return (__bf16)v; }  // RNE
template <>
__device__ __forceinline__ _Float16 to_elem<_Float16>(float v) { return (_Float16)v; }  // RNE

// Row i by one wave: ops[i][k] = T(P[i][k] - own[k]) (0 in the padding) and
// the row's cost term |P[i] - oth|^2 - |own - oth|^2 / 2 in fp32, summed in a
// fixed order (own: this cloud's centre, oth: the other cloud's).  Returns
// the lane's last converted value (for dp <= 64 lane k holds element k).
template <typename T>
__device__ __forceinline__ float convert_row(const float* __restrict__ P,
                                            const float* __restrict__ rscale, int64_t i,
                                            int64_t n, int d, int dp,
                                            const float* __restrict__ own,
                                            const float* __restrict__ oth, T* __restrict__ ops,
                                            float* __restrict__ nrm, int* __restrict__ flag) {
    const int lane = threadIdx.x & 63;
    float acc = 0.f, off = 0.f, last = 0.f;
    int bad = 0;
    for (int k = lane; k < dp; k += 64) {
        T t = to_elem<T>(0.f);
        if (i < n && k < d) {
            const float v = rscale ? P[i * d + k] * rscale[i] : P[i * d + k];
            if (!(fabsf(v) <= 3.402823466e38f)) bad |= FLAG_NONFINITE_POINT;
            t = to_elem<T>(v - own[k]);
            if (!(fabsf((float)t) <= 3.402823466e38f)) bad |= FLAG_RANGE;
            const float u = v - oth[k], c = own[k] - oth[k];
            acc = fmaf(u, u, acc);
            off = fmaf(c, c, off);
        }
        ops[i * dp + k] = t;
        last = (float)t;
    }
    acc = wave_sum(acc);
    off = wave_sum(off);
    if (i < n && lane == 0) nrm[i] = fmaf(off, -0.5f, acc);
    if (bad) atomicOr(flag, bad);
    return last;
}

// One wave per row (4 rows per workgroup).
template <typename T>
__global__ __launch_bounds__(256) void convert_kernel(const float* __restrict__ P,
                                                      const float* __restrict__ rscale, int64_t n,
                                                      int64_t n_pad, int d, int dp,
                                                      const float* __restrict__ own,
                                                      const float* __restrict__ oth,
                                                      T* __restrict__ ops,
                                                      float* __restrict__ nrm,
                                                      int* __restrict__ flag) {
    const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= n_pad) return;
    convert_row<T>(P, rscale, i, n, d, dp, own, oth, ops, nrm, flag);
}

// One wave per row: inv[i] = 1 / |P[i]| (cosine cost: the points are
// normalised to unit length, where |x^ - y^|^2 = 2 - 2 cos(x, y)).  A zero or
// non-finite row is flagged.
__global__ __launch_bounds__(256) void inv_norm_kernel(const float* __restrict__ P, int64_t n,
                                                       int d, float* __restrict__ inv,
                                                       int* __restrict__ flag) {
    const int lane = threadIdx.x & 63;
    const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= n) return;
    float s = 0.f;
    for (int k = lane; k < d; k += 64) {
        const float v = P[i * d + k];
        s = fmaf(v, v, s);
    }
    s = wave_sum(s);
    if (lane == 0) {
        const bool ok = s > 0.f && s <= 3.402823466e38f;
        inv[i] = ok ? 1.0f / sqrtf(s) : 0.f;
        if (!ok) atomicOr(flag, FLAG_ZERO_NORM);
    }
}

__device__ __forceinline__ void weight_point(const float* __restrict__ w, int64_t i,
                                             float* __restrict__ lw2, float* __restrict__ wcopy,
                                             float* __restrict__ pot, int* __restrict__ flag) {
    const float v = w[i];
    // Weights must be normal positive floats (log2 of a subnormal would lose
    // accuracy on the transcendental unit).
    if (!(v >= 1.17549435e-38f && v <= 3.402823466e38f)) atomicOr(flag, FLAG_BAD_WEIGHT);
    lw2[i] = lg2(v);
    wcopy[i] = v;
    if (pot) pot[i] = 0.f;
}

__global__ __launch_bounds__(256) void weights_kernel(const float* __restrict__ w, int64_t n,
                                                      float* __restrict__ lw2,
                                                      float* __restrict__ wcopy,
                                                      float* __restrict__ pot,
                                                      int* __restrict__ flag) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    weight_point(w, i, lw2, wcopy, pot, flag);
}

// ---- small problems: the whole preparation in two launches
// (the same arithmetic as the kernels above, so the results are the same
// bits; only the launches are merged)

// Workgroup c (0: X, 1: Y) forms its cloud's centre from the exact
// per-coordinate min and max over all its rows (d <= 8); workgroup 0 also
// clears the flag word and the two L1 maxima.
__global__ __launch_bounds__(256) void prep_small_centre_kernel(SmallPrepArgs a) {
    __shared__ float red[2][8][256];
    const int c = blockIdx.x;
    const float* __restrict__ P = c ? a.Y : a.X;
    const int64_t n = c ? a.m : a.n;
    const int d = a.d;
    if (c == 0 && threadIdx.x == 0) {
        a.flag[0] = 0;
        if (a.xl1) *a.xl1 = 0.f;
        if (a.yl1) *a.yl1 = 0.f;
    }
    float mn[8], mx[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        mn[k] = INFINITY;
        mx[k] = -INFINITY;
    }
    for (int64_t r = threadIdx.x; r < n; r += 256)
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (k < d) {
                const float v = P[r * d + k];
                mn[k] = fminf(mn[k], v);
                mx[k] = fmaxf(mx[k], v);
            }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        red[0][k][threadIdx.x] = mn[k];
        red[1][k][threadIdx.x] = mx[k];
    }
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
        if (threadIdx.x < w)
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                red[0][k][threadIdx.x] = fminf(red[0][k][threadIdx.x], red[0][k][threadIdx.x + w]);
                red[1][k][threadIdx.x] = fmaxf(red[1][k][threadIdx.x], red[1][k][threadIdx.x + w]);
            }
        __syncthreads();
    }
    if (threadIdx.x < d) {
        // midpoint of the bounding box; 0 if the coordinate is all-NaN or
        // unbounded (the row pass reports the NaN / Inf)
        float ctr = (red[0][threadIdx.x][0] + red[1][threadIdx.x][0]) * 0.5f;
        if (!(fabsf(ctr) <= 3.402823466e38f)) ctr = 0.f;
        a.centre[c * d + threadIdx.x] = ctr;
    }
}

// One wave per padded row of either cloud (rows of X first): the fp32
// operand row and cost term (convert_row), the row's L1 norm into the
// cloud's maximum when asked (as row_l1max_kernel), and the point's weight
// terms (weight_point).
__global__ __launch_bounds__(256) void prep_small_rows_kernel(SmallPrepArgs a) {
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= a.n_pad + a.m_pad) return;
    const bool xs = t < a.n_pad;
    const int64_t i = xs ? t : t - a.n_pad;
    const int64_t n = xs ? a.n : a.m;
    const float* own = a.centre + (xs ? 0 : a.d);
    const float* oth = a.centre + (xs ? a.d : 0);
    float* ops = xs ? a.xops : a.yops;
    const float tv = convert_row<float>(xs ? a.X : a.Y, nullptr, i, n, a.d, a.dp, own, oth, ops,
                                        xs ? a.xn : a.yn, a.flag);
    float* l1 = xs ? a.xl1 : a.yl1;
    // the row's L1 norm summed in coordinate order, from the lanes' values
    float v = 0.f;
    for (int k = 0; k < a.d; ++k) v += fabsf(__shfl(tv, k, 64));
    if ((threadIdx.x & 63) == 0 && i < n) {
        if (l1 && v > 0.f) atomicMax((unsigned*)l1, __float_as_uint(v));
        weight_point(xs ? a.a : a.b, i, xs ? a.xlw : a.ylw, xs ? a.xw : a.yw, xs ? a.f : a.g,
                     a.flag);
    }
}

__global__ __launch_bounds__(256) void fill_kernel(float* __restrict__ p, int64_t n, float v) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_zero_flag(int* flag, hipStream_t s) {
    zero_flag_kernel<<<1, 64, 0, s>>>(flag);
    return hipGetLastError();
}

hipError_t launch_inv_norm(const float* P, int64_t n, int d, float* inv, int* flag,
                           hipStream_t s) {
    inv_norm_kernel<<<(unsigned)((n + 3) / 4), 256, 0, s>>>(P, n, d, inv, flag);
    return hipGetLastError();
}

hipError_t launch_bbox(const float* X, const float* xscale, int64_t n, const float* Y,
                       const float* yscale, int64_t m, int d, float* part_min, float* part_max,
                       int parts, float* centres, hipStream_t s) {
    const dim3 grid((d + 63) / 64, parts);
    bbox_partial_kernel<<<grid, 256, 0, s>>>(X, xscale, n, d, parts, part_min, part_max);
    bbox_partial_kernel<<<grid, 256, 0, s>>>(Y, yscale, m, d, parts,
                                             part_min + (int64_t)parts * d,
                                             part_max + (int64_t)parts * d);
    bbox_final_kernel<<<dim3((d + 255) / 256, 2), 256, 0, s>>>(part_min, part_max, parts, d,
                                                               centres);
    return hipGetLastError();
}

hipError_t launch_convert(const float* P, const float* rscale, int64_t n, int64_t n_pad, int d,
                          int dp, int path, const float* own, const float* oth, void* ops,
                          float* nrm, int* flag, hipStream_t s) {
    const int64_t blocks = (n_pad + 3) / 4;
    switch (path) {
        case PATH_VALU:
        case PATH_SMALL:
        case PATH_MFMA_F32:
            convert_kernel<float><<<blocks, 256, 0, s>>>(P, rscale, n, n_pad, d, dp, own, oth,
                                                         (float*)ops, nrm, flag);
            break;
        case PATH_MFMA_BF16:
            convert_kernel<__bf16><<<blocks, 256, 0, s>>>(P, rscale, n, n_pad, d, dp, own, oth,
                                                          (__bf16*)ops, nrm, flag);
            break;
        case PATH_MFMA_F16:
            convert_kernel<_Float16><<<blocks, 256, 0, s>>>(P, rscale, n, n_pad, d, dp, own, oth,
                                                            (_Float16*)ops, nrm, flag);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_weights(const float* w, int64_t n, float* lw2, float* wcopy, float* pot,
                          int* flag, hipStream_t s) {
    weights_kernel<<<(n + 255) / 256, 256, 0, s>>>(w, n, lw2, wcopy, pot, flag);
    return hipGetLastError();
}

hipError_t launch_prep_small(const SmallPrepArgs& a, hipStream_t s) {
    if (a.d < 1 || a.d > 8 || a.n < 1 || a.m < 1) return hipErrorInvalidValue;
    prep_small_centre_kernel<<<2, 256, 0, s>>>(a);
    prep_small_rows_kernel<<<(unsigned)((a.n_pad + a.m_pad + 3) / 4), 256, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    fill_kernel<<<(n + 255) / 256, 256, 0, s>>>(p, n, v);
    return hipGetLastError();
}

}  // namespace fs
