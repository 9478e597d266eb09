// fs_prep.hip -- one-time preparation of a problem: common shift of both
// clouds, conversion to the score element type, squared norms, log-weights
// and input validation.
//
// The pages ("FlashSinkhorn" explainer, "Method" part 1) call the bias terms
// of the attention form "precomputed log-weight biases"; this pass computes
// everything of that kind that does not depend on the potentials, once.
//
// Common shift.  C_ij = |x_i - y_j|^2 is unchanged when both clouds move by
// the same vector, so f and g are unchanged too.  Moving both clouds to the
// midpoint of their joint bounding box keeps |x|^2 and |y|^2 small, which
// bounds the cancellation of the expanded form |x|^2 + |y|^2 - 2 x.y that the
// streaming kernels evaluate in fp32.  Min and max are exact, so the shift
// (min + max) * 0.5 is reproducible bit for bit by any IEEE implementation.
#include "fs_device.hpp"
#include "fs_internal.h"

namespace fs {

namespace {

enum : int { FLAG_NONFINITE_POINT = 1, FLAG_BAD_WEIGHT = 2, FLAG_RANGE = 4 };

__global__ void zero_flag_kernel(int* flag) {
    if (threadIdx.x == 0) flag[0] = 0;
}

// Per-coordinate min/max of one row chunk.  grid = (ceil(d/256), parts).
__global__ __launch_bounds__(256) void bbox_partial_kernel(const float* __restrict__ P,
                                                           int64_t n, int d, int parts,
                                                           float* __restrict__ pmin,
                                                           float* __restrict__ pmax) {
    const int k = blockIdx.x * 256 + threadIdx.x;
    if (k >= d) return;
    const int part = blockIdx.y;
    const int64_t chunk = (n + parts - 1) / parts;
    const int64_t r0 = part * chunk;
    const int64_t r1 = r0 + chunk < n ? r0 + chunk : n;
    float mn = INFINITY, mx = -INFINITY;
    for (int64_t r = r0; r < r1; ++r) {
        const float v = P[r * d + k];
        mn = fminf(mn, v);
        mx = fmaxf(mx, v);
    }
    pmin[(int64_t)part * d + k] = mn;
    pmax[(int64_t)part * d + k] = mx;
}

__global__ __launch_bounds__(256) void bbox_final_kernel(const float* __restrict__ pmin,
                                                         const float* __restrict__ pmax,
                                                         int total_parts, int d,
                                                         float* __restrict__ shift) {
    const int k = blockIdx.x * 256 + threadIdx.x;
    if (k >= d) return;
    float mn = INFINITY, mx = -INFINITY;
    for (int p = 0; p < total_parts; ++p) {
        mn = fminf(mn, pmin[(int64_t)p * d + k]);
        mx = fmaxf(mx, pmax[(int64_t)p * d + k]);
    }
    // Midpoint of the joint bounding box; 0 if the coordinate is all-NaN
    // (the convert pass reports the NaN).
    float s = (mn + mx) * 0.5f;
    if (!(s == s) || s == INFINITY || s == -INFINITY) s = 0.f;
    shift[k] = s;
}

template <typename T>
__device__ __forceinline__ T to_elem(float v);
template <>
__device__ __forceinline__ float to_elem<float>(float v) { return v; }
template <>
__device__ __forceinline__ __bf16 to_elem<__bf16>(float v) { return (__bf16)v; }  // RNE
template <>
__device__ __forceinline__ _Float16 to_elem<_Float16>(float v) { return (_Float16)v; }  // RNE

// One wave per row: ops[i][k] = T(P[i][k] - shift[k]) (0 in the padding),
// nrm[i] = sum_k float(ops[i][k])^2 in a fixed order.
template <typename T>
__global__ __launch_bounds__(256) void convert_kernel(const float* __restrict__ P, int64_t n,
                                                      int64_t n_pad, int d, int dp,
                                                      const float* __restrict__ shift,
                                                      T* __restrict__ ops,
                                                      float* __restrict__ nrm,
                                                      int* __restrict__ flag) {
    const int lane = threadIdx.x & 63;
    const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= n_pad) return;
    float acc = 0.f;
    int bad = 0;
    for (int k = lane; k < dp; k += 64) {
        T t = to_elem<T>(0.f);
        if (i < n && k < d) {
            const float v = P[i * d + k];
            if (!(fabsf(v) <= 3.402823466e38f)) bad |= FLAG_NONFINITE_POINT;
            t = to_elem<T>(v - shift[k]);
            const float tf = (float)t;
            if (!(fabsf(tf) <= 3.402823466e38f)) bad |= FLAG_RANGE;
            acc += tf * tf;
        }
        ops[i * dp + k] = t;
    }
    acc = wave_sum(acc);
    if (i < n && lane == 0) nrm[i] = acc;
    if (bad) atomicOr(flag, bad);
}

__global__ __launch_bounds__(256) void weights_kernel(const float* __restrict__ w, int64_t n,
                                                      float* __restrict__ lw2,
                                                      float* __restrict__ wcopy,
                                                      float* __restrict__ pot,
                                                      int* __restrict__ flag) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const float v = w[i];
    // Weights must be normal positive floats (log2 of a subnormal would lose
    // accuracy on the transcendental unit).
    if (!(v >= 1.17549435e-38f && v <= 3.402823466e38f)) atomicOr(flag, FLAG_BAD_WEIGHT);
    lw2[i] = lg2(v);
    wcopy[i] = v;
    if (pot) pot[i] = 0.f;
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

hipError_t launch_bbox(const float* X, int64_t n, const float* Y, int64_t m, int d,
                       float* part_min, float* part_max, int parts, float* shift,
                       hipStream_t s) {
    const dim3 grid((d + 255) / 256, parts);
    bbox_partial_kernel<<<grid, 256, 0, s>>>(X, n, d, parts, part_min, part_max);
    bbox_partial_kernel<<<grid, 256, 0, s>>>(Y, m, d, parts, part_min + (int64_t)parts * d,
                                             part_max + (int64_t)parts * d);
    bbox_final_kernel<<<(d + 255) / 256, 256, 0, s>>>(part_min, part_max, 2 * parts, d, shift);
    return hipGetLastError();
}

hipError_t launch_convert(const float* P, int64_t n, int64_t n_pad, int d, int dp, int path,
                          const float* shift, void* ops, float* nrm, int* flag,
                          hipStream_t s) {
    const int64_t blocks = (n_pad + 3) / 4;
    switch (path) {
        case PATH_VALU:
        case PATH_SMALL:
        case PATH_MFMA_F32:
            convert_kernel<float><<<blocks, 256, 0, s>>>(P, n, n_pad, d, dp, shift,
                                                         (float*)ops, nrm, flag);
            break;
        case PATH_MFMA_BF16:
            convert_kernel<__bf16><<<blocks, 256, 0, s>>>(P, n, n_pad, d, dp, shift,
                                                          (__bf16*)ops, nrm, flag);
            break;
        case PATH_MFMA_F16:
            convert_kernel<_Float16><<<blocks, 256, 0, s>>>(P, n, n_pad, d, dp, shift,
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

hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    fill_kernel<<<(n + 255) / 256, 256, 0, s>>>(p, n, v);
    return hipGetLastError();
}

}  // namespace fs
