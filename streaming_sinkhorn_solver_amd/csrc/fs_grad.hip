// fs_grad.hip -- the pieces of the gradient of the entropic OT dual and of its
// value that are not a transport application.
//
// The pages ("FlashSinkhorn" explainer, "Method" part 3) compute gradients
// with respect to the points by the same streaming traversal as the transport
// application.  For squared-Euclidean cost, with the plan P of (f, g),
//   d/dx_i of the dual = sum_j P_ij 2 (x_i - y_j)
//                      = 2 ( r_i (x_i - c) - sum_j P_ij (y_j - c) ),
// r_i = sum_j P_ij, for any vector c; c is the other cloud's centre, so the
// transported values are as small as that cloud's spread.  The transport
// kernels deliver sum_j P_ij (y_j - c); this pass forms the rest.
#include "fs_device.hpp"
#include "fs_internal.h"

namespace fs {

namespace {

// One wave per row.  With p_i = P[i] (or P[i] rscale_i, unit length, for the
// cosine cost) and r_i = 2^(L_i + (pot_i - nrm_i) c_bias) w_i (the row sums of
// the plan: the same factor the transport applies to row i):
//   G_i <- 2 (r_i (p_i - c) - G_i),
// the gradient with respect to p_i; for the cosine cost it is then taken back
// through p_i = x_i / |x_i|, whose Jacobian is (I - p_i p_i^T) / |x_i|:
//   G_i <- rscale_i (G_i - p_i (p_i . G_i)).
__global__ __launch_bounds__(256) void grad_finish_kernel(const float* __restrict__ P,
                                                          const float* __restrict__ rscale,
                                                          const float* __restrict__ c,
                                                          const float* __restrict__ lse2,
                                                          const float* __restrict__ pot,
                                                          const float* __restrict__ nrm,
                                                          const float* __restrict__ w,
                                                          float c_bias, int64_t n, int d,
                                                          float* __restrict__ G) {
    const int lane = threadIdx.x & 63;
    const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= n) return;
    const float r = ex2(lse2[i] + (pot[i] - nrm[i]) * c_bias) * w[i];
    const float s = rscale ? rscale[i] : 1.f;
    float dot = 0.f;
    for (int k = lane; k < d; k += 64) {
        const int64_t idx = i * d + k;
        const float p = P[idx] * s;
        const float gk = 2.f * fmaf(r, p - c[k], -G[idx]);
        G[idx] = gk;
        dot = fmaf(p, gk, dot);
    }
    if (!rscale) return;
    dot = wave_sum(dot);
    for (int k = lane; k < d; k += 64) {
        const int64_t idx = i * d + k;
        G[idx] = s * fmaf(-P[idx] * s, dot, G[idx]);
    }
}

// out[0] = sum_i a_i f_i + sum_j b_j g_j, accumulated in fp64 in a fixed
// order (one workgroup: strided per-thread sums, then a tree).
__global__ __launch_bounds__(1024) void dual_value_kernel(const float* __restrict__ a,
                                                          const float* __restrict__ f,
                                                          int64_t n,
                                                          const float* __restrict__ b,
                                                          const float* __restrict__ g,
                                                          int64_t m, double* __restrict__ out) {
    __shared__ double red[1024];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += 1024) s += (double)a[i] * (double)f[i];
    for (int64_t j = threadIdx.x; j < m; j += 1024) s += (double)b[j] * (double)g[j];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int o = 512; o >= 1; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[0] = red[0];
}

}  // namespace

hipError_t launch_grad_finish(const float* P, const float* rscale, const float* c,
                              const float* lse2, const float* pot, const float* nrm,
                              const float* w, float c_bias, int64_t n, int d, float* G,
                              hipStream_t s) {
    if (n <= 0) return hipSuccess;
    grad_finish_kernel<<<(unsigned)((n + 3) / 4), 256, 0, s>>>(P, rscale, c, lse2, pot, nrm, w,
                                                               c_bias, n, d, G);
    return hipGetLastError();
}

hipError_t launch_dual_value(const float* a, const float* f, int64_t n, const float* b,
                             const float* g, int64_t m, double* out, hipStream_t s) {
    dual_value_kernel<<<1, 1024, 0, s>>>(a, f, n, b, g, m, out);
    return hipGetLastError();
}

}  // namespace fs
