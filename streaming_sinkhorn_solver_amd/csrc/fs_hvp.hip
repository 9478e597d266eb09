// fs_hvp.hip -- the pointwise and reduction steps of the streaming
// Hessian-vector product of the entropic OT loss with respect to X.
//
// The pages ("FlashSinkhorn" explainer, "Method" part 3) evaluate HVPs as
// sequences of transport-vector and transport-matrix products.  The product
// here differentiates the gradient G_i = 2 sum_j P_ij (x_i - y_j) along X + tV
// with both marginals of P held fixed (implicit differentiation through the
// Sinkhorn fixed point):
//   dC_ij = 2 (x_i - y_j).v_i,   dP_ij = P_ij (df_i + dg_j - dC_ij) / eps,
//   r_i df_i + (P dg)_i = u_i := sum_j P_ij dC_ij,
//   (P^T df)_j + c_j dg_j = w_j := sum_i P_ij dC_ij,
// solved for dg on the Schur complement K = diag(c) - P^T diag(1/r) P (CG
// preconditioned by diag(c), on the complement of the constant vector, K's
// null space), df = (u - P dg)/r.
// With all points centred on the same vector mu (x~, y~) and s_i = x~_i.v_i,
// PY_i = sum_j P_ij y~_j, M_i = sum_j P_ij (y~_j.v_i) y~_j:
//   u_i = 2 (r_i s_i - PY_i.v_i),   w_j = 2 ((P^T s)_j - y~_j.(P^T V)_j),
//   (H V)_i = 2 r_i v_i - (2/eps) (df_i PY_i + (P (dg y~))_i - 2 s_i PY_i + 2 M_i).
// The transports run on the streaming kernels; these kernels form their
// inputs and combine their outputs.  Reductions for the CG scalars are
// single-workgroup and fixed-order (deterministic).
#include "fs_device.hpp"
#include "fs_internal.h"

namespace fs {

namespace {

// r_i = 2^(lse2_i + (pot_i - nrm_i) c_bias) w_i: the plan's row sums (the
// row factor of the transport).
__global__ __launch_bounds__(256) void marginal_kernel(const float* __restrict__ lse2,
                                                       const float* __restrict__ pot,
                                                       const float* __restrict__ nrm,
                                                       const float* __restrict__ w, float c_bias,
                                                       int64_t n, float* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) out[i] = ex2(lse2[i] + (pot[i] - nrm[i]) * c_bias) * w[i];
}

// One wave per row i: s_i = (x_i - mu).v_i, u_i = 2 (r_i s_i - PY_i.v_i);
// W_i = [v_i | s_i | u_i / r_i] (d + 2 columns), the column transport's input.
__global__ __launch_bounds__(256) void hvp_rows_kernel(const float* __restrict__ X,
                                                       const float* __restrict__ V,
                                                       const float* __restrict__ mu,
                                                       const float* __restrict__ PY,
                                                       const float* __restrict__ r, int64_t n,
                                                       int d, float* __restrict__ u,
                                                       float* __restrict__ W) {
    const int lane = threadIdx.x & 63;
    const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= n) return;
    float s = 0.f, t = 0.f;
    for (int k = lane; k < d; k += 64) {
        const float v = V[i * d + k];
        s = fmaf(X[i * d + k] - mu[k], v, s);
        t = fmaf(PY[i * d + k], v, t);
        W[i * (d + 2) + k] = v;
    }
    s = wave_sum(s);
    t = wave_sum(t);
    if (lane == 0) {
        const float ui = 2.f * fmaf(r[i], s, -t);
        u[i] = ui;
        W[i * (d + 2) + d] = s;
        W[i * (d + 2) + d + 1] = r[i] > 0.f ? ui / r[i] : 0.f;
    }
}

// One wave per column j: rhs_j = 2 (PtW_j[d] - (y_j - mu).PtW_j[0:d]) - PtW_j[d+1]
// (w_j minus (P^T (u/r))_j).
__global__ __launch_bounds__(256) void hvp_cols_kernel(const float* __restrict__ Y,
                                                       const float* __restrict__ mu,
                                                       const float* __restrict__ PtW, int64_t m,
                                                       int d, float* __restrict__ rhs) {
    const int lane = threadIdx.x & 63;
    const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (j >= m) return;
    float t = 0.f;
    for (int k = lane; k < d; k += 64) t = fmaf(Y[j * d + k] - mu[k], PtW[j * (d + 2) + k], t);
    t = wave_sum(t);
    if (lane == 0)
        rhs[j] = 2.f * (PtW[j * (d + 2) + d] - t) - PtW[j * (d + 2) + d + 1];
}

// out[0] = sum_k x_k y_k, out[1] = sum_k x_k, out[2] = sum_k x_k^2 (one
// workgroup, fixed order, fp64)
__global__ __launch_bounds__(1024) void dot_kernel(const float* __restrict__ x,
                                                   const float* __restrict__ y, int64_t len,
                                                   double* __restrict__ out) {
    __shared__ double red[3][1024];
    double s = 0.0, t = 0.0, q = 0.0;
    for (int64_t k = threadIdx.x; k < len; k += 1024) {
        const double xv = (double)x[k];
        s += xv * (double)y[k];
        t += xv;
        q += xv * xv;
    }
    red[0][threadIdx.x] = s;
    red[1][threadIdx.x] = t;
    red[2][threadIdx.x] = q;
    __syncthreads();
    for (int o = 512; o >= 1; o >>= 1) {
        if ((int)threadIdx.x < o) {
            red[0][threadIdx.x] += red[0][threadIdx.x + o];
            red[1][threadIdx.x] += red[1][threadIdx.x + o];
            red[2][threadIdx.x] += red[2][threadIdx.x + o];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        out[0] = red[0][0];
        out[1] = red[1][0];
        out[2] = red[2][0];
    }
}

// y <- alpha x + beta y - shift (shift: nullable device scalar, subtracted
// as shift[0] * shift_scale)
__global__ __launch_bounds__(256) void axpby_kernel(float alpha, const float* __restrict__ x,
                                                    float beta, float* __restrict__ y, int64_t len,
                                                    const double* __restrict__ shift,
                                                    double shift_scale) {
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k >= len) return;
    float v = fmaf(alpha, x[k], beta * y[k]);
    if (shift) v -= (float)(shift[0] * shift_scale);
    y[k] = v;
}

// out_k = a_k * x_k - y_k  (a nullable: 1), or with `divide`, out_k = x_k / a_k
__global__ __launch_bounds__(256) void scale_sub_kernel(const float* __restrict__ a,
                                                        const float* __restrict__ x,
                                                        const float* __restrict__ y, int64_t len,
                                                        int divide, float* __restrict__ out) {
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k >= len) return;
    if (divide)
        out[k] = a[k] > 0.f ? x[k] / a[k] : 0.f;
    else
        out[k] = (a ? a[k] : 1.f) * x[k] - (y ? y[k] : 0.f);
}

// V2_j = [dg_j (y_j - mu) | dg_j]  (m x (d+1))
__global__ __launch_bounds__(256) void hvp_dgy_kernel(const float* __restrict__ Y,
                                                      const float* __restrict__ mu,
                                                      const float* __restrict__ dg, int64_t m,
                                                      int d, float* __restrict__ V2) {
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = m * (d + 1);
    if (k >= total) return;
    const int64_t j = k / (d + 1);
    const int c = (int)(k - j * (d + 1));
    V2[k] = c < d ? dg[j] * (Y[j * d + c] - mu[c]) : dg[j];
}

// Second-moment columns q in [q0, q0 + w): V3_j[q - q0] = y~_j[q / d] y~_j[q % d]
__global__ __launch_bounds__(256) void hvp_outer_kernel(const float* __restrict__ Y,
                                                        const float* __restrict__ mu, int64_t m,
                                                        int d, int64_t q0, int w,
                                                        float* __restrict__ V3) {
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k >= m * w) return;
    const int64_t j = k / w;
    const int64_t q = q0 + (k - j * w);
    const int a = (int)(q / d), b = (int)(q % d);
    V3[k] = (Y[j * d + a] - mu[a]) * (Y[j * d + b] - mu[b]);
}

// M_i[q / d] += T3_i[q - q0] v_i[q % d] for the chunk's columns (one thread
// per (row, output coordinate); the chunk covers whole or partial rows of
// the d x d moment, summed in column order)
__global__ __launch_bounds__(256) void hvp_moment_kernel(const float* __restrict__ T3,
                                                         const float* __restrict__ V, int64_t n,
                                                         int d, int64_t q0, int w,
                                                         float* __restrict__ M) {
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k >= n * d) return;
    const int64_t i = k / d;
    const int a = (int)(k - i * d);
    // columns of this chunk with first index a: q in [max(q0, a d), min(q0 + w, (a+1) d))
    const int64_t lo = q0 > (int64_t)a * d ? q0 : (int64_t)a * d;
    const int64_t hi = q0 + w < (int64_t)(a + 1) * d ? q0 + w : (int64_t)(a + 1) * d;
    float acc = M[k];
    for (int64_t q = lo; q < hi; ++q) acc = fmaf(T3[i * w + (q - q0)], V[i * d + (q % d)], acc);
    M[k] = acc;
}

// Direction rows in the score type for the second-moment kernel: row i of
// [n_pad][dp] is v_i sigma_i (zero-padded to dp; zero rows past n), sigma_i
// the power of two that brings max_k |v_ik| into [0.5, 1); inv_sigma_i = 1 /
// sigma_i undoes it exactly.  One wave per row.
template <class T>
__global__ __launch_bounds__(256) void hvp_vconv_kernel(const float* __restrict__ V, int64_t n,
                                                        int64_t n_pad, int d, int dp,
                                                        T* __restrict__ out,
                                                        float* __restrict__ inv_sigma) {
    const int lane = threadIdx.x & 63;
    const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= n_pad) return;
    float amax = 0.f;
    if (i < n)
        for (int k = lane; k < d; k += 64) amax = fmaxf(amax, fabsf(V[i * d + k]));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    int e = 0;
    if (amax > 0.f) frexpf(amax, &e);  // amax in [2^(e-1), 2^e)
    const float sigma = ldexpf(1.f, -e);
    for (int k = lane; k < dp; k += 64)
        out[i * dp + k] = (T)(i < n && k < d ? V[i * d + k] * sigma : 0.f);
    if (lane == 0 && i < n) inv_sigma[i] = ldexpf(1.f, e);
}

// df_i = (u_i - T_i[d]) / r_i;
// HV_i = 2 r_i v_i - (2/eps) (df_i PY_i + T_i[0:d] - 2 s_i PY_i + 2 M_i),
// s_i = W_i[d].
__global__ __launch_bounds__(256) void hvp_final_kernel(const float* __restrict__ V,
                                                        const float* __restrict__ r,
                                                        const float* __restrict__ u,
                                                        const float* __restrict__ W,
                                                        const float* __restrict__ PY,
                                                        const float* __restrict__ T,
                                                        const float* __restrict__ M,
                                                        const float* __restrict__ m_scale,
                                                        int64_t n, int d, float inv_eps,
                                                        float* __restrict__ HV) {
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k >= n * d) return;
    const int64_t i = k / d;
    const int c = (int)(k - i * d);
    const float ri = r[i];
    const float df = ri > 0.f ? (u[i] - T[i * (d + 1) + d]) / ri : 0.f;
    const float s = W[i * (d + 2) + d];
    const float py = PY[k];
    const float mk = m_scale ? M[k] * m_scale[i] : M[k];
    const float br = fmaf(df, py, T[i * (d + 1) + c]) + 2.f * fmaf(-s, py, mk);
    HV[k] = 2.f * fmaf(ri, V[k], -inv_eps * br);
}

unsigned blocks_for(int64_t count, int per) { return (unsigned)((count + per - 1) / per); }

}  // namespace

hipError_t launch_marginal(const float* lse2, const float* pot, const float* nrm, const float* w,
                           float c_bias, int64_t n, float* out, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    marginal_kernel<<<blocks_for(n, 256), 256, 0, s>>>(lse2, pot, nrm, w, c_bias, n, out);
    return hipGetLastError();
}

hipError_t launch_hvp_rows(const float* X, const float* V, const float* mu, const float* PY,
                           const float* r, int64_t n, int d, float* u, float* W, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hvp_rows_kernel<<<blocks_for(n, 4), 256, 0, s>>>(X, V, mu, PY, r, n, d, u, W);
    return hipGetLastError();
}

hipError_t launch_hvp_cols(const float* Y, const float* mu, const float* PtW, int64_t m, int d,
                           float* rhs, hipStream_t s) {
    if (m <= 0) return hipSuccess;
    hvp_cols_kernel<<<blocks_for(m, 4), 256, 0, s>>>(Y, mu, PtW, m, d, rhs);
    return hipGetLastError();
}

hipError_t launch_dot(const float* x, const float* y, int64_t len, double* out, hipStream_t s) {
    dot_kernel<<<1, 1024, 0, s>>>(x, y, len, out);
    return hipGetLastError();
}

hipError_t launch_axpby(float alpha, const float* x, float beta, float* y, int64_t len,
                        const double* shift, double shift_scale, hipStream_t s) {
    if (len <= 0) return hipSuccess;
    axpby_kernel<<<blocks_for(len, 256), 256, 0, s>>>(alpha, x, beta, y, len, shift, shift_scale);
    return hipGetLastError();
}

hipError_t launch_scale_sub(const float* a, const float* x, const float* y, int64_t len,
                            int divide, float* out, hipStream_t s) {
    if (len <= 0) return hipSuccess;
    scale_sub_kernel<<<blocks_for(len, 256), 256, 0, s>>>(a, x, y, len, divide, out);
    return hipGetLastError();
}

hipError_t launch_hvp_dgy(const float* Y, const float* mu, const float* dg, int64_t m, int d,
                          float* V2, hipStream_t s) {
    if (m <= 0) return hipSuccess;
    hvp_dgy_kernel<<<blocks_for(m * (d + 1), 256), 256, 0, s>>>(Y, mu, dg, m, d, V2);
    return hipGetLastError();
}

hipError_t launch_hvp_outer(const float* Y, const float* mu, int64_t m, int d, int64_t q0, int w,
                            float* V3, hipStream_t s) {
    if (m <= 0) return hipSuccess;
    hvp_outer_kernel<<<blocks_for(m * w, 256), 256, 0, s>>>(Y, mu, m, d, q0, w, V3);
    return hipGetLastError();
}

hipError_t launch_hvp_moment(const float* T3, const float* V, int64_t n, int d, int64_t q0, int w,
                             float* M, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hvp_moment_kernel<<<blocks_for(n * d, 256), 256, 0, s>>>(T3, V, n, d, q0, w, M);
    return hipGetLastError();
}

hipError_t launch_hvp_final(const float* V, const float* r, const float* u, const float* W,
                            const float* PY, const float* T, const float* M,
                            const float* m_scale, int64_t n, int d, float inv_eps, float* HV,
                            hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hvp_final_kernel<<<blocks_for(n * d, 256), 256, 0, s>>>(V, r, u, W, PY, T, M, m_scale, n, d,
                                                           inv_eps, HV);
    return hipGetLastError();
}

hipError_t launch_hvp_vconv(int path, const float* V, int64_t n, int64_t n_pad, int d, int dp,
                            void* out, float* inv_sigma, hipStream_t s) {
    if (n_pad <= 0) return hipSuccess;
    if (path == PATH_MFMA_BF16)
        hvp_vconv_kernel<__bf16><<<blocks_for(n_pad, 4), 256, 0, s>>>(V, n, n_pad, d, dp,
                                                                      (__bf16*)out, inv_sigma);
    else if (path == PATH_MFMA_F16)
        hvp_vconv_kernel<_Float16><<<blocks_for(n_pad, 4), 256, 0, s>>>(V, n, n_pad, d, dp,
                                                                        (_Float16*)out, inv_sigma);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace fs
