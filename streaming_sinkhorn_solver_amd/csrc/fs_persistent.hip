// fs_persistent.hip -- the whole alternating schedule of a small low-
// dimensional problem in one launch.
//
// "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU" (gist.science
// explainer), section "Method", part 1: the f-update
//   f_i <- -eps LSE_j[(g_j - C_ij)/eps + log b_j]
// and its mirror for g, alternated (the g-update reads the new f).  In base 2,
// with the clouds centred and the cost split as C = A(x) + B(y) - 2 x'.y',
//   f_i = -eps ln2 * LSE2_j[ c_score x'_i.y'_j + beta_j ] + A_i,
//   beta_j = (g_j - B_j) c_bias + log2 b_j,  c_bias = log2(e)/eps = c_score/2.
//
// For a few hundred points per cloud a half-step is a few microseconds of
// work, and issuing it as separate kernels (key packing, the streaming pass)
// costs more in launch gaps than the work itself.  Here W workgroups (W <= 16,
// all resident at once on a 256-CU device) run every half-step of every
// stage: workgroup k owns a contiguous range of rows of the side being
// updated; it stages the other side's points with their fresh biases in LDS,
// forms the scores by fp32 FMA (one lane per row, the four waves splitting the
// keys), keeps a running (reference, sum) per row whose reference moves only
// when a chunk's terms would exceed 2^64, merges the four partials in a fixed
// order and writes its rows of the new potential.  A grid barrier then
// publishes them before the other side's update reads them.
//
// The barrier: one counter in the workspace, zeroed before the launch;
// barrier b waits until it reaches (b+1) W.  After a workgroup barrier,
// thread 0 issues an agent-scope fence (releasing the workgroup's writes),
// arrives with a relaxed atomic add, polls the counter with relaxed loads and
// issues a second agent-scope fence once it has seen every arrival (acquiring
// the others' writes) before the workgroup barrier that releases the rest of
// its workgroup.  The wait is bounded: after kSpinLimit polls a
// workgroup records an error and stops iterating (and every other workgroup
// stops at its next barrier), so every wave exits even if the workgroups were
// not resident together; each workgroup that stops this way fills f and g
// with NaN, so an unfinished solve cannot pass for a finished one.
#include <hip/hip_runtime.h>

#include "fs_device.hpp"
#include "fs_internal.h"

namespace fs {

namespace {

constexpr int kPThreads = 256;         // four waves
constexpr int kPMaxQ = 4;              // rows per lane
constexpr unsigned kSpinLimit = 1u << 22;
constexpr float kPBig = 0x1p64f;

template <int D>
struct KeyRec {
    static constexpr int F = D + 1 <= 4 ? 4 : (D + 1 <= 8 ? 8 : 12);  // floats per record
};

__device__ __forceinline__ bool grid_barrier(unsigned* counter, unsigned target, int* err) {
    __shared__ int ok;
    // the workgroup barrier orders every wave's stores before thread 0's
    // agent-scope fence, which releases them before the arrival
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        unsigned polls = 0;
        int good = 1;
        while (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            if (++polls > kSpinLimit ||
                __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
                good = 0;
                __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        __threadfence();  // acquire: the other workgroups' stores are visible
        ok = good;
    }
    __syncthreads();
    return ok != 0;
}

// One half-step of workgroup `wg` of `W`: rows [r0, r1) of cloud R against
// every point of cloud K with potential kpot.
template <int D>
__device__ void persistent_half_step(const PersistentArgs& a, bool f_side, float eps, int wg,
                                     float* __restrict__ lds_rec, float2* __restrict__ lds_part) {
    constexpr int F = KeyRec<D>::F;
    const float* __restrict__ R = f_side ? a.X : a.Y;
    const float* __restrict__ K = f_side ? a.Y : a.X;
    const float* __restrict__ Rn = f_side ? a.xn : a.yn;
    const float* __restrict__ Kn = f_side ? a.yn : a.xn;
    const float* __restrict__ Kl = f_side ? a.yl : a.xl;
    float* kpot = f_side ? a.g : a.f;
    float* out = f_side ? a.f : a.g;
    const int nr = f_side ? a.n : a.m;
    const int nk = f_side ? a.m : a.n;
    const int per = (nr + a.W - 1) / a.W;
    const int r0 = wg * per;
    const int r1 = min(nr, r0 + per);
    const double e = (double)eps;
    const float c_bias = (float)(1.4426950408889634 / e);
    const float c_score = (float)(2.8853900817779268 / e);
    const float out_scale = (float)(-e * 0.6931471805599453);

    // key records: y'_0..y'_{D-1}, beta, zeros
    for (int j = threadIdx.x; j < nk; j += kPThreads) {
        const float pot = __hip_atomic_load(kpot + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        float* rec = lds_rec + (int64_t)j * F;
#pragma unroll
        for (int c = 0; c < F; ++c)
            rec[c] = c < D ? K[(int64_t)j * a.stride + c]
                           : (c == D ? fmaf(pot - Kn[j], c_bias, Kl[j]) : 0.f);
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    // wave-uniform values are kept in scalar registers so that the key loop
    // below branches on scalars only
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // keys of this wave: a contiguous quarter
    const int kq = (nk + 3) / 4;
    const int k0 = wave * kq;
    const int k1 = min(nk, k0 + kq);
    // row slots that hold a row for at least one lane of the workgroup
    const int nq = min(kPMaxQ, (r1 - r0 + 63) / 64);
    float x[kPMaxQ][D];
    float ref[kPMaxQ], sum[kPMaxQ];
#pragma unroll
    for (int q = 0; q < kPMaxQ; ++q) {
        const int i = r0 + lane + 64 * q;
        const bool in = q < nq && i < r1;
#pragma unroll
        for (int c = 0; c < D; ++c) x[q][c] = in ? c_score * R[(int64_t)i * a.stride + c] : 0.f;
        ref[q] = -INFINITY;
        sum[q] = 0.f;
    }
    // one chunk of CH keys (cnt of them real) for every row slot
    constexpr int CH = 8;  // keys per chunk of the lazy reference
    auto chunk = [&](int j0, int cnt) {
        float kr[CH][D + 1];
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            const float* rec = lds_rec + (int64_t)(j0 + (u < cnt ? u : 0)) * F;
#pragma unroll
            for (int c = 0; c <= D; ++c) kr[u][c] = rec[c];
        }
#pragma unroll
        for (int q = 0; q < kPMaxQ; ++q) {
            if (q >= nq) break;
            float z[CH], t = 0.f;
#pragma unroll
            for (int u = 0; u < CH; ++u) {
                float acc = kr[u][D];
#pragma unroll
                for (int c = 0; c < D; ++c) acc = fmaf(x[q][c], kr[u][c], acc);
                z[u] = u < cnt ? acc : -INFINITY;
                t += ex2(z[u] - ref[q]);
            }
            if (!(t <= kPBig)) {
                // first chunk of the row, or a score far above the reference
                float mx = z[0];
#pragma unroll
                for (int u = 1; u < CH; ++u) mx = fmaxf(mx, z[u]);
                const float rn = fmaxf(ref[q], mx);
                float s = sum[q] * ex2(ref[q] - rn);
#pragma unroll
                for (int u = 0; u < CH; ++u) s += ex2(z[u] - rn);
                sum[q] = s;
                ref[q] = rn;
            } else {
                sum[q] += t;
            }
        }
    };
    int j0 = k0;
    for (; j0 + CH <= k1; j0 += CH) chunk(j0, CH);
    if (j0 < k1) chunk(j0, k1 - j0);
    // merge the four waves' partials of each row in wave order
#pragma unroll
    for (int q = 0; q < kPMaxQ; ++q)
        lds_part[(wave * kPMaxQ + q) * 64 + lane] = make_float2(ref[q], sum[q]);
    __syncthreads();
    for (int t = threadIdx.x; t < kPMaxQ * 64; t += kPThreads) {
        const int q = t >> 6, l = t & 63;
        const int i = r0 + l + 64 * q;
        if (i >= r1) continue;
        float2 p = lds_part[(0 * kPMaxQ + q) * 64 + l];
        float M = p.x, S = p.y;
#pragma unroll
        for (int w = 1; w < 4; ++w) {
            const float2 o = lds_part[(w * kPMaxQ + q) * 64 + l];
            lse_merge(M, S, o.x, o.y);
        }
        out[i] = fmaf(out_scale, M + lg2(S), Rn[i]);
    }
}

template <int D>
__global__ __launch_bounds__(kPThreads) void solve_persistent_kernel(PersistentArgs a) {
    constexpr int F = KeyRec<D>::F;
    extern __shared__ __attribute__((aligned(16))) float lds[];
    float* lds_rec = lds;
    float2* lds_part = (float2*)(lds + (int64_t)a.rec_cap * F);
    const int wg = blockIdx.x;
    unsigned bar = 0;
    // a barrier that timed out: the potentials are left as NaN, so an
    // unfinished solve cannot pass for a finished one
    auto abandon = [&]() {
        for (int i = threadIdx.x; i < a.n; i += kPThreads) a.f[i] = __builtin_nanf("");
        for (int j = threadIdx.x; j < a.m; j += kPThreads) a.g[j] = __builtin_nanf("");
    };
    for (int s = 0; s < a.n_stages; ++s) {
        const float eps = a.eps[s];
        for (int it = 0; it < a.iters; ++it) {
            persistent_half_step<D>(a, true, eps, wg, lds_rec, lds_part);
            if (!grid_barrier(a.counter, (++bar) * a.W, a.err)) return abandon();
            persistent_half_step<D>(a, false, eps, wg, lds_rec, lds_part);
            if (!grid_barrier(a.counter, (++bar) * a.W, a.err)) return abandon();
        }
    }
}

template <int D>
hipError_t persistent_launch(const PersistentArgs& a, hipStream_t s) {
    constexpr int F = KeyRec<D>::F;
    const size_t lds = sizeof(float) * (size_t)a.rec_cap * F + sizeof(float2) * 4 * kPMaxQ * 64;
    solve_persistent_kernel<D><<<a.W, kPThreads, lds, s>>>(a);
    return hipGetLastError();
}

}  // namespace

int persistent_record_floats(int d) {
    return d + 1 <= 4 ? 4 : (d + 1 <= 8 ? 8 : 12);
}

int persistent_max_points(int d) {
    // key records within 56 KiB of LDS (64 KiB with the partials), rows within
    // W = 16 workgroups x 64 lanes x kPMaxQ
    const int by_lds = (56 * 1024) / (4 * persistent_record_floats(d));
    return by_lds < 16 * 64 * kPMaxQ ? by_lds : 16 * 64 * kPMaxQ;
}

int persistent_workgroups(int64_t n, int64_t m) {
    const int64_t big = n > m ? n : m;
    int w = (int)((big + 63) / 64);
    return w < 1 ? 1 : (w > 16 ? 16 : w);
}

hipError_t launch_solve_persistent(const PersistentArgs& a, hipStream_t s) {
    if (a.W < 1 || a.W > 16 || (a.n + a.W - 1) / a.W > 64 * kPMaxQ ||
        (a.m + a.W - 1) / a.W > 64 * kPMaxQ || a.n_stages < 1 || a.n_stages > kPersistentMaxStages)
        return hipErrorInvalidValue;
    switch (a.d) {
        case 1: return persistent_launch<1>(a, s);
        case 2: return persistent_launch<2>(a, s);
        case 3: return persistent_launch<3>(a, s);
        case 4: return persistent_launch<4>(a, s);
        case 5: return persistent_launch<5>(a, s);
        case 6: return persistent_launch<6>(a, s);
        case 7: return persistent_launch<7>(a, s);
        case 8: return persistent_launch<8>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fs
