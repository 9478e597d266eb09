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
// costs more in launch gaps than the work itself.  Here W workgroups (all
// resident at once) run every half-step of every stage:
//
// * Both clouds stay in each workgroup's LDS for the whole launch: per point
//   a record of F floats (the D coordinates, then the point's current bias
//   beta when it is a key, zero padding) and a pair (A or B, log2 weight).
//   A half-step reads from global memory only the other side's potential,
//   which the workgroups wrote in the previous half-step.
// * Workgroup k owns a contiguous range of `per` rows of the side being
//   updated.  Its 64-lane waves hold RL = min(64, next power of two >= per)
//   rows per lane group and G = 64 / RL lane groups; the four waves take a
//   contiguous quarter of the keys each and the G groups of a wave take every
//   G-th key of that quarter, so small row ranges still keep every lane busy.
//   Each lane keeps a running (reference, sum) per row whose reference moves
//   only when a chunk's terms would exceed 2^64; the 4 G partials of a row are
//   merged in a fixed order (a pairwise tree across the lane groups of each
//   wave, then the waves in order) and the row's new potential written.
// * The workgroups exchange the potentials as tagged 64-bit words (the
//   value's bits, and above them the number of the half-step that produced
//   it, counted from 1 over the whole launch), stored and loaded as agent-
//   scope atomics: a workgroup that needs the other side's potential of
//   half-step h polls each word until it carries tag h (the first f-update
//   reads the caller's g).  No fence and no barrier counter are needed (each
//   word carries its own value), and a workgroup starts on half-step h + 1 as
//   soon as the words it reads are there.  A producer cannot overwrite a word
//   that a consumer still needs: before any workgroup writes the f of half-
//   step h + 2 it has read the g of half-step h + 1 from every workgroup,
//   each of which had by then finished reading the f of half-step h.  The
//   tags are zeroed before the launch.  The wait is bounded: after
//   kSpinLimit polls a workgroup records an error and stops iterating (and
//   every other workgroup stops when it next waits), so every wave exits even
//   if the workgroups were not resident together; each workgroup that stops
//   this way fills f and g with NaN, so an unfinished solve cannot pass for a
//   finished one.
#include <hip/hip_runtime.h>

#include "fs_device.hpp"
#include "fs_internal.h"

namespace fs {

namespace {

constexpr int kPThreads = 256;         // four waves
constexpr int kPMaxQ = 4;              // row slots per lane
constexpr int kPMaxPer = 64 * kPMaxQ;  // rows per workgroup
constexpr int kPMaxW = 64;             // workgroups
constexpr unsigned kSpinLimit = 1u << 22;
constexpr float kPBig = 0x1p64f;
constexpr size_t kPLdsBytes = 64 * 1024;
constexpr size_t kPPartBytes = sizeof(float2) * 4 * kPMaxQ * 64;

constexpr int record_floats(int d) { return d + 1 <= 4 ? 4 : (d + 1 <= 8 ? 8 : 12); }

size_t lds_bytes(int64_t n, int64_t m, int d) {
    return sizeof(float) * (size_t)(n + m) * (record_floats(d) + 2) + kPPartBytes;
}

__device__ __forceinline__ unsigned long long tagged(unsigned tag, float v) {
    return ((unsigned long long)tag << 32) | __float_as_uint(v);
}

// One cloud in LDS: records rec[j*F + c] (coordinates, then the bias slot)
// and aux[2j] = cost term, aux[2j+1] = log2 weight.
struct LdsCloud {
    float* rec;
    float* aux;
};

// Half-step h (counted from 0 over the launch) of workgroup `wg`: rows
// [r0, r1) of cloud R against every point of cloud K, whose potential (ktag
// with tag h; at h = 0 the caller's g, kpot, or zero when a.g_zero) gives the
// keys' biases.
// Writes the rows' new potentials to out and, tagged h + 1, to otag.
// Returns false when the wait for the keys' potentials timed out here or in
// another workgroup (the same value in every thread of the workgroup).
template <int D>
__device__ bool persistent_half_step(const PersistentArgs& a, LdsCloud R, LdsCloud K, int nr,
                                     int nk, const float* kpot, const unsigned long long* ktag,
                                     float* out, unsigned long long* otag, unsigned h, float eps,
                                     int wg, float2* __restrict__ lds_part, int* lds_bad) {
    constexpr int F = record_floats(D);
    const int per = (nr + a.W - 1) / a.W;
    const int r0 = min(nr, wg * per);
    const int r1 = min(nr, r0 + per);
    const double e = (double)eps;
    const float c_bias = (float)(1.4426950408889634 / e);
    const float c_score = (float)(2.8853900817779268 / e);
    const float out_scale = (float)(-e * 0.6931471805599453);

    // the keys' biases: every potential is requested before any is used
    constexpr int kBatch = 8;
    for (int j0 = threadIdx.x; j0 < nk; j0 += kPThreads * kBatch) {
        float pv[kBatch];
        if (h == 0) {
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                pv[u] = a.g_zero ? 0.f : kpot[min(j0 + u * kPThreads, nk - 1)];
        } else {
            // poll every word that is not there yet in the same round
            unsigned long long w[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                w[u] = __hip_atomic_load(ktag + min(j0 + u * kPThreads, nk - 1),
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (unsigned polls = 1;; ++polls) {
                bool there = true;
#pragma unroll
                for (int u = 0; u < kBatch; ++u) there = there && (unsigned)(w[u] >> 32) == h;
                if (there) break;
                if ((polls & 63) == 0 &&
                    (polls > kSpinLimit ||
                     __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) {
                    __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    *lds_bad = 1;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
#pragma unroll
                for (int u = 0; u < kBatch; ++u)
                    if ((unsigned)(w[u] >> 32) != h)
                        w[u] = __hip_atomic_load(ktag + min(j0 + u * kPThreads, nk - 1),
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) pv[u] = __uint_as_float((unsigned)w[u]);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int j = j0 + u * kPThreads;
            if (j < nk) K.rec[j * F + D] = fmaf(pv[u] - K.aux[2 * j], c_bias, K.aux[2 * j + 1]);
        }
    }
    __syncthreads();
    if (*lds_bad) return false;

    // lane layout (uniform values in scalar registers: the loops below branch
    // on scalars only, apart from the tail chunk's per-lane key mask)
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int rl_bits = 0;
    while ((1 << rl_bits) < per && rl_bits < 6) ++rl_bits;
    const int RL = 1 << rl_bits;  // rows per lane group
    const int G = 64 >> rl_bits;  // lane groups
    const int grp = lane >> rl_bits;
    const int rl = lane & (RL - 1);
    const int nq = min(kPMaxQ, (r1 - r0 + RL - 1) / RL);  // row slots in use
    const int kq = (nk + 3) / 4;
    const int k0 = min(nk, wave * kq);
    const int cw = min(nk, k0 + kq) - k0;  // keys of this wave
    const int steps = (cw + G - 1) / G;    // key steps of a lane group
    const int full = cw / G;               // steps where every group has a key

    float x[kPMaxQ][D];
    float ref[kPMaxQ], sum[kPMaxQ];
#pragma unroll
    for (int q = 0; q < kPMaxQ; ++q) {
        const int i = min(r0 + rl + RL * q, nr - 1);
#pragma unroll
        for (int c = 0; c < D; ++c) x[q][c] = q < nq ? c_score * R.rec[i * F + c] : 0.f;
        ref[q] = -INFINITY;
        sum[q] = 0.f;
    }
    // keys k0 + (t0 + u) G + grp for u < CH; `masked`: some of them may lie
    // past the wave's range (their terms are dropped); `first`: the row's
    // first chunk, whose maximum becomes the reference directly
    constexpr int CH = D <= 4 ? 16 : 8;  // keys per chunk of the lazy reference
    auto chunk = [&](int t0, bool masked, bool first) {
        float kr[CH][D + 1];
        bool live[CH];
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            const int t = t0 + u;
            live[u] = !masked || t * G + grp < cw;
            const int j = k0 + (live[u] ? t * G + grp : 0);
#pragma unroll
            for (int c = 0; c <= D; ++c) kr[u][c] = K.rec[j * F + c];
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
                z[u] = live[u] ? acc : -INFINITY;
                if (!first) t += ex2(z[u] - ref[q]);
            }
            if (first || !(t <= kPBig)) {
                // first chunk of the row, or a score far above the reference
                // (a chunk with no live key leaves the state as it is)
                float mx = z[0];
#pragma unroll
                for (int u = 1; u < CH; ++u) mx = fmaxf(mx, z[u]);
                const float rn = fmaxf(ref[q], mx);
                if (rn != -INFINITY) {
                    float s = sum[q] * ex2(ref[q] - rn);
#pragma unroll
                    for (int u = 0; u < CH; ++u) s += ex2(z[u] - rn);
                    sum[q] = s;
                    ref[q] = rn;
                }
            } else {
                sum[q] += t;
            }
        }
    };
    if (cw > 0) {
        int t0 = 0;
        if (CH <= full) {
            chunk(0, false, true);
            for (t0 = CH; t0 + CH <= full; t0 += CH) chunk(t0, false, false);
            if (t0 < steps) chunk(t0, true, false);
        } else {
            chunk(0, true, true);
        }
    }

    // merge the partials of each row: the G lane groups of a wave pairwise
    // across lanes (lane l with lane l ^ s for s = RL, 2 RL, .., 32: both
    // lanes form the same sum), then the four waves in order
    for (int sh = RL; sh < 64; sh <<= 1) {
#pragma unroll
        for (int q = 0; q < kPMaxQ; ++q) {
            if (q >= nq) break;
            const float Mo = __shfl_xor(ref[q], sh);
            const float So = __shfl_xor(sum[q], sh);
            lse_merge(ref[q], sum[q], Mo, So);
        }
    }
    if (grp == 0) {
#pragma unroll
        for (int q = 0; q < kPMaxQ; ++q)
            lds_part[(wave * kPMaxQ + q) * 64 + rl] = make_float2(ref[q], sum[q]);
    }
    __syncthreads();
    for (int t = threadIdx.x; t < r1 - r0; t += kPThreads) {
        const int q = t >> rl_bits, l = t & (RL - 1);
        const float2 p0 = lds_part[q * 64 + l];
        float M = p0.x, S = p0.y;
#pragma unroll
        for (int w = 1; w < 4; ++w) {
            const float2 o = lds_part[(w * kPMaxQ + q) * 64 + l];
            lse_merge(M, S, o.x, o.y);
        }
        const float v = fmaf(out_scale, M + lg2(S), R.aux[2 * (r0 + t)]);
        out[r0 + t] = v;
        __hip_atomic_store(otag + r0 + t, tagged(h + 1, v), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    return true;
}

template <int D>
__global__ __launch_bounds__(kPThreads) void solve_persistent_kernel(PersistentArgs a) {
    constexpr int F = record_floats(D);
    extern __shared__ __attribute__((aligned(16))) float lds[];
    const int nm = a.n + a.m;
    const LdsCloud cx{lds, lds + nm * F};
    const LdsCloud cy{lds + a.n * F, lds + nm * F + 2 * a.n};
    float2* lds_part = (float2*)(lds + nm * (F + 2));
    // both clouds into LDS, once
    for (int t = threadIdx.x; t < nm * F; t += kPThreads) {
        const bool xs = t < a.n * F;
        const int j = (xs ? t : t - a.n * F) / F, c = t % F;
        const float* src = xs ? a.X : a.Y;
        lds[t] = c < D ? src[(int64_t)j * a.stride + c] : 0.f;
    }
    for (int j = threadIdx.x; j < nm; j += kPThreads) {
        const bool xs = j < a.n;
        const int k = xs ? j : j - a.n;
        float* aux = xs ? cx.aux : cy.aux;
        aux[2 * k] = xs ? a.xn[k] : a.yn[k];
        aux[2 * k + 1] = xs ? a.xl[k] : a.yl[k];
    }
    __shared__ int bad;
    if (threadIdx.x == 0) bad = 0;
    __syncthreads();
    const int wg = blockIdx.x;
    unsigned h = 0;
    for (int s = 0; s < a.n_stages; ++s) {
        const float eps = a.eps[s];
        for (int it = 0; it < a.iters; ++it) {
            if (!persistent_half_step<D>(a, cx, cy, a.n, a.m, a.g, a.tg, a.f, a.tf, h++, eps, wg,
                                         lds_part, &bad) ||
                !persistent_half_step<D>(a, cy, cx, a.m, a.n, a.f, a.tf, a.g, a.tg, h++, eps, wg,
                                         lds_part, &bad)) {
                // a wait that timed out: the potentials are left as NaN, so
                // an unfinished solve cannot pass for a finished one
                for (int i = threadIdx.x; i < a.n; i += kPThreads) a.f[i] = __builtin_nanf("");
                for (int j = threadIdx.x; j < a.m; j += kPThreads) a.g[j] = __builtin_nanf("");
                return;
            }
        }
    }
}

template <int D>
hipError_t persistent_launch(const PersistentArgs& a, hipStream_t s) {
    solve_persistent_kernel<D><<<a.W, kPThreads, lds_bytes(a.n, a.m, D), s>>>(a);
    return hipGetLastError();
}

}  // namespace

bool persistent_fits(int64_t n, int64_t m, int d) {
    return d >= 1 && d <= 8 && n >= 1 && m >= 1 && lds_bytes(n, m, d) <= kPLdsBytes &&
           (n + kPMaxW - 1) / kPMaxW <= kPMaxPer && (m + kPMaxW - 1) / kPMaxW <= kPMaxPer;
}

int persistent_workgroups(int64_t n, int64_t m) {
    // about 8 rows per workgroup (every lane busy with eight lane groups),
    // at most kPMaxW workgroups: measured on the 512 x 512, 3-D recipe, 100
    // iterations take 0.78 ms with 64 workgroups, 0.90 ms with 32, 1.12 ms
    // with 16 (and 0.82-0.83 ms with 96 or 128)
    const int64_t big = n > m ? n : m;
    const int64_t w = (big + 7) / 8;
    return (int)(w < 1 ? 1 : (w > kPMaxW ? kPMaxW : w));
}

hipError_t launch_solve_persistent(const PersistentArgs& a, hipStream_t s) {
    if (a.W < 1 || a.W > kPMaxW || !persistent_fits(a.n, a.m, a.d) ||
        (a.n + a.W - 1) / a.W > kPMaxPer || (a.m + a.W - 1) / a.W > kPMaxPer ||
        a.n_stages < 1 || a.n_stages > kPersistentMaxStages || a.iters < 1 ||
        2 * (int64_t)a.n_stages * a.iters >= (int64_t)0xffffffff)
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
