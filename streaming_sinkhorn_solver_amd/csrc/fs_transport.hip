// fs_transport.hip -- streaming application of the transport plan, U = P.V.
//
// "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU" (gist.science
// explainer), section "Method", part 3: the barycentric projection and the
// gradient are weighted averages under the plan, computed by the same
// streaming traversal as the Sinkhorn update, without ever storing P.
//
// With the plan P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps) and the base-2
// scores z2_ij = c_score x~_i.y~_j + beta_j, beta_j = (g_j - |y~_j|^2) c_bias
// + log2 b_j (the f-update's scores under the current g):
//     P_ij = a_i 2^(z2_ij - R_i) 2^(R_i + (f_i - |x~_i|^2) c_bias)
// for any row reference R_i.  The weights p_ij = 2^(z2_ij - R_i) go through
// a float16 product, so R_i must keep them in range: near the row LSE
// L_i = log2 sum_j 2^(z2_ij) they lie in (0, 1] and sum to 1.  The vector and
// 1024-wide kernels take R_i = L_i from an exact LSE pass run first.  The
// streaming kernel takes R_i = L_i - 10, with L_i read from the row
// potential when no LSE is given -- f_i is the f-update's output, -L_i/c_bias
// + |x~_i|^2, up to the change of g since -- and checks afterwards that the
// weights stayed in range (rows that did not are recomputed); the row factor
// is applied once at the end.
//
// Matrix-core kernel: per 32-key tile the score MFMAs of the LSE kernel give,
// in each lane, 16 weights of ONE row; they are packed to f16 and used
// directly as the A operand of v_mfma_f32_32x32x16_f16 against a transposed
// f16 copy of V (keys on the contraction axis, in the same slot order), so
// the weights never leave registers.  V is copied once, transposed and scaled
// by a power of two into the f16 range; the scale is undone exactly at the end.
// Kernels: transport_stream_kernel (d_pad <= 512; 256 output columns per
// workgroup), transport_wide_kernel (two-byte scores at d_pad = 1024; the
// contraction and the output columns split over wave pairs),
// transport_mfma_kernel (the remaining matrix case, fp32 at d_pad = 512) and
// transport_valu_kernel (d <= 8, fp32 vector arithmetic).
#include <algorithm>
#include <functional>
#include <vector>

#include "fs_device.hpp"
#include "fs_internal.h"

namespace fs {

namespace {

// ---------------------------------------------------- V -> f16, transposed
// max|V| over all entries as the bit pattern of a non-negative float (for
// which integer order is float order), so an atomic max is order independent.
__device__ __forceinline__ float v_value(const float* __restrict__ V, int64_t j, int dv, int k,
                                         const float* __restrict__ rs,
                                         const float* __restrict__ off) {
    float v = V[j * dv + k];
    if (rs) v *= rs[j];
    if (off) v -= off[k];
    return v;
}

__global__ __launch_bounds__(256) void vmax_kernel(const float* __restrict__ V, int64_t count,
                                                   int dv, const float* __restrict__ rs,
                                                   const float* __restrict__ off,
                                                   unsigned* __restrict__ maxbits) {
    __shared__ float red[256];
    float mx = 0.f;
    const int64_t stride = (int64_t)gridDim.x * 256;
    if (!rs && !off) {
        // plain values: no row/column index needed; 16-byte loads when aligned
        int64_t k0 = 0;
        if (((uintptr_t)V & 15) == 0) {
            const int64_t n4 = count / 4;
            const float4* V4 = (const float4*)V;
            for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < n4; k += stride) {
                const float4 v = V4[k];
                mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
            }
            k0 = n4 * 4;
        }
        for (int64_t k = k0 + (int64_t)blockIdx.x * 256 + threadIdx.x; k < count; k += stride)
            mx = fmaxf(mx, fabsf(V[k]));
    } else {
        for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < count; k += stride)
            mx = fmaxf(mx, fabsf(v_value(V, k / dv, dv, (int)(k % dv), rs, off)));
    }
    red[threadIdx.x] = mx;
    __syncthreads();
    for (int o = 128; o >= 1; o >>= 1) {
        if (threadIdx.x < o) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
        __syncthreads();
    }
    // one atomic per workgroup, and none where the word already holds as
    // much (after the first workgroups almost none: contended atomics on one
    // word would serialise the grid)
    if (threadIdx.x == 0) {
        const unsigned seen = __hip_atomic_load(maxbits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (__float_as_uint(red[0]) > seen) atomicMax(maxbits, __float_as_uint(red[0]));
    }
}

// scratch[0] = 2^s, scratch[1] = 2^-s, with s chosen so max|V| 2^s < 2^14.
__global__ void vscale_kernel(const unsigned* __restrict__ maxbits, float* __restrict__ scratch) {
    if (threadIdx.x != 0) return;
    const float m = __uint_as_float(maxbits[0]);
    int s = 0;
    if (m > 0.f && m <= 3.402823466e38f) {
        int e;
        frexpf(m, &e);  // m in [2^(e-1), 2^e)
        s = 14 - e;
        s = s > 100 ? 100 : (s < -100 ? -100 : s);
    }
    scratch[0] = ldexpf(1.f, s);
    scratch[1] = ldexpf(1.f, -s);
}

// Vt[k][pos(j)] = f16((V[j][k] rs[j] - off[k]) * 2^s) (rs: 1 and off: 0 when
// NULL) for j < m, 0 for m <= j < m_pad, where
// pos(j) = j, or with `swap` j with bits 2 and 3 exchanged (the key order the
// streaming kernel reads: each 16-key group as [0-3, 8-11, 4-7, 12-15]).
__global__ __launch_bounds__(256) void transpose_v_kernel(const float* __restrict__ V, int m,
                                                          int64_t m_pad, int dv,
                                                          const float* __restrict__ scratch,
                                                          _Float16* __restrict__ Vt, int swap,
                                                          const float* __restrict__ rs,
                                                          const float* __restrict__ off) {
    __shared__ float tile[32][33];
    const float sc = scratch[0];
    const int j0 = blockIdx.x * 32, k0 = blockIdx.y * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
    for (int yy = ty; yy < 32; yy += 8) {
        const int j = j0 + yy, k = k0 + tx;
        tile[yy][tx] = (j < m && k < dv) ? v_value(V, j, dv, k, rs, off) * sc : 0.f;
    }
    __syncthreads();
    for (int yy = ty; yy < 32; yy += 8) {
        const int k = k0 + yy, j = j0 + tx;
        const int pj = swap ? (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1) : j;
        if (k < dv && j < m_pad) Vt[(int64_t)k * m_pad + pj] = (_Float16)tile[tx][yy];
    }
}

// ------------------------------------------------------------ vector path
// d <= 8: R rows per thread and DVC output columns per thread (grid.y over
// column blocks; DVC the smallest of 1, 2, 4, 8, 16, 32 that covers dv, or 32
// with several blocks).  Tiles of KT keys -- their coordinates, the biased
// score term and the block's V values -- are staged in LDS by the whole
// workgroup and read back as broadcasts, so each key costs one LDS pass per
// wave instead of a chain of scalar loads per thread.  Per pair: D FMAs,
// one exponential, DVC FMAs.
template <int D, int R, int DVC>
__global__ __launch_bounds__(256) void transport_valu_kernel(TransportArgs a) {
    constexpr int DP = D <= 4 ? 4 : 8;
    constexpr int KT = 64;
    constexpr int KW = D + 1;  // coordinates, then the bias
    __shared__ float kx[KT * KW];
    __shared__ float kv[KT * DVC];
    const float* __restrict__ rows = (const float*)a.rows;
    const float* __restrict__ keys = (const float*)a.keys;
    const int t = threadIdx.x;
    const int64_t row_base = (int64_t)blockIdx.x * 256 * R;
    const int c0 = blockIdx.y * DVC;
    float x[R][D], L[R], u[R][DVC];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t i = row_base + r * 256 + t;
        const bool live = i < a.n_rows;
#pragma unroll
        for (int k = 0; k < D; ++k) x[r][k] = live ? rows[i * DP + k] * a.c_score : 0.f;
        L[r] = live ? a.row_lse2[i] : INFINITY;  // rows past n: every weight 0
#pragma unroll
        for (int c = 0; c < DVC; ++c) u[r][c] = 0.f;
    }
    for (int j0 = 0; j0 < a.n_keys; j0 += KT) {
        __syncthreads();  // the previous tile is consumed
        for (int e = t; e < KT * KW; e += 256) {
            const int jj = e / KW, k = e - jj * KW;
            const int j = j0 + jj;
            float v;
            if (k < D)
                v = j < a.n_keys ? keys[(int64_t)j * DP + k] : 0.f;
            else
                v = j < a.n_keys ? fmaf(a.key_pot[j] - a.key_nrm[j], a.c_bias, a.key_lw2[j])
                                 : -INFINITY;
            kx[e] = v;
        }
        for (int e = t; e < KT * DVC; e += 256) {
            const int jj = e / DVC, c = e - jj * DVC;
            const int j = j0 + jj;
            kv[e] = (j < a.n_keys && c0 + c < a.dv)
                        ? v_value(a.V, j, a.dv, c0 + c, a.v_rscale, a.v_off)
                        : 0.f;
        }
        __syncthreads();
        const int kn = min(KT, a.n_keys - j0);
        for (int jj = 0; jj < kn; ++jj) {
            float ky[KW], vv[DVC];
#pragma unroll
            for (int k = 0; k < KW; ++k) ky[k] = kx[jj * KW + k];
#pragma unroll
            for (int c = 0; c < DVC; ++c) vv[c] = kv[jj * DVC + c];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float z = ky[D];
#pragma unroll
                for (int k = 0; k < D; ++k) z = fmaf(x[r][k], ky[k], z);
                const float p = ex2(z - L[r]);
#pragma unroll
                for (int c = 0; c < DVC; ++c) u[r][c] = fmaf(p, vv[c], u[r][c]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t i = row_base + r * 256 + t;
        if (i >= a.n_rows) continue;
        float sc = ex2(L[r] + (a.row_pot[i] - a.row_nrm[i]) * a.c_bias);
        if (!a.divide_by_a) sc *= a.row_w[i];
        float* ur = a.U + i * a.dv + c0;
#pragma unroll
        for (int c = 0; c < DVC; ++c)
            if (c0 + c < a.dv) ur[c] = u[r][c] * sc;
    }
}

// ------------------------------------------------------ matrix-core path
template <int OP>
__device__ __forceinline__ f32x16 score_step(const uint4& av, const uint4& bv, f32x16 acc) {
    if constexpr (OP == OP_BF16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                       __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
    } else if constexpr (OP == OP_F16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, av),
                                                      __builtin_bit_cast(f16x8, bv), acc, 0, 0, 0);
    } else {
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(av.x), __uint_as_float(bv.x), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(av.y), __uint_as_float(bv.y), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(av.z), __uint_as_float(bv.z), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(av.w), __uint_as_float(bv.w), acc, 0, 0, 0);
        return acc;
    }
}

// The same two-byte score step with the accumulators in vector registers.
// The streaming kernel's 512-column output block takes all 256 accumulation
// registers, so its score accumulators must live in vector registers; the
// compiler places every matrix instruction's accumulators in the
// accumulation registers of a kernel that uses them and would shuttle one
// output block in and out of them on every tile.  Written as inline
// assembly, the instruction has no compiler-inserted hazard waits, so the
// caller keeps the rules of its result: back-to-back accumulation into the
// same registers needs none; a vector instruction reading the result waits
// for the instruction to finish (score_result_wait); a vector write of the
// accumulators right before the first step is covered by score_seed_wait.
template <int OP>
__device__ __forceinline__ void score_step_vgpr(const uint4& av, const u32x4& bv, f32x16& acc) {
    const u32x4 a = __builtin_bit_cast(u32x4, av);
    if constexpr (OP == OP_BF16)
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(bv));
    else
        asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(bv));
}
// 24 wait states: more than an 8-pass matrix instruction's result needs
// before a vector instruction may read it.
__device__ __forceinline__ void score_result_wait(f32x16& acc) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc));
}
__device__ __forceinline__ void score_seed_wait(f32x16& acc) {
    asm volatile("s_nop 3" : "+v"(acc));
}

// 16x16x32 score step of the 1024-wide kernel (two-byte types only)
template <int OP>
__device__ __forceinline__ f32x4 mfma16_step(const uint4& av, const u32x4& bv, f32x4 acc) {
    if constexpr (OP == OP_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                       __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av),
                                                      __builtin_bit_cast(f16x8, bv), acc, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    const _Float16 l = (_Float16)lo, h = (_Float16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, l) | ((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
}

// Transport kernel: 4 waves x 32 rows, output columns [c0, c0 + 32*NB).
// Pipeline stage t: DMA key tile t+2 and V^T tile t+1; score MFMAs of tile
// t+1; for tile t the weights p = 2^(z2 - L) are packed to f16 in registers
// and multiplied with the V^T tile on v_mfma_f32_32x32x16_f16.  Register r
// of the score accumulator holds key 8*(r/4) + 4*h + (r%4); registers 0..7
// and 8..15 are the A operands of the two products over the tile's 32 keys,
// and the V^T fragments are fetched for the same keys in the same slot order.
// V^T tile rows are 64 bytes (32 f16 keys); 16-byte chunk c of row r sits at
// r*4 + (c ^ ((r >> 2) & 3)) so that 16 consecutive rows hit distinct banks.
template <int OP, int NG, int NB>
__global__ __launch_bounds__(256, 1) void transport_mfma_kernel(TransportArgs a, int64_t m_pad) {
    constexpr int WAVES = 4;
    constexpr int CPR = 2 * NG;
    constexpr int ROW_BYTES = CPR * 16;
    constexpr int TILE_CHUNKS = kKeyTile * CPR;
    constexpr int TILE_INSTR = TILE_CHUNKS / 64;
    constexpr int INSTR_PER_WAVE = (TILE_INSTR + WAVES - 1) / WAVES;
    constexpr int SWZ = CPR >= 16 ? 15 : CPR - 1;
    constexpr int JB = SWZ + 1 < 2 * NG ? (SWZ + 1) / 2 : NG;
    constexpr int KB = NG / JB;
    constexpr int DVC = 32 * NB;
    constexpr int VT_CHUNKS = DVC * 4;
    constexpr int VT_INSTR = VT_CHUNKS / 64;
    constexpr int VT_PER_WAVE = (VT_INSTR + WAVES - 1) / WAVES;

    __shared__ __attribute__((aligned(16))) uint4 kbuf0[TILE_CHUNKS];
    __shared__ __attribute__((aligned(16))) uint4 kbuf1[TILE_CHUNKS];
    __shared__ __attribute__((aligned(16))) uint4 vbuf0[VT_CHUNKS];
    __shared__ __attribute__((aligned(16))) uint4 vbuf1[VT_CHUNKS];
    __shared__ __attribute__((aligned(16))) float bbuf[3][kKeyTile];
    __shared__ float rowscale[WAVES][32];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 31, h = lane >> 5;
    const int row0 = blockIdx.x * (WAVES * 32) + wave * 32;
    const int c0 = blockIdx.y * DVC;

    uint4 q[NG];
    {
        const char* rp = (const char*)a.rows + (int64_t)(row0 + ln) * ROW_BYTES + h * 16;
#pragma unroll
        for (int g = 0; g < NG; ++g) q[g] = *(const uint4*)(rp + g * 32);
    }
    const int myrow = row0 + ln;
    const float L = myrow < a.n_rows ? a.row_lse2[myrow] : 0.f;

    const int ntiles = (a.n_keys + kKeyTile - 1) / kKeyTile;
    const char* __restrict__ keys = (const char*)a.keys;
    const char* __restrict__ Vt = (const char*)a.Vt;

    auto issue_k = [&](int k, uint4* dst) __attribute__((always_inline)) {
        const char* tbase = keys + (int64_t)(k * kKeyTile) * ROW_BYTES;
#pragma unroll
        for (int l = 0; l < INSTR_PER_WAVE; ++l) {
            const int Li = l * WAVES + wave;
            if (TILE_INSTR % WAVES == 0 || Li < TILE_INSTR) {
                const int P = Li * 64 + lane;
                const int m = P / CPR, cp = P % CPR;
                const char* src = tbase + m * ROW_BYTES + (cp ^ (m & SWZ)) * 16;
                __builtin_amdgcn_global_load_lds(
                    (const void*)src, (__attribute__((address_space(3))) void*)(dst + Li * 64), 16, 0,
                    0);
            }
        }
    };
    auto issue_v = [&](int k, uint4* dst) __attribute__((always_inline)) {
#pragma unroll
        for (int l = 0; l < VT_PER_WAVE; ++l) {
            const int Li = l * WAVES + wave;
            if (VT_INSTR % WAVES == 0 || Li < VT_INSTR) {
                const int P = Li * 64 + lane;
                const int r = P >> 2, cp = P & 3;
                const int col = min(c0 + r, a.dv - 1);  // rows past dv: any valid row, unused
                const char* src = Vt + ((int64_t)col * m_pad + k * kKeyTile) * 2 +
                                  (cp ^ ((r >> 2) & 3)) * 16;
                __builtin_amdgcn_global_load_lds(
                    (const void*)src, (__attribute__((address_space(3))) void*)(dst + Li * 64), 16, 0,
                    0);
            }
        }
    };
    auto load_beta = [&](int k) __attribute__((always_inline)) -> float {
        const int j = k * kKeyTile + tid;
        float b = -INFINITY;
        if (tid < kKeyTile && j < a.n_keys)
            b = fmaf(a.key_pot[j] - a.key_nrm[j], a.c_bias, a.key_lw2[j]);
        return b;
    };

    int abase[JB];
#pragma unroll
    for (int j = 0; j < JB; ++j) abase[j] = (ln * CPR + ((2 * j + h) ^ (ln & SWZ))) * 16;
    auto scores = [&](const uint4* src, f32x16& acc) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
        const char* kb = (const char*)src;
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            uint4 av[JB];
#pragma unroll
            for (int j = 0; j < JB; ++j) av[j] = *(const uint4*)(kb + abase[j] + k * (2 * JB * 16));
#pragma unroll
            for (int j = 0; j < JB; ++j) acc = score_step<OP>(av[j], q[JB * k + j], acc);
        }
    };

    f32x16 u[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) u[nb][r] = 0.f;

    // V^T fragment offsets (bytes within a tile) of this lane for chunk c.
    auto voff = [&](int nb, int c) __attribute__((always_inline)) -> int {
        const int r = nb * 32 + ln;
        return (r * 4 + (c ^ ((r >> 2) & 3))) * 16 + 8 * h;
    };
    auto weights_pv = [&](const f32x16& acc, const float* bb, const uint4* vsrc)
                          __attribute__((always_inline)) {
        f16x8 p0, p1;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const float4 bv = *(const float4*)&bb[8 * qq + 4 * h];
            const float bq[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p = ex2(fmaf(acc[4 * qq + e], a.c_score, bq[e]) - L);
                if (qq < 2)
                    p0[4 * qq + e] = (_Float16)p;
                else
                    p1[4 * (qq - 2) + e] = (_Float16)p;
            }
        }
        const char* vb = (const char*)vsrc;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const uint2 k0 = *(const uint2*)(vb + voff(nb, 0));
            const uint2 k1 = *(const uint2*)(vb + voff(nb, 1));
            const uint2 k2 = *(const uint2*)(vb + voff(nb, 2));
            const uint2 k3 = *(const uint2*)(vb + voff(nb, 3));
            const f16x8 b0 = __builtin_bit_cast(f16x8, make_uint4(k0.x, k0.y, k1.x, k1.y));
            const f16x8 b1 = __builtin_bit_cast(f16x8, make_uint4(k2.x, k2.y, k3.x, k3.y));
            u[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(p0, b0, u[nb], 0, 0, 0);
            u[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(p1, b1, u[nb], 0, 0, 0);
        }
    };

    // prologue: key tiles 0, 1 and V^T tile 0 loaded; scores of tile 0
    float bn0 = 0.f, bn1 = 0.f;
    issue_k(0, kbuf0);
    issue_v(0, vbuf0);
    bn0 = load_beta(0);
    if (ntiles > 1) {
        issue_k(1, kbuf1);
        bn1 = load_beta(1);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (tid < kKeyTile) {
        bbuf[0][tid] = bn0;
        bbuf[1][tid] = bn1;
    }
    __syncthreads();
    f32x16 accA, accB;
    scores(kbuf0, accA);
    __syncthreads();  // all waves done with key tile 0 before kbuf0 is reloaded

#define FS_TSTAGE(t_, CUR, NXT, KCUR, KNEXT, VCUR, VNEXT)                          \
    do {                                                                          \
        const int ts = (t_);                                                      \
        float bn = 0.f;                                                           \
        if (ts + 2 < ntiles) {                                                    \
            issue_k(ts + 2, KCUR);                                                \
            bn = load_beta(ts + 2);                                               \
        }                                                                         \
        if (ts + 1 < ntiles) issue_v(ts + 1, VNEXT);                              \
        scores(KNEXT, NXT);                                                       \
        weights_pv(CUR, bbuf[ts % 3], VCUR);                                      \
        if (ts + 1 < ntiles) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");     \
        if (ts + 2 < ntiles && tid < kKeyTile) bbuf[(ts + 2) % 3][tid] = bn;       \
        __syncthreads();                                                          \
    } while (0)

    for (int t = 0; t < ntiles; t += 2) {
        FS_TSTAGE(t, accA, accB, kbuf0, kbuf1, vbuf0, vbuf1);
        if (t + 1 < ntiles) FS_TSTAGE(t + 1, accB, accA, kbuf1, kbuf0, vbuf1, vbuf0);
    }
#undef FS_TSTAGE

    // Row factor 2^(L_i + (f_i - |x~_i|^2) c_bias) [* a_i] * 2^-s.
    if (h == 0) {
        float sc = 0.f;
        if (myrow < a.n_rows) {
            sc = ex2(L + (a.row_pot[myrow] - a.row_nrm[myrow]) * a.c_bias);
            if (!a.divide_by_a) sc *= a.row_w[myrow];
            sc *= a.v_unscale_dev[0];
        }
        rowscale[wave][ln] = sc;
    }
    __syncthreads();
    // Output register r of lane (ln, h): row 8*(r/4) + 4*h + (r%4), column ln.
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int col = c0 + nb * 32 + ln;
        if (col >= a.dv) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int rr = 8 * (r >> 2) + 4 * h + (r & 3);
            const int row = row0 + rr;
            if (row < a.n_rows) a.U[(int64_t)row * a.dv + col] = u[nb][r] * rowscale[wave][rr];
        }
    }
}

// ------------------------------------------- streaming kernel (d <= 512)
// Key biases in dot-product units, the seeds of the score accumulators:
// The streaming kernel's row reference R sits kRefSlack below the row's LSE2
// (when it is known), so the weights of a row sum to about 2^10 and its
// largest weights are normal float16 values whatever the number of keys,
// while none exceeds 2^10.  A reference taken from the row potential is
// checked after the pass: rows whose score maximum exceeds it by more than
// kMaxOver (weights near the float16 limit) or whose weights are too small
// for their rounding are recomputed against their score maximum.
constexpr float kRefSlack = 10.f;
constexpr float kMaxOver = 15.f;

// kb[j] = (g_j - B_j)/2 + log2(b_j)/(2 c_bias) (c_score = 2 c_bias), -inf for
// the padding keys m <= j < m_pad.  Written with the same expression as the
// LSE kernel's seeds, so both passes form bit-identical scores.
__global__ __launch_bounds__(256) void key_bias_kernel(TransportArgs a, int64_t m_pad,
                                                       float* __restrict__ kb) {
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= m_pad) return;
    kb[j] = j < a.n_keys
                ? fmaf(a.key_lw2[j], 0.5f / a.c_bias, 0.5f * (a.key_pot[j] - a.key_nrm[j]))
                : -INFINITY;
}

// U = P.V for one (row block, column block, key range): 4 waves x 32 rows,
// 32*NBV output columns, keys [j0, j1), weights against the row reference R
// (REF_GIVEN: row_lse2 - kRefSlack; REF_ONLINE: from the row potential;
// REF_REPAIR: the score maximum the first pass recorded, only in row blocks
// holding a marked row).  With row_ref the pass records per row its R, the
// sum of its weights and its score maximum.  Everything the pass needs per row
// stays in registers: the resident row block (B operand of the scores), the
// 16 score accumulators of two tiles and the NBV output blocks (32 x 32 each;
// with NBV = 16 they take the 256 accumulation registers).
//
// Stage t (32-key tiles; K slot t%2 holds tile t, V slot t%2 holds V^T of
// tile t):
//   (1) DMA key tile t+2 (and its 32 biases) into the K slot tile t used and
//       the V^T tile t+1 into the other V slot (loads past the end are
//       clamped to the last tile: in-bounds copies into slots no one reads);
//   (2) the score instructions of tile t+1 (accumulators seeded with the key
//       biases, as in the LSE kernel);
//   (3) the weights of tile t, p = 2^(c_score acc - R) (summed into S), packed to
//       f16 in accumulator order: register r of lane (row, h) holds key
//       8(r/4) + 4h + (r%4), so registers 0..7 and 8..15 are the A operands
//       of the two 16-key products of the tile;
//   (4) the P.V instructions of tile t against V^T fragments read from LDS;
//   (5) wait for this stage's loads, barrier.
// V^T rows hold the keys of each 16-key group in the order [0-3, 8-11, 4-7,
// 12-15] (bits 2 and 3 of the key index swapped), so that the eight keys lane
// half h needs for one product -- 4h..4h+3 and 8+4h..8+4h+3 -- are one
// 16-byte chunk, 2q + h for group q; chunk c of V^T row r is stored at
// r*4 + (c ^ ((r >> 2) & 3)), conflict-free for 16 consecutive rows.
template <int OP, int NG, int NBV>
__global__ __launch_bounds__(256, 1) void transport_stream_kernel(TransportArgs a,
                                                                  int64_t m_pad) {
    constexpr int WAVES = 4;
    constexpr int CPR = 2 * NG;
    constexpr int ROW_BYTES = CPR * 16;
    constexpr int KT_CHUNKS = kKeyTile * CPR;
    constexpr int KT_INSTR = KT_CHUNKS / 64;
    constexpr int KT_PER_WAVE = (KT_INSTR + WAVES - 1) / WAVES;
    constexpr int SWZ = CPR >= 16 ? 15 : CPR - 1;
    constexpr int JB = SWZ + 1 < 2 * NG ? (SWZ + 1) / 2 : NG;
    constexpr int AP = NG < 4 ? NG : 4;  // key fragments in flight
    constexpr int DVC = 32 * NBV;
    constexpr int VT_CHUNKS = DVC * 4;
    // score accumulators in vector registers (see score_step_vgpr)
    constexpr bool VGPR_SCORES = NBV == 16 && OP != OP_F32;
    constexpr int VT_INSTR = VT_CHUNKS / 64;
    constexpr int VT_PER_WAVE = (VT_INSTR + WAVES - 1) / WAVES;

    // tile slots: three when they fit in LDS (loads then have two stages to
    // land), else two (one stage)
    constexpr int NB = 3 * (KT_CHUNKS + VT_CHUNKS) * 16 + 1024 <= 163840 ? 3 : 2;
    __shared__ __attribute__((aligned(16))) uint4 kbuf[NB * KT_CHUNKS];
    __shared__ __attribute__((aligned(16))) uint4 vbuf[NB * VT_CHUNKS];
    __shared__ __attribute__((aligned(16))) float bbuf[NB * kKeyTile];
    __shared__ float rowscale[WAVES][32];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 31, h = lane >> 5;
    const int n_cb = (a.dv + DVC - 1) / DVC;
    // Work (1-D grid): workgroup b runs on XCD b % 8 as that XCD's item
    // k = b / 8.  Each XCD owns a contiguous run of Ux work units ((row
    // block, column block) pairs) and runs all their first key ranges, then
    // all their second ones, ...: the ranges come longest first, so the
    // XCD's compute units take the short ones as they free up, and the
    // workgroups an XCD runs together stream the same key range through its
    // L2.  Items past the XCD's share exit at once.
    int row_block, cb, split;
    {
        const int b = blockIdx.x, x = b & 7, k = b >> 3;
        const int q = a.n_units >> 3, rem = a.n_units & 7;
        const int ux = q + (x < rem ? 1 : 0), start = x * q + min(x, rem);
        if (k >= ux * a.n_split) return;
        split = k / ux;
        const int u = start + (k - split * ux);
        row_block = u / n_cb;
        cb = u - row_block * n_cb;
    }
    const int row0 = row_block * (WAVES * 32) + wave * 32;
    const int c0 = cb * DVC;
    const int j0 = a.split_tile[split] * kKeyTile;
    const int j1 = min(a.n_keys, a.split_tile[split + 1] * kKeyTile);
    const int ntiles = (j1 - j0 + kKeyTile - 1) / kKeyTile;
    const char* __restrict__ keys = (const char*)a.keys;
    const char* __restrict__ Vt = (const char*)a.Vt;
    const char* __restrict__ kbias = (const char*)a.key_bias;

    // (1) loads.  K: as the LSE kernel (64-chunk slices, swizzled).  V^T:
    // LDS position P = L*64 + lane is row r = P/4 of the tile, stored chunk
    // P%4, fetched from source chunk (P%4) ^ ((r >> 2) & 3); the per-lane
    // offsets do not depend on the tile.  Columns past dv read row dv-1.
    const uint32_t lane16 = (uint32_t)lane * 16u;
    uint32_t voffs[VT_PER_WAVE];
#pragma unroll
    for (int l = 0; l < VT_PER_WAVE; ++l) {
        const int P = (l * WAVES + wave) * 64 + lane;
        const int r = P >> 2, cp = P & 3;
        const int col = min(c0 + r, a.dv - 1);
        voffs[l] = (uint32_t)((int64_t)col * m_pad * 2) + (uint32_t)((cp ^ ((r >> 2) & 3)) * 16);
    }
    auto issue_k = [&](int k, int slot) __attribute__((always_inline)) {
        const char* tbase = keys + (int64_t)(j0 + k * kKeyTile) * ROW_BYTES;
        uint4* dst = kbuf + slot * KT_CHUNKS;
#pragma unroll
        for (int l = 0; l < KT_PER_WAVE; ++l) {
            const int L = l * WAVES + wave;
            if (KT_INSTR % WAVES == 0 || L < KT_INSTR) {
                if constexpr (CPR >= 64) {
                    constexpr int IPR = CPR / 64;
                    const int m = L / IPR;
                    uint32_t sw = (uint32_t)(m & SWZ) * 16u;
                    asm volatile("" : "+s"(sw));
                    dma_to_lds16(tbase + m * ROW_BYTES + (L % IPR) * 1024, lane16 ^ sw,
                                 dst + L * 64);
                } else {
                    const int P = L * 64 + lane;
                    const int m = P / CPR, cp = P % CPR;
                    dma_to_lds16(tbase, (uint32_t)(m * ROW_BYTES + (cp ^ (m & SWZ)) * 16),
                                 dst + L * 64);
                }
            }
        }
        // every wave copies the 32 biases (the same bytes to the same place),
        // so that every wave issues the same number of loads per stage
        if (lane < 8)
            dma_to_lds16(kbias + (int64_t)(j0 + k * kKeyTile) * 4, lane16,
                         bbuf + slot * kKeyTile);
    };
    auto issue_v = [&](int k, int slot) __attribute__((always_inline)) {
        const char* tbase = Vt + (int64_t)(j0 + k * kKeyTile) * 2;
        uint4* dst = vbuf + slot * VT_CHUNKS;
#pragma unroll
        for (int l = 0; l < VT_PER_WAVE; ++l) {
            const int L = l * WAVES + wave;
            if (VT_INSTR % WAVES == 0 || L < VT_INSTR) dma_to_lds16(tbase, voffs[l], dst + L * 64);
        }
    };

    // One stage's loads as NPIECE single instructions (K slices, the biases,
    // V^T slices), so the loop can spread them over its score instructions:
    // a wave's load instructions issued back to back hold up the matrix
    // instructions behind them.
    constexpr int NPIECE = KT_PER_WAVE + 1 + VT_PER_WAVE;
    auto issue_piece = [&](int i, int kt, int kslot, int vt, int vslot)
                           __attribute__((always_inline)) {
        if (i < KT_PER_WAVE) {
            const char* tbase = keys + (int64_t)(j0 + kt * kKeyTile) * ROW_BYTES;
            uint4* dst = kbuf + kslot * KT_CHUNKS;
            const int L = i * WAVES + wave;
            if (KT_INSTR % WAVES == 0 || L < KT_INSTR) {
                if constexpr (CPR >= 64) {
                    constexpr int IPR = CPR / 64;
                    const int m = L / IPR;
                    uint32_t sw = (uint32_t)(m & SWZ) * 16u;
                    asm volatile("" : "+s"(sw));
                    dma_to_lds16(tbase + m * ROW_BYTES + (L % IPR) * 1024, lane16 ^ sw,
                                 dst + L * 64);
                } else {
                    const int P = L * 64 + lane;
                    const int m = P / CPR, cp = P % CPR;
                    dma_to_lds16(tbase, (uint32_t)(m * ROW_BYTES + (cp ^ (m & SWZ)) * 16),
                                 dst + L * 64);
                }
            }
        } else if (i == KT_PER_WAVE) {
            if (lane < 8)
                dma_to_lds16(kbias + (int64_t)(j0 + kt * kKeyTile) * 4, lane16,
                             bbuf + kslot * kKeyTile);
        } else {
            const int l = i - KT_PER_WAVE - 1;
            const int L = l * WAVES + wave;
            if (VT_INSTR % WAVES == 0 || L < VT_INSTR)
                dma_to_lds16(Vt + (int64_t)(j0 + vt * kKeyTile) * 2, voffs[l],
                             vbuf + vslot * VT_CHUNKS + L * 64);
        }
    };

    // the repair pass recomputes only row blocks holding a marked row
    if (a.ref_mode == REF_REPAIR) {
        const int r = row_block * (WAVES * 32) + tid;
        const int fl = tid < WAVES * 32 && r < a.n_rows ? a.row_flag[r] : 0;
        if (!__syncthreads_or(fl)) return;
    }

    // prologue: K tiles 0, 1 (clamped), V^T tile 0, the resident rows
#pragma unroll
    for (int k = 0; k < NB; ++k) issue_k(min(k, ntiles - 1), k);
#pragma unroll
    for (int k = 0; k < NB - 1; ++k) issue_v(min(k, ntiles - 1), k);
    u32x4 q[NG];
    {
        const char* rp = (const char*)a.rows + (int64_t)(row0 + ln) * ROW_BYTES + h * 16;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            q[g] = *(const u32x4*)(rp + g * 32);
            asm volatile("" ::"v"(q[g]));  // waits for these loads stay in the prologue
        }
    }
    const int myrow = row0 + ln;
    // the row's reference (rows past n: +inf makes every weight 0); the
    // repair pass starts from the row's score maximum over all key ranges
    float R = INFINITY;
    if (myrow < a.n_rows) {
        if (a.ref_mode == REF_GIVEN) {
            R = a.row_lse2[myrow] - kRefSlack;
        } else if (a.ref_mode == REF_ONLINE) {
            R = (a.row_nrm[myrow] - a.row_pot[myrow]) * a.c_bias - kRefSlack;
        } else {
            R = -INFINITY;
            for (int sp = 0; sp < a.n_split; ++sp)
                R = fmaxf(R, a.row_max[(int64_t)sp * a.n_rows + myrow]);
            if (!(R > -INFINITY)) R = 0.f;
        }
    }
    asm volatile("" : "+v"(R));  // its load's wait stays in the prologue
    // the lane's weight sum (relative to 2^R) and accumulator maximum
    float S = 0.f, Mraw = -INFINITY;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // (2) scores of the tile in K slot SL (biases in bias slot SL): the key
    // fragments stream from LDS through a ring of AP registers kept ahead of
    // the matrix instruction that consumes them.
    int abase[JB];
#pragma unroll
    for (int j = 0; j < JB; ++j) abase[j] = (ln * CPR + ((2 * j + h) ^ (ln & SWZ))) * 16;
    auto kfrag = [&](const char* kb, int g) __attribute__((always_inline)) -> uint4 {
        return *(const uint4*)(kb + abase[g % JB] + (g / JB) * (2 * JB * 16));
    };
    auto score_begin = [&](int slot, f32x16& acc, uint4 (&av)[AP]) __attribute__((always_inline)) {
        const char* kb = (const char*)(kbuf + slot * KT_CHUNKS);
        const float* bb = bbuf + slot * kKeyTile;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const float4 v = *(const float4*)&bb[8 * qq + 4 * h];
            acc[4 * qq + 0] = v.x;
            acc[4 * qq + 1] = v.y;
            acc[4 * qq + 2] = v.z;
            acc[4 * qq + 3] = v.w;
        }
#pragma unroll
        for (int g = 0; g < AP; ++g) av[g] = kfrag(kb, g);
        if constexpr (VGPR_SCORES) score_seed_wait(acc);
    };
    // fragments [G0, G1) of the tile in K slot `slot`; dma(g) after fragment g
    auto score_steps = [&](int slot, f32x16& acc, uint4 (&av)[AP], auto g0_c, auto g1_c,
                           auto&& dma) __attribute__((always_inline)) {
        constexpr int G0 = decltype(g0_c)::value;
        constexpr int G1 = decltype(g1_c)::value;
        const char* kb = (const char*)(kbuf + slot * KT_CHUNKS);
#pragma unroll
        for (int g = G0; g < G1; ++g) {
            if constexpr (VGPR_SCORES)
                score_step_vgpr<OP>(av[g % AP], q[g], acc);
            else
                acc = score_step<OP>(av[g % AP], __builtin_bit_cast(uint4, q[g]), acc);
            if (g + AP < NG) av[g % AP] = kfrag(kb, g + AP);
            dma(g);
        }
    };
    auto scores = [&](int slot, f32x16& acc) __attribute__((always_inline)) {
        uint4 av[AP];
        score_begin(slot, acc, av);
        score_steps(slot, acc, av, std::integral_constant<int, 0>{},
                    std::integral_constant<int, NG>{}, [](int) {});
    };
    // (3) weights of scores [R0, R1) of a tile
    auto weights = [&](const f32x16& acc, f16x8& p0, f16x8& p1, auto r0_c, auto r1_c)
                       __attribute__((always_inline)) {
        constexpr int R0 = decltype(r0_c)::value;
        constexpr int R1 = decltype(r1_c)::value;
#pragma unroll
        for (int r = R0; r < R1; ++r) {
            const float w = ex2(fmaf(acc[r], a.c_score, -R));
            S += w;
            if (r < 8)
                p0[r] = (_Float16)w;
            else
                p1[r - 8] = (_Float16)w;
        }
    };
    // (4) P.V of a tile against the V^T tile in V slot SL.  Fragment k is the
    // 16-key half k%2 of output block k/2: chunk 2(k%2) + h of V^T row
    // 32(k/2) + ln; a ring of APV fragments runs ahead of the instructions.
    constexpr int NVF = 2 * NBV;
    constexpr int APV = NVF < 4 ? NVF : 4;
    f32x16 u[NBV];
#pragma unroll
    for (int nb = 0; nb < NBV; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) u[nb][r] = 0.f;
    auto vfrag = [&](const char* vb, int k) __attribute__((always_inline)) -> uint4 {
        const int r = (k >> 1) * 32 + ln;
        return *(const uint4*)(vb + (r * 4 + ((2 * (k & 1) + h) ^ ((r >> 2) & 3))) * 16);
    };
    auto pv = [&](int slot, const f16x8& p0, const f16x8& p1) __attribute__((always_inline)) {
        const char* vb = (const char*)(vbuf + slot * VT_CHUNKS);
        uint4 bv[APV];
#pragma unroll
        for (int k = 0; k < APV; ++k) bv[k] = vfrag(vb, k);
#pragma unroll
        for (int k = 0; k < NVF; ++k) {
            u[k >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                (k & 1) ? p1 : p0, __builtin_bit_cast(f16x8, bv[k % APV]), u[k >> 1], 0, 0, 0);
            if (k + APV < NVF) bv[k % APV] = vfrag(vb, k + APV);
        }
    };
    // Pins the order of a stage's two scheduling regions (left alone, the
    // scheduler hoists every LDS read of the region to its top, which needs
    // more registers than the row block and the output blocks leave):
    //   scores + weights: bias and first key reads, then per key fragment its
    //     matrix instruction(s), its refill read, up to 2 vector instructions
    //     and one exponential of the weights;
    //   P.V: the first V^T reads, then per fragment its matrix instruction
    //     and refill read.
    constexpr int MF_PER_FRAG = OP == OP_F32 ? 4 : 1;
    auto pin_scores = [&](auto g0_c, auto g1_c, auto first_c) __attribute__((always_inline)) {
        constexpr int G0 = decltype(g0_c)::value;
        constexpr int G1 = decltype(g1_c)::value;
        if constexpr (decltype(first_c)::value)
            __builtin_amdgcn_sched_group_barrier(0x100, AP + 4, 0);
#pragma unroll
        for (int g = G0; g < G1; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, MF_PER_FRAG, 0);
            if (g + AP < NG) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x400, 1, 0);
        }
    };
    auto pin_pv = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_group_barrier(0x100, APV, 0);
#pragma unroll
        for (int k = 0; k < NVF; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (k + APV < NVF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    };

    // One accumulator set: at the start of stage t it holds the scores of
    // tile t, which move to vector registers (the only copy) before the
    // scores of tile t+1 are seeded into it.  The stage body is the same
    // every time (slots by parity), so the output blocks stay in place
    // across the loop.  The weights of tile t are spread over the score
    // instructions of tile t+1 in four fenced chunks.
    constexpr int CH = NG >= 4 ? NG / 4 : 1;  // fragments per chunk
    using F0 = std::integral_constant<int, 0>;
    using F1 = std::integral_constant<int, (CH < NG ? CH : NG)>;
    using F2 = std::integral_constant<int, (2 * CH < NG ? 2 * CH : NG)>;
    using F3 = std::integral_constant<int, (3 * CH < NG ? 3 * CH : NG)>;
    using F4 = std::integral_constant<int, NG>;
    using W0 = std::integral_constant<int, 0>;
    using W1 = std::integral_constant<int, 4>;
    using W2 = std::integral_constant<int, 8>;
    using W3 = std::integral_constant<int, 12>;
    using W4 = std::integral_constant<int, 16>;
    f32x16 acc;
    scores(0, acc);
    __syncthreads();  // every wave is done with K slot 0 before tile 2 lands there
    // loads one wave issues per stage (bias copy included); waiting until
    // only the current stage's are outstanding lands every older tile
    constexpr int PER_STAGE = (KT_INSTR % WAVES == 0 ? KT_INSTR / WAVES : -1000) + 1 +
                              (VT_INSTR % WAVES == 0 ? VT_INSTR / WAVES : -1000);
    int cs = 0, ns = 1, ls = NB - 1;  // slots of tiles t, t+1 and t+NB-1
    for (int t = 0; t < ntiles; ++t) {
        const int kt = min(t + NB, ntiles - 1), vt = min(t + NB - 1, ntiles - 1);
        const int kslot = cs, vslot = ls;
        // with NPIECE <= NG, piece i goes after score fragment i*NG/NPIECE
        auto dma = [&](int g) __attribute__((always_inline)) {
            if constexpr (VGPR_SCORES && NPIECE <= NG) {
                const int i = (g * NPIECE + NG - 1) / NG;
                if (i < NPIECE && (i * NG) / NPIECE == g) issue_piece(i, kt, kslot, vt, vslot);
            }
        };
        if constexpr (!(VGPR_SCORES && NPIECE <= NG)) {
            issue_k(kt, cs);
            issue_v(vt, ls);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (VGPR_SCORES) score_result_wait(acc);
        f32x16 cur = acc;
        asm volatile("" : "+v"(cur));
#pragma unroll
        for (int r = 0; r < 16; ++r) Mraw = fmaxf(Mraw, cur[r]);
        f16x8 p0, p1;
        uint4 av[AP];
        score_begin(ns, acc, av);
        score_steps(ns, acc, av, F0{}, F1{}, dma);
        weights(cur, p0, p1, W0{}, W1{});
        pin_scores(F0{}, F1{}, std::true_type{});
        __builtin_amdgcn_sched_barrier(0);
        score_steps(ns, acc, av, F1{}, F2{}, dma);
        weights(cur, p0, p1, W1{}, W2{});
        pin_scores(F1{}, F2{}, std::false_type{});
        __builtin_amdgcn_sched_barrier(0);
        score_steps(ns, acc, av, F2{}, F3{}, dma);
        weights(cur, p0, p1, W2{}, W3{});
        pin_scores(F2{}, F3{}, std::false_type{});
        __builtin_amdgcn_sched_barrier(0);
        score_steps(ns, acc, av, F3{}, F4{}, dma);
        weights(cur, p0, p1, W3{}, W4{});
        pin_scores(F3{}, F4{}, std::false_type{});
        __builtin_amdgcn_sched_barrier(0);
        pv(cs, p0, p1);
        pin_pv();
        if constexpr (NB == 3 && PER_STAGE > 0)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER_STAGE) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        stage_barrier();
        ls = cs;
        cs = ns;
        ns = ns + 1 == NB ? 0 : ns + 1;
    }

    // Row factor 2^(R_i + (f_i - A_i) c_bias) [* a_i] * 2^-s, or 1 when the
    // key range is one of several (the merge applies it to the sum, from the
    // references recorded here).
    // both lane halves of a row: the sum in a fixed order, the maximum
    float M;
    {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(S), __float_as_uint(S),
                                                         false, false);
        S = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        const auto mw = __builtin_amdgcn_permlane32_swap(__float_as_uint(Mraw),
                                                         __float_as_uint(Mraw), false, false);
        M = fmaxf(__uint_as_float(mw[0]), __uint_as_float(mw[1])) * a.c_score;
    }
    if (h == 0) {
        float sc = 0.f;
        if (myrow < a.n_rows) {
            if (a.row_ref) {
                const int64_t o = (int64_t)split * a.n_rows + myrow;
                a.row_ref[o] = R;
                a.row_sum[o] = S;
                a.row_max[o] = M;
            }
            if (a.n_split == 1) {
                sc = ex2(R + (a.row_pot[myrow] - a.row_nrm[myrow]) * a.c_bias);
                if (!a.divide_by_a) sc *= a.row_w[myrow];
                sc *= a.v_unscale_dev[0];
                if (a.lse_out) a.lse_out[myrow] = R + lg2(S);
            } else {
                sc = 1.f;
            }
        }
        rowscale[wave][ln] = sc;
    }
    __syncthreads();
    float* out = a.n_split == 1 ? a.U : a.U_part + (int64_t)split * a.part_stride;
    // output register r of lane (ln, h): row 8(r/4) + 4h + (r%4), column ln
#pragma unroll
    for (int nb = 0; nb < NBV; ++nb) {
        const int col = c0 + nb * 32 + ln;
        if (col >= a.dv) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int rr = 8 * (r >> 2) + 4 * h + (r & 3);
            const int row = row0 + rr;
            if (row < a.n_rows) out[(int64_t)row * a.dv + col] = u[nb][r] * rowscale[wave][rr];
        }
    }
}

// ------------------------------------- streaming kernel, 1024-wide rows
// U = P.V for 1024-wide two-byte rows.  Rows this wide leave no room for a
// 32-row resident block next to a wide output block in one wave, so the work
// of a 32-row group is split over a pair of waves (on different SIMDs), as in
// the 1024-wide LSE kernel: wave dh of the pair holds half dh of the
// contraction (512 values of each row, 128 registers) and output columns
// [dh*32*NBV, (dh+1)*32*NBV) of the workgroup's column block (NBV blocks of
// 32 columns in the accumulation registers; 256 at NBV = 16).  Two pairs make
// a 64-row workgroup.
//
// Keys stream in 16-key tiles (so that double-buffered key and V^T tiles fit
// in LDS next to each other).  Per tile each wave forms the partial scores of
// its half with v_mfma_f32_16x16x32 (keys x rows, two 16-row blocks per key
// fragment; the first wave's accumulators are seeded with the key biases),
// the pair exchanges the partials through LDS, and each wave forms the
// weights p = 2^(c_score (own + partner) - L) of all 16 keys x 32 rows.  In
// the score layout lane l holds rows l%16 of both row blocks for keys
// 4(l/16)..+3; one v_permlane16_swap per packed register pair turns that into
// the A layout of v_mfma_f32_32x32x16_f16 (lane l: row l%32, keys
// 8(l/32)..+7), which multiplies the V^T tile of the same 16 keys.
//
// Stage t (K, bias slot t%2 hold tile t; V slot (t-1)%2 holds V^T of tile t-1):
//   the partner's partial of tile t-1 is read; the score instructions of tile
//   t run with the loads of K(t+1), its biases and V^T(t) interleaved (one
//   slice per key fragment); then the weights of tile t-1 and its P.V
//   instructions; the wave's partial of tile t goes to the exchange buffer
//   (and stays in registers); loads waited for, barrier.  A last stage does
//   only the weights and P.V of the last tile.
// LDS: V^T row c (a column of V) holds the tile's 16 keys as two 16-byte
// chunks, stored at c*2 + (half ^ ((c >> 3) & 1)) so that 16 consecutive rows
// hit distinct banks.
//
// NG: 16-byte chunk pairs per operand row (d_pad = 16 NG); the transport uses
// NG = 64, the second-moment form NG <= 32.  MOMENT: the second-moment form
// of the Hessian-vector product, M_i = sum_j P_ij s_ij V_j with
// s_ij = v~_i.y~_j: a second resident row block (a.rows2, the direction rows
// scaled per row into the score type) is multiplied with the same key
// fragments, its partials are exchanged with the scores', and the weights
// become p_ij s_ij.
template <int OP, int NG, int NBV, bool MOMENT>
__global__ __launch_bounds__(256, 1) void transport_wide_kernel(TransportArgs a, int64_t m_pad) {
    constexpr int CPR = 2 * NG;                 // 16-byte chunks per key row
    constexpr int ROW_BYTES = CPR * 16;
    constexpr int KT = 16;                      // keys per tile
    constexpr int KT_CHUNKS = KT * CPR;         // 32 KiB at d_pad 1024
    constexpr int KT_SLICES = KT_CHUNKS / 64;   // slices of 1 KiB
    constexpr int KPW = (KT_SLICES + 3) / 4;    // key slices per wave
    constexpr int SWZ = NG >= 16 ? 15 : NG - 1; // XOR swizzle, within a half row
    constexpr int DVC = 64 * NBV;               // columns per workgroup (both waves of a pair)
    constexpr int VT_CHUNKS = DVC * 2;          // 16 keys x 2 bytes per column
    constexpr int VT_SLICES = VT_CHUNKS / 64;
    constexpr int VT_PER_WAVE = (VT_SLICES + 3) / 4;
    constexpr int KS = NG / 4;                  // 32-value contraction steps per half row
    constexpr int AP = KS < 4 ? KS : 4;         // key fragments in flight
    constexpr int APV = NBV < 4 ? NBV : 4;      // V^T fragments in flight
    constexpr int NP = MOMENT ? 4 : 2;          // exchanged partial blocks per wave
    constexpr int JOBS = KPW + VT_PER_WAVE;     // loads per wave per tile
    static_assert(KS >= 1 && KPW <= 8 && VT_PER_WAVE <= 8, "tile shapes");
    static_assert(!MOMENT || NG <= 32, "two resident blocks fit up to d_pad 512");

    __shared__ __attribute__((aligned(16))) uint4 kbuf[2 * KT_CHUNKS];
    __shared__ __attribute__((aligned(16))) uint4 vbuf[2 * VT_CHUNKS];
    __shared__ __attribute__((aligned(16))) float bbuf[2][KT];
    // [tile parity][row group][wave of the pair][partial block][lane]; blocks
    // 0-1 the scores' row blocks, 2-3 (MOMENT) the direction scores'
    __shared__ __attribute__((aligned(16))) float4 xbuf[2][2][2][NP][64];
    __shared__ float rowscale[64];
    __shared__ float rowref[64];  // each row's final reference (score layout -> P.V layout)

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rg = wave >> 1, dh = wave & 1;
    const int l16 = lane & 15, kg = lane >> 4;  // score layout: row, key group
    const int l32 = lane & 31, hh = lane >> 5;  // P.V layout: row / column, key half
    int row_block, yb;
    xcd_work(row_block, yb);
    const int n_cb = (a.dv + DVC - 1) / DVC;
    const int cb0 = yb % n_cb, split = yb / n_cb;
    const int row0 = row_block * 64 + rg * 32;
    const int c0 = cb0 * DVC;
    const int j0 = split * a.keys_per_split;
    const int j1 = min(a.n_keys, j0 + a.keys_per_split);
    const int ntiles = (j1 - j0 + KT - 1) / KT;
    const char* __restrict__ keys = (const char*)a.keys;
    const char* __restrict__ Vt = (const char*)a.Vt;
    const char* __restrict__ kbias = (const char*)a.key_bias;

    // ---- loads: K slices L = 4l + wave (l < 8), V^T slices 4l + wave (< VT_SLICES)
    const uint32_t lane16 = (uint32_t)lane * 16u;
    // V^T slice L, lane: tile row c = (64 L + lane) / 2, stored chunk lane & 1,
    // which holds key half (lane & 1) ^ ((c >> 3) & 1)
    auto voff = [&](int L) __attribute__((always_inline)) -> uint32_t {
        const int c = 32 * L + (lane >> 1);
        const int kh = (lane & 1) ^ ((c >> 3) & 1);
        const int col = min(c0 + c, a.dv - 1);  // columns past dv: any valid one, unused
        return (uint32_t)col * (uint32_t)(m_pad * 2) + (uint32_t)(kh * 16);
    };
    auto issue_k_slice = [&](int k, int slot, int l) __attribute__((always_inline)) {
        const int L = 4 * l + wave;
        if (KT_SLICES % 4 != 0 && L >= KT_SLICES) return;
        if constexpr (CPR >= 64) {
            // a slice lies in one key row: uniform base, lane chunk ^ (m & SWZ)
            constexpr int IPR = CPR / 64;
            const int m = L / IPR;
            const char* src = keys + (int64_t)(j0 + k * KT + m) * ROW_BYTES + (L % IPR) * 1024;
            uint32_t sw = (uint32_t)(m & SWZ) * 16u;
            asm volatile("" : "+s"(sw));
            dma_to_lds16(src, lane16 ^ sw, kbuf + slot * KT_CHUNKS + L * 64);
        } else {
            // a slice spans 64 / CPR key rows: position P holds chunk
            // (P % CPR) ^ (m & SWZ) of key m = P / CPR
            const int P = L * 64 + lane;
            const int m = P / CPR, cp = P % CPR;
            dma_to_lds16(keys + (int64_t)(j0 + k * KT) * ROW_BYTES,
                         (uint32_t)(m * ROW_BYTES + (cp ^ (m & SWZ)) * 16),
                         kbuf + slot * KT_CHUNKS + L * 64);
        }
    };
    auto issue_v_slice = [&](int k, int slot, int l) __attribute__((always_inline)) {
        const int L = 4 * l + wave;
        if (VT_SLICES % 4 == 0 || L < VT_SLICES)
            dma_to_lds16(Vt + (int64_t)(j0 + k * KT) * 2, voff(L), vbuf + slot * VT_CHUNKS + L * 64);
    };
    auto issue_bias = [&](int k, int slot) __attribute__((always_inline)) {
        if (wave == 0 && lane < 4)
            dma_to_lds16(kbias + (int64_t)(j0 + k * KT) * 4, lane16, &bbuf[slot][0]);
    };
    // the repair pass recomputes only row blocks holding a marked row
    if (a.ref_mode == REF_REPAIR) {
        const int r = row_block * 64 + tid;
        const int fl = tid < 64 && r < a.n_rows ? a.row_flag[r] : 0;
        if (!__syncthreads_or(fl)) return;
    }
    if (ntiles > 0) {
#pragma unroll
        for (int l = 0; l < KPW; ++l) issue_k_slice(0, 0, l);
        issue_bias(0, 0);
    }

    // ---- resident rows: q[rb][ks] = chunk NG dh + 4 ks + kg of row row0 + 16 rb + l16
    // (and the direction rows vq likewise, MOMENT)
    u32x4 q[2][KS], vq[MOMENT ? 2 : 1][MOMENT ? KS : 1];
    {
        const int64_t off = (int64_t)(row0 + l16) * ROW_BYTES + (NG * dh + kg) * 16;
        const char* rp = (const char*)a.rows + off;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) q[rb][ks] = *(const u32x4*)(rp + rb * 16 * ROW_BYTES + ks * 64);
        if constexpr (MOMENT) {
            const char* vp = (const char*)a.rows2 + off;
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    vq[rb][ks] = *(const u32x4*)(vp + rb * 16 * ROW_BYTES + ks * 64);
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                asm volatile("" ::"v"(q[rb][ks]));
                if constexpr (MOMENT) asm volatile("" ::"v"(vq[rb][ks]));
            }
    }
    // each row's reference, as in the streaming kernel (the second-moment
    // form keeps the exact LSE: its weights carry the direction scores too);
    // rows past n: +inf makes every weight 0
    constexpr float slack = MOMENT ? 0.f : kRefSlack;
    float Lr[2], S[2] = {0.f, 0.f}, Mx[2] = {-INFINITY, -INFINITY};
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int row = row0 + 16 * rb + l16;
        float R = INFINITY;
        if (row < a.n_rows) {
            if (a.ref_mode == REF_GIVEN) {
                R = a.row_lse2[row] - slack;
            } else if (a.ref_mode == REF_ONLINE) {
                R = (a.row_nrm[row] - a.row_pot[row]) * a.c_bias - slack;
            } else {
                R = -INFINITY;
                for (int sp = 0; sp < a.n_split; ++sp)
                    R = fmaxf(R, a.row_max[(int64_t)sp * a.n_rows + row]);
                if (!(R > -INFINITY)) R = 0.f;
            }
        }
        Lr[rb] = R;
        asm volatile("" : "+v"(Lr[rb]));
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // key fragment ks of the tile in slot `slot`: chunk NG dh + 4 ks + kg of
    // key l16, stored at l16*CPR + (chunk ^ (l16 & SWZ)) (the XOR stays in
    // the half)
    int kbase[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        kbase[j] = (l16 * CPR + NG * dh + (((4 * j + kg) & (NG - 1)) ^ (l16 & SWZ))) * 16;
    auto kfrag = [&](int slot, int ks) __attribute__((always_inline)) -> uint4 {
        return *(const uint4*)((const char*)kbuf + kbase[ks & 3] + slot * (KT_CHUNKS * 16) +
                               (ks >> 2) * 256);
    };
    // V^T fragment of output block cb (this wave's half): row
    // dh*32*NBV + 32 cb + l32, key half hh
    const int vrow = dh * 32 * NBV + l32;
    const int vbase = (vrow * 2 + (hh ^ ((vrow >> 3) & 1))) * 16;
    auto vfrag = [&](int slot, int cb) __attribute__((always_inline)) -> uint4 {
        return *(const uint4*)((const char*)vbuf + vbase + slot * (VT_CHUNKS * 16) + cb * 1024);
    };

    f32x16 u[NBV];
#pragma unroll
    for (int nb = 0; nb < NBV; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) u[nb][r] = 0.f;

    for (int t = 0; t <= ntiles; ++t) {
        const int cs = t & 1, ps = cs ^ 1;
        if (t < ntiles) {
            // scores of tile t, the loads of the next tiles interleaved
            const int kn = min(t + 1, ntiles - 1);
            f32x4 acc[NP];
            {
                float4 seed = make_float4(0.f, 0.f, 0.f, 0.f);
                if (dh == 0) seed = *(const float4*)&bbuf[cs][4 * kg];
#pragma unroll
                for (int rb = 0; rb < NP; ++rb) {
                    const bool sc = rb < 2;  // score blocks take the key biases
                    acc[rb][0] = sc ? seed.x : 0.f;
                    acc[rb][1] = sc ? seed.y : 0.f;
                    acc[rb][2] = sc ? seed.z : 0.f;
                    acc[rb][3] = sc ? seed.w : 0.f;
                }
            }
            uint4 av[AP];
#pragma unroll
            for (int g = 0; g < AP; ++g) av[g] = kfrag(cs, g);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
                    acc[rb] = mfma16_step<OP>(av[ks % AP], q[rb][ks], acc[rb]);
                if constexpr (MOMENT) {
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb)
                        acc[2 + rb] = mfma16_step<OP>(av[ks % AP], vq[rb][ks], acc[2 + rb]);
                }
                if (ks + AP < KS) av[ks % AP] = kfrag(cs, ks + AP);
                // this step's share of the next tiles' loads
#pragma unroll
                for (int jb = ks * JOBS / KS; jb < (ks + 1) * JOBS / KS; ++jb) {
                    if (jb < KPW)
                        issue_k_slice(kn, ps, jb);
                    else
                        issue_v_slice(t, cs, jb - KPW);
                }
                if (ks == 0) issue_bias(kn, ps);
            }
            // pinned ring order: the seed and first AP reads, then per key
            // fragment its matrix instructions and its refill read
            __builtin_amdgcn_sched_group_barrier(0x100, AP + 1, 0);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                __builtin_amdgcn_sched_group_barrier(0x008, NP, 0);
                if (ks + AP < KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            // this wave's partials of tile t, for both waves of the pair
#pragma unroll
            for (int rb = 0; rb < NP; ++rb)
                xbuf[cs][rg][dh][rb][lane] = make_float4(acc[rb][0], acc[rb][1], acc[rb][2], acc[rb][3]);
        }
        if (t > 0) {
            // weights and P.V of tile t-1 (both partials from the exchange buffer)
            float z[2][4];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const float4 o = xbuf[ps][rg][dh][rb][lane];
                const float4 p = xbuf[ps][rg][dh ^ 1][rb][lane];
                z[rb][0] = o.x + p.x;
                z[rb][1] = o.y + p.y;
                z[rb][2] = o.z + p.z;
                z[rb][3] = o.w + p.w;
            }
            float wt[2][4];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    wt[rb][e] = ex2(fmaf(z[rb][e], a.c_score, -Lr[rb]));
                    if constexpr (!MOMENT) {
                        S[rb] += wt[rb][e];
                        Mx[rb] = fmaxf(Mx[rb], z[rb][e]);
                    }
                }
            if constexpr (MOMENT) {
                // weights p_ij s_ij
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    const float4 o = xbuf[ps][rg][dh][2 + rb][lane];
                    const float4 p = xbuf[ps][rg][dh ^ 1][2 + rb][lane];
                    wt[rb][0] *= o.x + p.x;
                    wt[rb][1] *= o.y + p.y;
                    wt[rb][2] *= o.z + p.z;
                    wt[rb][3] *= o.w + p.w;
                }
            }
            uint32_t x[2], y[2];
#pragma unroll
            for (int hp = 0; hp < 2; ++hp) {
                x[hp] = pack_f16x2(wt[0][2 * hp], wt[0][2 * hp + 1]);
                y[hp] = pack_f16x2(wt[1][2 * hp], wt[1][2 * hp + 1]);
            }
            // lane rows 2i keep row block 0 and take the odd neighbour's
            // row-block-0 keys; rows 2i+1 keep block 1 and take the even
            // neighbour's: afterwards lane l holds row l%32, keys 8(l/32)..+7
            const auto s0 = __builtin_amdgcn_permlane16_swap(x[0], y[0], false, false);
            const auto s1 = __builtin_amdgcn_permlane16_swap(x[1], y[1], false, false);
            uint4 au;
            au.x = s0[0];
            au.y = s1[0];
            au.z = s0[1];
            au.w = s1[1];
            const f16x8 A = __builtin_bit_cast(f16x8, au);
            __builtin_amdgcn_sched_barrier(0);
            uint4 bv[APV];
#pragma unroll
            for (int k = 0; k < APV; ++k) bv[k] = vfrag(ps, k);
#pragma unroll
            for (int k = 0; k < NBV; ++k) {
                u[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, __builtin_bit_cast(f16x8, bv[k % APV]),
                                                            u[k], 0, 0, 0);
                if (k + APV < NBV) bv[k % APV] = vfrag(ps, k + APV);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, APV, 0);
#pragma unroll
            for (int k = 0; k < NBV; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (k + APV < NBV) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        stage_barrier();
    }

    // Each row's weight sum and maximum over the four key groups of its
    // lanes (the same in both waves of the pair, which form the same
    // weights); the records and the reference for the P.V layout from wave
    // dh = 0, key group 0.
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        S[rb] += __shfl_xor(S[rb], 16, 64);
        S[rb] += __shfl_xor(S[rb], 32, 64);
        Mx[rb] = fmaxf(Mx[rb], __shfl_xor(Mx[rb], 16, 64));
        Mx[rb] = fmaxf(Mx[rb], __shfl_xor(Mx[rb], 32, 64));
    }
    if (dh == 0 && kg == 0) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const int rr = 16 * rb + l16, row = row0 + rr;
            rowref[rg * 32 + rr] = Lr[rb];
            if (row < a.n_rows && a.row_ref) {
                const int64_t o = (int64_t)split * a.n_rows + row;
                a.row_ref[o] = Lr[rb];
                a.row_sum[o] = S[rb];
                a.row_max[o] = Mx[rb] * a.c_score;
            }
            if (row < a.n_rows && a.n_split == 1 && a.lse_out) a.lse_out[row] = Lr[rb] + lg2(S[rb]);
        }
    }
    __syncthreads();
    // Row factor 2^(R_i + (f_i - A_i) c_bias) [* a_i] * 2^-s, or 1 when the
    // key range is one of several (the merge applies it to the sum, from the
    // references recorded above).
    if (dh == 0 && hh == 0) {
        const int row = row0 + l32;
        float sc = 0.f;
        if (row < a.n_rows) {
            if (a.n_split == 1) {
                sc = ex2(rowref[rg * 32 + l32] + (a.row_pot[row] - a.row_nrm[row]) * a.c_bias);
                if (!a.divide_by_a) sc *= a.row_w[row];
                sc *= a.v_unscale_dev[0];
            } else {
                sc = 1.f;
            }
        }
        rowscale[rg * 32 + l32] = sc;
    }
    __syncthreads();
    float* out = a.n_split == 1 ? a.U : a.U_part + (int64_t)split * a.part_stride;
    // output register r of lane (l32, hh): row 8(r/4) + 4hh + (r%4), column l32
#pragma unroll
    for (int nb = 0; nb < NBV; ++nb) {
        const int col = c0 + dh * 32 * NBV + nb * 32 + l32;
        if (col >= a.dv) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int rr = 8 * (r >> 2) + 4 * hh + (r & 3);
            const int row = row0 + rr;
            if (row < a.n_rows) out[(int64_t)row * a.dv + col] = u[nb][r] * rowscale[rg * 32 + rr];
        }
    }
}

// U = (sum over key ranges of the partial products, in range order, each
// brought to the largest of the ranges' references Rb) times the row factor
// 2^(Rb + (f_i - A_i) c_bias) [* a_i] * 2^-s.  Kernels that record no
// references (row_ref NULL) weighted every range against row_lse2.  With
// lse_out, column 0 also writes the row's LSE2, Rb + log2(sum of the ranges'
// weight sums brought to Rb).
// Grid: x = groups of 256/tpr rows, y = blocks of 4*tpr columns; tpr threads
// per row, each 4 columns (16-byte accesses when every row starts 16-byte
// aligned).  The row's range factors and scale are computed once per thread.
__global__ __launch_bounds__(256) void transport_merge_kernel(TransportArgs a, int tpr) {
    const int row = blockIdx.x * (256 / tpr) + threadIdx.x / tpr;
    if (row >= a.n_rows) return;
    const int t = threadIdx.x % tpr;
    float fac[kTransportMaxSplit];
    float Rb;
    if (a.row_ref) {
        Rb = -INFINITY;
        for (int s = 0; s < a.n_split; ++s) Rb = fmaxf(Rb, a.row_ref[(int64_t)s * a.n_rows + row]);
        for (int s = 0; s < a.n_split; ++s) fac[s] = ex2(a.row_ref[(int64_t)s * a.n_rows + row] - Rb);
        if (a.lse_out && blockIdx.y == 0 && t == 0) {
            float T = 0.f;
            for (int s = 0; s < a.n_split; ++s) T += a.row_sum[(int64_t)s * a.n_rows + row] * fac[s];
            a.lse_out[row] = Rb + lg2(T);
        }
    } else {
        Rb = a.row_lse2[row];
        for (int s = 0; s < a.n_split; ++s) fac[s] = 1.f;
    }
    float sc = ex2(Rb + (a.row_pot[row] - a.row_nrm[row]) * a.c_bias);
    if (!a.divide_by_a) sc *= a.row_w[row];
    sc *= a.v_unscale_dev[0];
    const int c = (blockIdx.y * tpr + t) * 4;
    if (c >= a.dv) return;
    const int64_t base = (int64_t)row * a.dv + c;
    const bool vec = (a.dv & 3) == 0 && (((uintptr_t)a.U | (uintptr_t)a.U_part) & 15) == 0;
    if (vec) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int s = 0; s < a.n_split; ++s) {
            const float4 v = *(const float4*)(a.U_part + (int64_t)s * a.part_stride + base);
            acc.x += v.x * fac[s];
            acc.y += v.y * fac[s];
            acc.z += v.z * fac[s];
            acc.w += v.w * fac[s];
        }
        *(float4*)(a.U + base) = make_float4(acc.x * sc, acc.y * sc, acc.z * sc, acc.w * sc);
    } else {
        for (int k = 0; k < 4 && c + k < a.dv; ++k) {
            float acc = 0.f;
            for (int s = 0; s < a.n_split; ++s)
                acc += a.U_part[(int64_t)s * a.part_stride + base + k] * fac[s];
            a.U[base + k] = acc * sc;
        }
    }
}

// Marks the rows whose first-pass weights may be wrong: a weight above
// 2^kMaxOver (near the float16 limit) in some key range, or weights too small
// for their rounding -- float16 errs by at most 2^-12 of a weight, or 2^-25
// absolutely where the weight is subnormal, so the absolute bound, m_s
// 2^(R_s - 25) summed over the key ranges, is compared with the relative
// one, 2^-13 of the row's weight sum.  Only a row potential far from its
// update's value (the reference taken from it far from the row's LSE2) trips
// either.
__global__ __launch_bounds__(256) void transport_flag_kernel(TransportArgs a) {
    const int row = blockIdx.x * 256 + threadIdx.x;
    if (row >= a.n_rows) return;
    float Rb = -INFINITY;
    bool over = false;
    for (int s = 0; s < a.n_split; ++s) {
        const int64_t o = (int64_t)s * a.n_rows + row;
        Rb = fmaxf(Rb, a.row_ref[o]);
        over = over || a.row_max[o] > a.row_ref[o] + kMaxOver;
    }
    float T = 0.f, E = 0.f;
    for (int s = 0; s < a.n_split; ++s) {
        const int64_t o = (int64_t)s * a.n_rows + row;
        const float fac = ex2(a.row_ref[o] - Rb);
        const int ms = min(a.n_keys, a.split_tile[s + 1] * kKeyTile) - a.split_tile[s] * kKeyTile;
        T += a.row_sum[o] * fac;
        E += (float)ms * fac;
    }
    a.row_flag[row] = (!over && E <= 4096.f * T) ? 0 : 1;
}

template <int D, int DVC>
hipError_t transport_valu_launch_c(const TransportArgs& a, hipStream_t s) {
    // rows per thread: as many as the output registers allow, fewer when
    // that would leave the GPU short of workgroups
    constexpr int RMAX = DVC <= 8 ? 4 : (DVC == 16 ? 2 : 1);
    const int n_cb = (a.dv + DVC - 1) / DVC;
    if (RMAX > 1 && (int64_t)((a.n_rows + 256 * RMAX - 1) / (256 * RMAX)) * n_cb >= 1024) {
        const dim3 grid((a.n_rows + 256 * RMAX - 1) / (256 * RMAX), n_cb);
        transport_valu_kernel<D, RMAX, DVC><<<grid, 256, 0, s>>>(a);
    } else {
        const dim3 grid((a.n_rows + 255) / 256, n_cb);
        transport_valu_kernel<D, 1, DVC><<<grid, 256, 0, s>>>(a);
    }
    return hipGetLastError();
}

template <int D>
hipError_t transport_valu_launch(const TransportArgs& a, hipStream_t s) {
    if (a.dv <= 1) return transport_valu_launch_c<D, 1>(a, s);
    if (a.dv <= 2) return transport_valu_launch_c<D, 2>(a, s);
    if (a.dv <= 4) return transport_valu_launch_c<D, 4>(a, s);
    if (a.dv <= 8) return transport_valu_launch_c<D, 8>(a, s);
    if (a.dv <= 16) return transport_valu_launch_c<D, 16>(a, s);
    return transport_valu_launch_c<D, 32>(a, s);
}

template <int OP, int NG>
hipError_t transport_mfma_launch(const TransportArgs& a, int64_t m_pad, hipStream_t s) {
    // output columns per workgroup: 256 (128 when the resident block is 256 VGPRs)
    constexpr int NB = NG >= 64 ? 4 : 8;
    const dim3 grid((a.n_rows + 127) / 128, (a.dv + 32 * NB - 1) / (32 * NB));
    transport_mfma_kernel<OP, NG, NB><<<grid, 256, 0, s>>>(a, m_pad);
    return hipGetLastError();
}

template <int OP>
hipError_t transport_mfma_dispatch(int ng, const TransportArgs& a, int64_t m_pad, hipStream_t s) {
    switch (ng) {
        case 1: return transport_mfma_launch<OP, 1>(a, m_pad, s);
        case 2: return transport_mfma_launch<OP, 2>(a, m_pad, s);
        case 4: return transport_mfma_launch<OP, 4>(a, m_pad, s);
        case 8: return transport_mfma_launch<OP, 8>(a, m_pad, s);
        case 16: return transport_mfma_launch<OP, 16>(a, m_pad, s);
        case 32: return transport_mfma_launch<OP, 32>(a, m_pad, s);
        case 64: return transport_mfma_launch<OP, 64>(a, m_pad, s);
        default: return hipErrorInvalidValue;
    }
}

template <int OP, int NG, int NBV>
hipError_t transport_stream_launch(const TransportArgs& a, int64_t m_pad, hipStream_t s) {
    // n_units = row blocks x column blocks (set by the planner for this NBV)
    const int64_t blocks = 8 * (int64_t)((a.n_units + 7) / 8) * a.n_split;
    transport_stream_kernel<OP, NG, NBV><<<(unsigned)blocks, 256, 0, s>>>(a, m_pad);
    return hipGetLastError();
}

// output blocks per wave of the streaming kernel: 4 up to 128 columns, else
// 8, or 16 (all 512 columns of a wide V in one block, so the scores are
// formed once) where the row block leaves room for them
constexpr int stream_nbv(int ng, int dv) { return dv <= 128 ? 4 : (dv <= 256 || ng < 16) ? 8 : 16; }

template <int OP, int NG>
hipError_t transport_stream_nbv(const TransportArgs& a, int64_t m_pad, hipStream_t s) {
    if constexpr (NG >= 16)
        if (stream_nbv(NG, a.dv) == 16) return transport_stream_launch<OP, NG, 16>(a, m_pad, s);
    return a.dv <= 128 ? transport_stream_launch<OP, NG, 4>(a, m_pad, s)
                       : transport_stream_launch<OP, NG, 8>(a, m_pad, s);
}

// output blocks per wave of the 1024-wide kernel: the fewest that cover dv
// in one column block (16: 1024 columns per workgroup)
int wide_nbv(int dv) { return dv <= 64 ? 1 : dv <= 128 ? 2 : dv <= 256 ? 4 : dv <= 512 ? 8 : 16; }

template <int OP, int NG, int NBV, bool MOMENT>
hipError_t transport_wide_launch(const TransportArgs& a, int64_t m_pad, hipStream_t s) {
    const int n_cb = (a.dv + 64 * NBV - 1) / (64 * NBV);
    const dim3 grid((a.n_rows + 63) / 64, n_cb * a.n_split);
    transport_wide_kernel<OP, NG, NBV, MOMENT><<<grid, 256, 0, s>>>(a, m_pad);
    return hipGetLastError();
}

template <int OP, int NG, bool MOMENT>
hipError_t transport_wide_nbv(const TransportArgs& a, int64_t m_pad, hipStream_t s) {
    switch (wide_nbv(a.dv)) {
        case 1: return transport_wide_launch<OP, NG, 1, MOMENT>(a, m_pad, s);
        case 2: return transport_wide_launch<OP, NG, 2, MOMENT>(a, m_pad, s);
        case 4: return transport_wide_launch<OP, NG, 4, MOMENT>(a, m_pad, s);
        case 8: return transport_wide_launch<OP, NG, 8, MOMENT>(a, m_pad, s);
        default: return transport_wide_launch<OP, NG, 16, MOMENT>(a, m_pad, s);
    }
}

template <int OP>
hipError_t transport_wide_dispatch(const TransportArgs& a, int64_t m_pad, hipStream_t s) {
    return transport_wide_nbv<OP, 64, false>(a, m_pad, s);
}

// second-moment form: d_pad = 16 NG in {64, 128, 256, 512}, dv <= 512 (the
// accumulation registers hold the direction block next to the scores')
template <int OP>
hipError_t transport_moment_dispatch(int ng, const TransportArgs& a, int64_t m_pad,
                                     hipStream_t s) {
    if (a.dv > 512) return hipErrorInvalidValue;
    switch (ng) {
        case 4: return transport_wide_nbv<OP, 4, true>(a, m_pad, s);
        case 8: return transport_wide_nbv<OP, 8, true>(a, m_pad, s);
        case 16: return transport_wide_nbv<OP, 16, true>(a, m_pad, s);
        case 32: return transport_wide_nbv<OP, 32, true>(a, m_pad, s);
        default: return hipErrorInvalidValue;
    }
}

template <int OP>
hipError_t transport_stream_dispatch(int ng, const TransportArgs& a, int64_t m_pad,
                                     hipStream_t s) {
    switch (ng) {
        case 1: return transport_stream_nbv<OP, 1>(a, m_pad, s);
        case 2: return transport_stream_nbv<OP, 2>(a, m_pad, s);
        case 4: return transport_stream_nbv<OP, 4>(a, m_pad, s);
        case 8: return transport_stream_nbv<OP, 8>(a, m_pad, s);
        case 16: return transport_stream_nbv<OP, 16>(a, m_pad, s);
        case 32: return transport_stream_nbv<OP, 32>(a, m_pad, s);
        default: return hipErrorInvalidValue;
    }
}

// Key-range splits of the streaming kernel: the count whose workgroups
// (row blocks x column blocks x splits) fill the compute units in whole
// rounds best, charging each workgroup a fixed start-up of 8 tiles and each
// extra range the traffic of its partial product (written once, read once).
void transport_split(const TransportArgs& a, bool wide, int ng, int max_split, int& S, int& kps) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    const int rpb = wide ? 64 : 128;
    const int cpb = wide ? 64 * wide_nbv(a.dv) : 32 * stream_nbv(ng, a.dv);
    const int64_t wg = (int64_t)((a.n_rows + rpb - 1) / rpb) * ((a.dv + cpb - 1) / cpb);
    const int64_t m_tiles = (a.n_keys + kKeyTile - 1) / kKeyTile;
    // one tile-stage of a workgroup ~ 1 us; partial traffic at ~4 bytes/ps
    double best = 1e300;
    S = 1;
    kps = (int)(m_tiles * kKeyTile);
    for (int s = 1; s <= max_split && s <= m_tiles; ++s) {
        const int64_t tiles = (m_tiles + s - 1) / s;
        if ((s - 1) * tiles >= m_tiles) continue;  // every range holds a key
        const int64_t rounds = (wg * s + cus - 1) / cus;
        double t = (double)rounds * (double)(tiles + 8);
        if (s > 1) t += (double)(s + 1) * a.n_rows * (double)a.dv * 4.0 / 4e6;
        if (t < best - 1e-9) {
            best = t;
            S = s;
            kps = (int)(tiles * kKeyTile);
        }
    }
}

// Makespan, in tiles, of one XCD of c compute units that runs ux work units
// in each of the s key ranges (sizes[] tiles each, longest first), every
// workgroup taking the next item as a unit frees up, plus a start-up of
// `overhead` tiles per workgroup.
double xcd_makespan(int ux, int c, const int* sizes, int s, int overhead) {
    std::vector<double> heap((size_t)c, 0.0);
    for (int r = 0; r < s; ++r)
        for (int i = 0; i < ux; ++i) {
            std::pop_heap(heap.begin(), heap.end(), std::greater<double>());
            heap.back() += sizes[r] + overhead;
            std::push_heap(heap.begin(), heap.end(), std::greater<double>());
        }
    return *std::max_element(heap.begin(), heap.end());
}

// Key ranges of the streaming kernel: up to kTransportMaxSplit ranges of
// unequal length (longest first) chosen by simulating the fullest XCD's
// schedule (xcd_makespan), charging each extra range its partial product's
// traffic (written once, read once at ~4 TB/s) in tile times of this kernel
// (one 32-key tile of a 128-row block at about half the matrix peak and
// 2 GHz).  Candidates: 1 to 4 equal ranges, and two and three unequal ones
// on a coarse grid refined around its best point.
void stream_ranges(TransportArgs& a, int ng, int nbv, bool f32) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    const int c = std::max(1, cus / 8);
    const int n_cb = (a.dv + 32 * nbv - 1) / (32 * nbv);
    a.n_units = ((a.n_rows + 127) / 128) * n_cb;
    const int ux = (a.n_units + 7) / 8;
    const int m = (a.n_keys + kKeyTile - 1) / kKeyTile;
    const double dpe = f32 ? 8.0 * ng : 16.0 * ng;
    const double tile_flops = 128.0 * kKeyTile * 2.0 * (dpe + 32.0 * nbv);
    const double flops_per_us = (f32 ? 256.0 : 4096.0) * 0.5 * 2.0e3;
    const double tile_us = tile_flops / flops_per_us;
    const double range_tiles = (double)a.n_rows * a.dv * 4.0 / 4.0e6 / tile_us;
    double best = 1e300;
    int bs = 1, bsz[kTransportMaxSplit] = {m, 0, 0, 0};
    auto consider = [&](const int* sz, int s) {
        for (int r = 0; r < s; ++r)
            if (sz[r] < 1 || (r > 0 && sz[r] > sz[r - 1])) return;
        const double t = xcd_makespan(ux, c, sz, s, 8) + (s > 1 ? (s + 1) * range_tiles : 0.0);
        if (t < best - 1e-9) {
            best = t;
            bs = s;
            for (int r = 0; r < s; ++r) bsz[r] = sz[r];
        }
    };
    for (int s = 1; s <= kTransportMaxSplit && s <= m; ++s) {
        int sz[kTransportMaxSplit];
        const int per = (m + s - 1) / s;
        for (int r = 0; r < s; ++r) sz[r] = std::min(per, m - r * per);
        consider(sz, s);
    }
    if (m >= 2) {
        const int st = std::max(1, m / 64);
        for (int x = (m + 1) / 2; x < m; x += st) {
            const int sz[2] = {x, m - x};
            consider(sz, 2);
        }
    }
    if (m >= 3) {
        auto grid3 = [&](int a0, int a1, int b0, int b1, int st) {
            for (int x = std::max(1, a0); x <= std::min(m - 2, a1); x += st)
                for (int y = std::max(1, b0); y <= std::min(x, b1); y += st) {
                    const int sz[3] = {x, y, m - x - y};
                    consider(sz, 3);
                }
        };
        const int st = std::max(1, m / 24);
        grid3((m + 2) / 3, m - 2, 1, m, st);
        if (bs == 3) {
            const int x = bsz[0], y = bsz[1], f = std::max(1, st / 4);
            grid3(x - st, x + st, y - st, y + st, f);
        }
    }
    a.n_split = bs;
    a.split_tile[0] = 0;
    for (int r = 0; r < bs; ++r) a.split_tile[r + 1] = a.split_tile[r] + bsz[r];
    for (int r = bs + 1; r <= kTransportMaxSplit; ++r) a.split_tile[r] = m;
    a.keys_per_split = bsz[0] * kKeyTile;
}

}  // namespace

namespace {
// the 1024-wide kernel: two-byte scores, 1024-value rows, and V^T offsets
// (column x padded key count) within a load's 32-bit offset
bool transport_wide(int path, int dp, int dv, int64_t m_pad) {
    return (path == PATH_MFMA_BF16 || path == PATH_MFMA_F16) && dp == 1024 &&
           (int64_t)dv * m_pad * 2 < ((int64_t)1 << 32);
}
}  // namespace

bool transport_streams(int path, int dp) {
    if (small_d_path(path)) return false;
    const int ng = path == PATH_MFMA_F32 ? dp / 8 : dp / 16;
    return ng <= 32 || ((path == PATH_MFMA_BF16 || path == PATH_MFMA_F16) && ng == 64);
}

bool transport_online(int path, int dp, int dv, int64_t m_pad, bool moment) {
    return !moment && transport_streams(path, dp) &&
           (dp < 1024 || transport_wide(path, dp, dv, m_pad));
}

hipError_t launch_transport(int path, const TransportArgs& a0, float* scratch, void* Vt_buf,
                            int64_t m_pad, float* key_bias_buf, float* part_buf, float* ref_buf,
                            hipStream_t s) {
    TransportArgs a = a0;
    if (a.ref_mode != REF_GIVEN && !transport_online(path, a.dp, a.dv, m_pad, a.rows2 != nullptr))
        return hipErrorInvalidValue;
    if (small_d_path(path)) {
        switch (a.dp) {
            case 1: return transport_valu_launch<1>(a, s);
            case 2: return transport_valu_launch<2>(a, s);
            case 3: return transport_valu_launch<3>(a, s);
            case 4: return transport_valu_launch<4>(a, s);
            case 5: return transport_valu_launch<5>(a, s);
            case 6: return transport_valu_launch<6>(a, s);
            case 7: return transport_valu_launch<7>(a, s);
            case 8: return transport_valu_launch<8>(a, s);
            default: return hipErrorInvalidValue;
        }
    }
    // scratch: [0..1] scale pair, [2] max bits
    unsigned* maxbits = (unsigned*)(scratch + 2);
    hipError_t e = launch_fill(scratch + 2, 1, 0.f, s);
    if (e != hipSuccess) return e;
    const int64_t count = (int64_t)a.n_keys * a.dv;
    const int64_t blocks = std::min<int64_t>((count + 255) / 256, 2048);
    vmax_kernel<<<(unsigned)blocks, 256, 0, s>>>(a.V, count, a.dv, a.v_rscale, a.v_off, maxbits);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    vscale_kernel<<<1, 64, 0, s>>>(maxbits, scratch);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const bool moment = a.rows2 != nullptr;
    if (moment && !((path == PATH_MFMA_BF16 || path == PATH_MFMA_F16) && a.dp >= 64 &&
                    a.dp <= 512 && a.dv <= 512 && (int64_t)a.dv * m_pad * 2 < ((int64_t)1 << 32)))
        return hipErrorInvalidValue;
    const bool wide = moment || transport_wide(path, a.dp, a.dv, m_pad);
    const bool streams = moment || (transport_streams(path, a.dp) && (a.dp < 1024 || wide));
    {
        const dim3 grid((unsigned)((m_pad + 31) / 32), (a.dv + 31) / 32);
        transpose_v_kernel<<<grid, 256, 0, s>>>(a.V, a.n_keys, m_pad, a.dv, scratch,
                                                (_Float16*)Vt_buf, streams && !wide ? 1 : 0, a.v_rscale,
                                                a.v_off);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    a.Vt = Vt_buf;
    a.v_unscale_dev = scratch + 1;
    const int ng = path == PATH_MFMA_F32 ? a.dp / 8 : a.dp / 16;
    if (streams) {
        if (!key_bias_buf || !part_buf) return hipErrorInvalidValue;
        key_bias_kernel<<<(unsigned)((m_pad + 255) / 256), 256, 0, s>>>(a, m_pad, key_bias_buf);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        a.key_bias = key_bias_buf;
        a.U_part = part_buf;
        a.part_stride = (int64_t)a.n_rows * a.dv;
        if (wide) {
            transport_split(a, wide, ng, kTransportMaxSplit, a.n_split, a.keys_per_split);
            // equal ranges (for the check kernel's key counts)
            for (int r = 0; r <= kTransportMaxSplit; ++r)
                a.split_tile[r] = std::min(r, a.n_split) * (a.keys_per_split / kKeyTile);
        } else {
            stream_ranges(a, ng, stream_nbv(ng, a.dv), path == PATH_MFMA_F32);
        }
        // the streaming kernel records its references; the others weight
        // against row_lse2 as given
        const bool own_ref = !moment && ref_buf != nullptr;
        if (own_ref) {
            const int64_t nr = (int64_t)kTransportMaxSplit * a.n_rows;
            a.row_ref = ref_buf;
            a.row_sum = ref_buf + nr;
            a.row_max = ref_buf + 2 * nr;
            a.row_flag = (int*)(ref_buf + 3 * nr);
        } else {
            if (a.ref_mode != REF_GIVEN) return hipErrorInvalidValue;
            a.row_ref = a.row_sum = a.row_max = nullptr;
            a.row_flag = nullptr;
            a.lse_out = nullptr;
        }
        {
            auto pass = [&](const TransportArgs& t) {
                if (moment)
                    return path == PATH_MFMA_BF16
                               ? transport_moment_dispatch<OP_BF16>(ng, t, m_pad, s)
                               : transport_moment_dispatch<OP_F16>(ng, t, m_pad, s);
                if (wide)
                    return path == PATH_MFMA_BF16 ? transport_wide_dispatch<OP_BF16>(t, m_pad, s)
                                                  : transport_wide_dispatch<OP_F16>(t, m_pad, s);
                if (path == PATH_MFMA_F32) return transport_stream_dispatch<OP_F32>(ng, t, m_pad, s);
                if (path == PATH_MFMA_BF16) return transport_stream_dispatch<OP_BF16>(ng, t, m_pad, s);
                return transport_stream_dispatch<OP_F16>(ng, t, m_pad, s);
            };
            e = pass(a);
            if (e == hipSuccess && a.ref_mode == REF_ONLINE) {
                // mark the rows whose weights came out too small, then
                // recompute their row blocks from the score maxima
                transport_flag_kernel<<<(unsigned)((a.n_rows + 255) / 256), 256, 0, s>>>(a);
                if ((e = hipGetLastError()) != hipSuccess) return e;
                TransportArgs r = a;
                r.ref_mode = REF_REPAIR;
                e = pass(r);
            }
        }
        if (e != hipSuccess || a.n_split == 1) return e;
        const int tpr = a.dv <= 256 ? 64 : (a.dv <= 512 ? 128 : 256);
        const dim3 mgrid((unsigned)((a.n_rows + 256 / tpr - 1) / (256 / tpr)),
                         (unsigned)((a.dv + 4 * tpr - 1) / (4 * tpr)));
        transport_merge_kernel<<<mgrid, 256, 0, s>>>(a, tpr);
        return hipGetLastError();
    }
    if (path == PATH_MFMA_F32) return transport_mfma_dispatch<OP_F32>(ng, a, m_pad, s);
    if (path == PATH_MFMA_BF16) return transport_mfma_dispatch<OP_BF16>(ng, a, m_pad, s);
    if (path == PATH_MFMA_F16) return transport_mfma_dispatch<OP_F16>(ng, a, m_pad, s);
    return hipErrorInvalidValue;
}

}  // namespace fs
