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
//     P_ij = a_i 2^(z2_ij - L_i) 2^(L_i + (f_i - |x~_i|^2) c_bias),
// where L_i = log2 sum_j 2^(z2_ij) is the exact row LSE, computed first by one
// streaming LSE pass.  The weights p_ij = 2^(z2_ij - L_i) lie in (0, 1] and
// sum to 1 over j, so they are well scaled for a float16 product; the row
// factor is applied once at the end.
//
// Matrix-core kernel: per 32-key tile the score MFMAs of the LSE kernel give,
// in each lane, 16 weights of ONE row; they are packed to f16 and used
// directly as the A operand of v_mfma_f32_32x32x16_f16 against a transposed
// f16 copy of V (keys on the contraction axis, in the same slot order), so
// the weights never leave registers.  V is copied once, transposed and scaled
// by a power of two into the f16 range; the scale is undone exactly at the end.
#include <algorithm>

#include "fs_device.hpp"
#include "fs_internal.h"

namespace fs {

namespace {

// ---------------------------------------------------- V -> f16, transposed
// max|V| over all entries as the bit pattern of a non-negative float (for
// which integer order is float order), so an atomic max is order independent.
__global__ __launch_bounds__(256) void vmax_kernel(const float* __restrict__ V, int64_t count,
                                                   unsigned* __restrict__ maxbits) {
    __shared__ float red[256];
    float mx = 0.f;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < count; k += stride)
        mx = fmaxf(mx, fabsf(V[k]));
    red[threadIdx.x] = mx;
    __syncthreads();
    for (int o = 128; o >= 1; o >>= 1) {
        if (threadIdx.x < o) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
        __syncthreads();
    }
    if (threadIdx.x == 0) atomicMax(maxbits, __float_as_uint(red[0]));
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

// Vt[k][j] = f16(V[j][k] * 2^s) for j < m, 0 for m <= j < m_pad.
__global__ __launch_bounds__(256) void transpose_v_kernel(const float* __restrict__ V, int m,
                                                          int64_t m_pad, int dv,
                                                          const float* __restrict__ scratch,
                                                          _Float16* __restrict__ Vt) {
    __shared__ float tile[32][33];
    const float sc = scratch[0];
    const int j0 = blockIdx.x * 32, k0 = blockIdx.y * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
    for (int yy = ty; yy < 32; yy += 8) {
        const int j = j0 + yy, k = k0 + tx;
        tile[yy][tx] = (j < m && k < dv) ? V[(int64_t)j * dv + k] * sc : 0.f;
    }
    __syncthreads();
    for (int yy = ty; yy < 32; yy += 8) {
        const int k = k0 + yy, j = j0 + tx;
        if (k < dv && j < m_pad) Vt[(int64_t)k * m_pad + j] = (_Float16)tile[tx][yy];
    }
}

// ------------------------------------------------------------ vector path
// One row per thread, 32 output columns per thread (grid.y over dv chunks).
template <int D>
__global__ __launch_bounds__(256) void transport_valu_kernel(TransportArgs a) {
    constexpr int DP = D <= 4 ? 4 : 8;
    constexpr int DVC = 32;
    const float* __restrict__ rows = (const float*)a.rows;
    const float* __restrict__ keys = (const float*)a.keys;
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int c0 = blockIdx.y * DVC;
    const bool live = i < a.n_rows;
    float x[D];
#pragma unroll
    for (int k = 0; k < D; ++k) x[k] = live ? rows[(int64_t)i * DP + k] * a.c_score : 0.f;
    const float L = live ? a.row_lse2[i] : 0.f;
    float u[DVC];
#pragma unroll
    for (int c = 0; c < DVC; ++c) u[c] = 0.f;
    for (int j = 0; j < a.n_keys; ++j) {
        float z = fmaf(a.key_pot[j] - a.key_nrm[j], a.c_bias, a.key_lw2[j]);
#pragma unroll
        for (int k = 0; k < D; ++k) z = fmaf(x[k], keys[(int64_t)j * DP + k], z);
        const float p = ex2(z - L);
        const float* vr = a.V + (int64_t)j * a.dv + c0;
#pragma unroll
        for (int c = 0; c < DVC; ++c)
            if (c0 + c < a.dv) u[c] = fmaf(p, vr[c], u[c]);
    }
    if (!live) return;
    float sc = ex2(L + (a.row_pot[i] - a.row_nrm[i]) * a.c_bias);
    if (!a.divide_by_a) sc *= a.row_w[i];
    float* ur = a.U + (int64_t)i * a.dv + c0;
#pragma unroll
    for (int c = 0; c < DVC; ++c)
        if (c0 + c < a.dv) ur[c] = u[c] * sc;
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

template <int D>
hipError_t transport_valu_launch(const TransportArgs& a, hipStream_t s) {
    const dim3 grid((a.n_rows + 255) / 256, (a.dv + 31) / 32);
    transport_valu_kernel<D><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
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

}  // namespace

hipError_t launch_transport(int path, const TransportArgs& a0, float* scratch, void* Vt_buf,
                            int64_t m_pad, hipStream_t s) {
    TransportArgs a = a0;
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
    vmax_kernel<<<(unsigned)blocks, 256, 0, s>>>(a.V, count, maxbits);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    vscale_kernel<<<1, 64, 0, s>>>(maxbits, scratch);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    {
        const dim3 grid((unsigned)((m_pad + 31) / 32), (a.dv + 31) / 32);
        transpose_v_kernel<<<grid, 256, 0, s>>>(a.V, a.n_keys, m_pad, a.dv, scratch,
                                                (_Float16*)Vt_buf);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    a.Vt = Vt_buf;
    a.v_unscale_dev = scratch + 1;
    const int ng = path == PATH_MFMA_F32 ? a.dp / 8 : a.dp / 16;
    if (path == PATH_MFMA_F32) return transport_mfma_dispatch<OP_F32>(ng, a, m_pad, s);
    if (path == PATH_MFMA_BF16) return transport_mfma_dispatch<OP_BF16>(ng, a, m_pad, s);
    if (path == PATH_MFMA_F16) return transport_mfma_dispatch<OP_F16>(ng, a, m_pad, s);
    return hipErrorInvalidValue;
}

}  // namespace fs
