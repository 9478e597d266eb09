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
#include "fs_device.hpp"
#include "fs_internal.h"

namespace fs {

namespace {

// ---------------------------------------------------- V -> f16, transposed
// scratch[0] = 2^s, scratch[1] = 2^-s, with s chosen so max|V| 2^s <= 2^14.
__global__ __launch_bounds__(256) void vmax_kernel(const float* __restrict__ V, int64_t count,
                                                   float* __restrict__ scratch) {
    __shared__ float red[256];
    float mx = 0.f;
    for (int64_t k = threadIdx.x; k < count; k += 256) mx = fmaxf(mx, fabsf(V[k]));
    red[threadIdx.x] = mx;
    __syncthreads();
    for (int o = 128; o >= 1; o >>= 1) {
        if (threadIdx.x < o) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const float m = red[0];
        int s = 0;
        if (m > 0.f && m <= 3.402823466e38f) {
            int e;
            frexpf(m, &e);  // m in [2^(e-1), 2^e)
            s = 14 - e;     // m 2^s < 2^14
            s = s > 100 ? 100 : (s < -100 ? -100 : s);
        }
        scratch[0] = ldexpf(1.f, s);
        scratch[1] = ldexpf(1.f, -s);
    }
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

constexpr int kVtStride = 36;  // f16 elements per LDS row of the V^T tile (32 keys + pad)

// Each wave: 32 rows; workgroup: 128 rows x (32*NB) output columns starting
// at column blockIdx.y * 32 * NB.
template <int OP, int NG, int NB>
__global__ __launch_bounds__(256, 1) void transport_mfma_kernel(TransportArgs a) {
    constexpr int CPR = 2 * NG;
    constexpr int ROW_BYTES = CPR * 16;
    constexpr int TILE_CHUNKS = kKeyTile * CPR;
    constexpr int LOADS = (TILE_CHUNKS + 255) / 256;
    constexpr int SWZ = CPR >= 8 ? 7 : CPR - 1;
    constexpr int DVC = 32 * NB;                          // output columns per workgroup
    constexpr int VT_ELEMS = DVC * kKeyTile;              // f16 values of one V^T tile
    constexpr int VLOADS = (VT_ELEMS / 8 + 255) / 256;    // 16-byte loads per thread

    __shared__ uint4 kbuf[2][TILE_CHUNKS];
    __shared__ float bbuf[2][kKeyTile];
    __shared__ __attribute__((aligned(16))) _Float16 vbuf[2][DVC * kVtStride];
    __shared__ float rowscale[4][32];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 31, h = lane >> 5;
    const int row0 = blockIdx.x * 128 + wave * 32;
    const int c0 = blockIdx.y * DVC;
    const int64_t m_pad = ((int64_t)a.n_keys + kRowPad - 1) / kRowPad * kRowPad;

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
    const _Float16* __restrict__ Vt = (const _Float16*)a.Vt;

    uint4 stg[LOADS];
    uint4 vstg[VLOADS];
    float bstg = 0.f;
    auto load_tile = [&](int t) __attribute__((always_inline)) {
        const char* base = keys + (int64_t)(t * kKeyTile) * ROW_BYTES;
#pragma unroll
        for (int l = 0; l < LOADS; ++l) {
            const int c = l * 256 + tid;
            if (TILE_CHUNKS % 256 == 0 || c < TILE_CHUNKS) stg[l] = *(const uint4*)(base + c * 16);
        }
        if (tid < kKeyTile) {
            const int j = t * kKeyTile + tid;
            bstg = j < a.n_keys ? fmaf(a.key_pot[j] - a.key_nrm[j], a.c_bias, a.key_lw2[j]) : -INFINITY;
        }
        // V^T tile: DVC rows (columns of V) x 32 keys, 4 chunks of 8 keys per row.
#pragma unroll
        for (int l = 0; l < VLOADS; ++l) {
            const int c = l * 256 + tid;
            if (c < VT_ELEMS / 8) {
                const int vr = c >> 2, part = c & 3;
                const int col = c0 + vr;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (col < a.dv) v = *(const uint4*)(Vt + (int64_t)col * m_pad + t * kKeyTile + part * 8);
                vstg[l] = v;
            }
        }
    };
    auto store_tile = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int l = 0; l < LOADS; ++l) {
            const int c = l * 256 + tid;
            if (TILE_CHUNKS % 256 == 0 || c < TILE_CHUNKS) {
                const int m = c / CPR, cc = c % CPR;
                kbuf[buf][m * CPR + (cc ^ (m & SWZ))] = stg[l];
            }
        }
        if (tid < kKeyTile) bbuf[buf][tid] = bstg;
#pragma unroll
        for (int l = 0; l < VLOADS; ++l) {
            const int c = l * 256 + tid;
            if (c < VT_ELEMS / 8) {
                const int vr = c >> 2, part = c & 3;
                // two 8-byte halves (rows are 72 bytes apart, 8-byte aligned)
                uint2* dst = (uint2*)(&vbuf[buf][vr * kVtStride + part * 8]);
                dst[0] = make_uint2(vstg[l].x, vstg[l].y);
                dst[1] = make_uint2(vstg[l].z, vstg[l].w);
            }
        }
    };

    f32x16 u[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) u[nb][r] = 0.f;

    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        if (t + 1 < ntiles) load_tile(t + 1);

        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
        const uint4* kb = kbuf[buf] + ln * CPR;
#pragma unroll
        for (int g = 0; g < NG; ++g) acc = score_step<OP>(kb[(2 * g + h) ^ (ln & SWZ)], q[g], acc);

        // weights p = 2^(z2 - L), register r <-> key 8*(r/4) + 4*h + (r%4)
        f16x8 p0, p1;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const float4 bv = *(const float4*)&bbuf[buf][8 * qq + 4 * h];
            const float bb[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p = ex2(fmaf(acc[4 * qq + e], a.c_score, bb[e]) - L);
                if (qq < 2)
                    p0[4 * qq + e] = (_Float16)p;
                else
                    p1[4 * (qq - 2) + e] = (_Float16)p;
            }
        }
        // U += P.V: A = weights (row ln, contraction slots 8h..8h+7), B = V^T
        // rows (column c0+nb*32+ln) at the same keys.
        const _Float16* vb = vbuf[buf];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const _Float16* vr = vb + (nb * 32 + ln) * kVtStride;
            const uint2 k0 = *(const uint2*)(vr + 4 * h);
            const uint2 k1 = *(const uint2*)(vr + 8 + 4 * h);
            const uint2 k2 = *(const uint2*)(vr + 16 + 4 * h);
            const uint2 k3 = *(const uint2*)(vr + 24 + 4 * h);
            const f16x8 b0 = __builtin_bit_cast(f16x8, make_uint4(k0.x, k0.y, k1.x, k1.y));
            const f16x8 b1 = __builtin_bit_cast(f16x8, make_uint4(k2.x, k2.y, k3.x, k3.y));
            u[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(p0, b0, u[nb], 0, 0, 0);
            u[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(p1, b1, u[nb], 0, 0, 0);
        }

        if (t + 1 < ntiles) store_tile(buf ^ 1);
        __syncthreads();
    }

    // Row factor 2^(L_i + (f_i - |x~_i|^2) c_bias) [* a_i] * 2^-s.
    if (h == 0) {
        float sc = 0.f;
        if (myrow < a.n_rows) {
            sc = ex2(L + (a.row_pot[myrow] - a.row_nrm[myrow]) * a.c_bias);
            if (!a.divide_by_a) sc *= a.row_w[myrow];
            sc *= a.v_unscale_dev ? a.v_unscale_dev[0] : 1.f;
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
hipError_t transport_mfma_launch(const TransportArgs& a, hipStream_t s) {
    constexpr int NB = NG >= 64 ? 2 : 4;
    const dim3 grid((a.n_rows + 127) / 128, (a.dv + 32 * NB - 1) / (32 * NB));
    transport_mfma_kernel<OP, NG, NB><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

template <int OP>
hipError_t transport_mfma_dispatch(int ng, const TransportArgs& a, hipStream_t s) {
    switch (ng) {
        case 1: return transport_mfma_launch<OP, 1>(a, s);
        case 2: return transport_mfma_launch<OP, 2>(a, s);
        case 4: return transport_mfma_launch<OP, 4>(a, s);
        case 8: return transport_mfma_launch<OP, 8>(a, s);
        case 16: return transport_mfma_launch<OP, 16>(a, s);
        case 32: return transport_mfma_launch<OP, 32>(a, s);
        case 64: return transport_mfma_launch<OP, 64>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_transport(int path, const TransportArgs& a0, float* scratch, void* Vt_buf,
                            int64_t m_pad, hipStream_t s) {
    TransportArgs a = a0;
    if (path == PATH_VALU) {
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
    vmax_kernel<<<1, 256, 0, s>>>(a.V, (int64_t)a.n_keys * a.dv, scratch);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    {
        const dim3 grid((unsigned)((m_pad + 31) / 32), (a.dv + 31) / 32);
        transpose_v_kernel<<<grid, 256, 0, s>>>(a.V, a.n_keys, m_pad, a.dv, scratch,
                                                (_Float16*)Vt_buf);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    a.Vt = Vt_buf;
    a.v_unscale_dev = scratch + 1;
    const int ng = path == PATH_MFMA_F32 ? a.dp / 8 : a.dp / 16;
    if (path == PATH_MFMA_F32) return transport_mfma_dispatch<OP_F32>(ng, a, s);
    if (path == PATH_MFMA_BF16) return transport_mfma_dispatch<OP_BF16>(ng, a, s);
    if (path == PATH_MFMA_F16) return transport_mfma_dispatch<OP_F16>(ng, a, s);
    return hipErrorInvalidValue;
}

}  // namespace fs
