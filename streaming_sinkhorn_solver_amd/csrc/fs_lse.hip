// fs_lse.hip -- the fused streaming log-sum-exp pass (one Sinkhorn half-step).
//
// "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU" (gist.science
// explainer), section "Method":
//  * part 1 (Proposition 1): for squared-Euclidean cost the stabilised update
//    f_i <- -eps LSE_j[(g_j - C_ij)/eps + log b_j] is a row-wise LSE of the
//    biased dot-product scores (2 x_i.y_j + g_j - |y_j|^2 + eps log b_j)/eps,
//    followed by adding |x_i|^2;
//  * part 2: the n x m score matrix never reaches HBM -- a block of rows stays
//    resident on chip while tiles of the other cloud stream past it, a running
//    row maximum and exp-sum are updated per tile (exact online LSE), and
//    score, bias, reduction and potential write are one kernel pass
//    (row-stationary traversal).
// The g-update is the same pass with the clouds' roles exchanged.
//
// Two kernel families:
//  * lse_valu_kernel<D, R>: d <= 8.  Each lane owns R rows; keys are
//    wave-uniform (scalar loads), scores are D fp32 FMAs per pair.  The bound
//    is the vector ALU / transcendental issue rate (one exp2 per pair).
//  * lse_mfma_kernel<OP, NG, QB>: d > 8.  The transposed score tile
//    S^T = K~ Q~^T is formed on the gfx950 matrix cores
//    (v_mfma_f32_32x32x{16_bf16,16_f16,2f32}), so every lane holds 16 scores of
//    ONE row and the row reduction stays inside the lane.  The row block
//    (4 waves x 32*QB rows x dp) lives in registers; 32-key tiles are
//    double-buffered through LDS in an XOR-swizzled layout.  The bound is the
//    matrix-core rate (2 n m d flops per half-step).
// Both can split the key range across workgroups (partial (max, sum) pairs
// merged afterwards in a fixed order), so results are deterministic.
#include "fs_device.hpp"
#include "fs_internal.h"

namespace fs {

namespace {

// ---------------------------------------------------------------- finalize
// Writes the output of row i from its base-2 LSE and returns the row's
// residual contribution w_i |2^((cur_i - out_i) c_bias) - 1| (0 without cur).
__device__ __forceinline__ float finalize_row(const LseArgs& a, int i, float lse2) {
    float o;
    if (a.mode == 0)
        o = fmaf(a.out_scale, lse2, a.row_nrm[i]);
    else
        o = lse2;
    float r = 0.f;
    if (a.cur) r = a.row_w[i] * fabsf(ex2((a.cur[i] - o) * a.c_bias) - 1.f);
    a.out[i] = o;
    return r;
}

// ------------------------------------------------------------ vector path
constexpr int kValuTile = 16;  // keys per inner tile

template <int D, int R>
__global__ __launch_bounds__(256) void lse_valu_kernel(LseArgs a) {
    constexpr int DP = D <= 4 ? 4 : 8;
    const float* __restrict__ rows = (const float*)a.rows;
    const float* __restrict__ keys = (const float*)a.keys;
    const int t = threadIdx.x;
    const int64_t row_base = (int64_t)blockIdx.x * 256 * R;
    const int split = blockIdx.y;

    float x[R][D];
    float M[R], S[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t i = row_base + r * 256 + t;
#pragma unroll
        for (int k = 0; k < D; ++k)
            x[r][k] = i < a.n_rows ? rows[i * DP + k] * a.c_score : 0.f;
        M[r] = -INFINITY;
        S[r] = 0.f;
    }

    const int j0 = split * a.keys_per_split;
    const int j1 = min(a.n_keys, j0 + a.keys_per_split);
    for (int jt = j0; jt < j1; jt += kValuTile) {
        float z[R][kValuTile];
#pragma unroll
        for (int jj = 0; jj < kValuTile; ++jj) {
            const int j = jt + jj;
            const bool valid = j < j1;
            const int jc = valid ? j : j1 - 1;
            const float beta = valid ? fmaf(a.key_pot[jc] - a.key_nrm[jc], a.c_bias, a.key_lw2[jc])
                                     : -INFINITY;
            float kc[D];
#pragma unroll
            for (int k = 0; k < D; ++k) kc[k] = keys[(int64_t)jc * DP + k];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float acc = beta;
#pragma unroll
                for (int k = 0; k < D; ++k) acc = fmaf(x[r][k], kc[k], acc);
                z[r][jj] = acc;
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float tmax = z[r][0];
#pragma unroll
            for (int jj = 1; jj < kValuTile; ++jj) tmax = fmaxf(tmax, z[r][jj]);
            const float Mn = fmaxf(M[r], tmax);
            float s = S[r] * ex2(M[r] - Mn);
#pragma unroll
            for (int jj = 0; jj < kValuTile; ++jj) s += ex2(z[r][jj] - Mn);
            S[r] = s;
            M[r] = Mn;
        }
    }

    float resid = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t i = row_base + r * 256 + t;
        if (i < a.n_rows) {
            if (a.n_split == 1)
                resid += finalize_row(a, (int)i, M[r] + lg2(S[r]));
            else
                a.part[(int64_t)split * a.n_rows + i] = make_float2(M[r], S[r]);
        }
    }
    if (a.n_split == 1 && a.cur) {
        __shared__ float red[16];
        resid = block_sum(resid, red);
        if (t == 0) a.resid_part[blockIdx.x] = resid;
    }
}

// ------------------------------------------------------ matrix-core path
template <int OP>
__device__ __forceinline__ f32x16 mfma_step(const uint4& av, const uint4& bv, f32x16 acc) {
    if constexpr (OP == OP_BF16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                       __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
    } else if constexpr (OP == OP_F16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, av),
                                                      __builtin_bit_cast(f16x8, bv), acc, 0, 0, 0);
    } else {
        // fp32: a 16-byte chunk holds 4 d-values; lane half h supplies the
        // values 4h..4h+3 of an 8-value group, one per instruction, so four
        // K=2 instructions cover the group (the same slot order on A and B).
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(av.x), __uint_as_float(bv.x), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(av.y), __uint_as_float(bv.y), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(av.z), __uint_as_float(bv.z), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(av.w), __uint_as_float(bv.w), acc, 0, 0, 0);
        return acc;
    }
}

// OP: score element type.  NG: 16-byte chunk pairs per operand row (a row is
// 2*NG chunks; dp = 16*NG for 2-byte types, 8*NG for fp32).  QB: 32-row
// blocks per wave.
template <int OP, int NG, int QB>
__global__ __launch_bounds__(256, 1) void lse_mfma_kernel(LseArgs a) {
    constexpr int CPR = 2 * NG;                    // 16-byte chunks per row
    constexpr int ROW_BYTES = CPR * 16;
    constexpr int TILE_CHUNKS = kKeyTile * CPR;    // chunks per key tile
    constexpr int LOADS = (TILE_CHUNKS + 255) / 256;
    constexpr int SWZ = CPR >= 8 ? 7 : CPR - 1;    // XOR swizzle of the chunk index

    __shared__ uint4 kbuf[2][TILE_CHUNKS];
    __shared__ float bbuf[2][kKeyTile];
    __shared__ float red[16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ln = lane & 31;  // row of the B block (a query row) / row of the A block (a key)
    const int h = lane >> 5;   // lane half: which 8 of each 16 contraction slots

    const int row0 = blockIdx.x * (4 * 32 * QB) + wave * (32 * QB);
    const int split = blockIdx.y;

    // Resident row block: lane (ln, h) holds chunk 2g+h of row row0+qb*32+ln.
    uint4 q[QB][NG];
    {
        const char* __restrict__ rows = (const char*)a.rows;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const char* rp = rows + (int64_t)(row0 + qb * 32 + ln) * ROW_BYTES + h * 16;
#pragma unroll
            for (int g = 0; g < NG; ++g) q[qb][g] = *(const uint4*)(rp + g * 32);
        }
    }

    const int j0 = split * a.keys_per_split;
    const int j1 = min(a.n_keys, j0 + a.keys_per_split);
    const int ntiles = (j1 - j0 + kKeyTile - 1) / kKeyTile;
    const char* __restrict__ keys = (const char*)a.keys;

    uint4 stg[LOADS];
    float bstg = 0.f;
// Global -> registers: tile t of this split (32 consecutive key rows) and the
// 32 key biases beta_j = (pot_j - |q~_j|^2) c_bias + log2 w_j (-inf past the end).
#define FS_LOAD_TILE(t_)                                                                      \
    do {                                                                                      \
        const char* base_ = keys + (int64_t)(j0 + (t_) * kKeyTile) * ROW_BYTES;               \
        _Pragma("unroll") for (int l = 0; l < LOADS; ++l) {                                   \
            const int c = l * 256 + tid;                                                      \
            if (TILE_CHUNKS % 256 == 0 || c < TILE_CHUNKS)                                    \
                stg[l] = *(const uint4*)(base_ + c * 16);                                     \
        }                                                                                     \
        if (tid < kKeyTile) {                                                                 \
            const int j = j0 + (t_) * kKeyTile + tid;                                         \
            bstg = j < j1 ? fmaf(a.key_pot[j] - a.key_nrm[j], a.c_bias, a.key_lw2[j])         \
                          : -INFINITY;                                                        \
        }                                                                                     \
    } while (0)
// Registers -> LDS buffer buf_, chunk c of key m at m*CPR + (c ^ (m & SWZ)).
#define FS_STORE_TILE(buf_)                                                                   \
    do {                                                                                      \
        _Pragma("unroll") for (int l = 0; l < LOADS; ++l) {                                   \
            const int c = l * 256 + tid;                                                      \
            if (TILE_CHUNKS % 256 == 0 || c < TILE_CHUNKS) {                                  \
                const int m = c / CPR, cc = c % CPR;                                          \
                kbuf[(buf_)][m * CPR + (cc ^ (m & SWZ))] = stg[l];                            \
            }                                                                                 \
        }                                                                                     \
        if (tid < kKeyTile) bbuf[(buf_)][tid] = bstg;                                         \
    } while (0)

    float M[QB], S[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        M[qb] = -INFINITY;
        S[qb] = 0.f;
    }

    FS_LOAD_TILE(0);
    FS_STORE_TILE(0);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        if (t + 1 < ntiles) FS_LOAD_TILE(t + 1);

        f32x16 acc[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[qb][r] = 0.f;

        const uint4* kb = kbuf[buf] + ln * CPR;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const uint4 av = kb[(2 * g + h) ^ (ln & SWZ)];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) acc[qb] = mfma_step<OP>(av, q[qb][g], acc[qb]);
        }

        // Epilogue.  Accumulator register r of lane (ln, h) is the score of row
        // ln with key 8*(r/4) + 4*h + (r%4) of the tile.
        float bv[16];
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const float4 v = *(const float4*)&bbuf[buf][8 * qq + 4 * h];
            bv[4 * qq + 0] = v.x;
            bv[4 * qq + 1] = v.y;
            bv[4 * qq + 2] = v.z;
            bv[4 * qq + 3] = v.w;
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float z[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) z[r] = fmaf(acc[qb][r], a.c_score, bv[r]);
            float tmax = z[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, z[r]);
            const float Mn = fmaxf(M[qb], tmax);
            float s = S[qb] * ex2(M[qb] - Mn);
#pragma unroll
            for (int r = 0; r < 16; ++r) s += ex2(z[r] - Mn);
            S[qb] = s;
            M[qb] = Mn;
        }

        if (t + 1 < ntiles) FS_STORE_TILE(buf ^ 1);
        __syncthreads();
    }

    // Merge the two lane halves (same row, disjoint keys) and finish.
    float resid = 0.f;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float M2 = __shfl_xor(M[qb], 32, 64);
        const float S2 = __shfl_xor(S[qb], 32, 64);
        lse_merge(M[qb], S[qb], M2, S2);
        const int row = row0 + qb * 32 + ln;
        if (h == 0 && row < a.n_rows) {
            if (a.n_split == 1)
                resid += finalize_row(a, row, M[qb] + lg2(S[qb]));
            else
                a.part[(int64_t)split * a.n_rows + row] = make_float2(M[qb], S[qb]);
        }
    }
    if (a.n_split == 1 && a.cur) {
        resid = block_sum(resid, red);
        if (tid == 0) a.resid_part[blockIdx.x] = resid;
    }
}

#undef FS_LOAD_TILE
#undef FS_STORE_TILE

// ----------------------------------------------------------------- merge
__global__ __launch_bounds__(256) void lse_merge_kernel(LseArgs a) {
    __shared__ float red[16];
    const int i = blockIdx.x * 256 + threadIdx.x;
    float r = 0.f;
    if (i < a.n_rows) {
        float M = -INFINITY, S = 0.f;
        for (int s = 0; s < a.n_split; ++s) {
            const float2 p = a.part[(int64_t)s * a.n_rows + i];
            lse_merge(M, S, p.x, p.y);
        }
        r = finalize_row(a, i, M + lg2(S));
    }
    if (a.cur) {
        r = block_sum(r, red);
        if (threadIdx.x == 0) a.resid_part[blockIdx.x] = r;
    }
}

__global__ __launch_bounds__(256) void resid_reduce_kernel(const float* __restrict__ part, int cnt,
                                                           float* __restrict__ out) {
    __shared__ float red[16];
    float v = 0.f;
    for (int k = threadIdx.x; k < cnt; k += 256) v += part[k];
    v = block_sum(v, red);
    if (threadIdx.x == 0) out[0] = v;
}

// --------------------------------------------------------------- dispatch
template <int D>
hipError_t valu_dispatch_r(const LseArgs& a, hipStream_t s, int R) {
    if (R == 4) {
        const dim3 grid((a.n_rows + 1023) / 1024, a.n_split);
        lse_valu_kernel<D, 4><<<grid, 256, 0, s>>>(a);
    } else {
        const dim3 grid((a.n_rows + 255) / 256, a.n_split);
        lse_valu_kernel<D, 1><<<grid, 256, 0, s>>>(a);
    }
    return hipGetLastError();
}

hipError_t valu_dispatch(int d, const LseArgs& a, hipStream_t s, int R) {
    switch (d) {
        case 1: return valu_dispatch_r<1>(a, s, R);
        case 2: return valu_dispatch_r<2>(a, s, R);
        case 3: return valu_dispatch_r<3>(a, s, R);
        case 4: return valu_dispatch_r<4>(a, s, R);
        case 5: return valu_dispatch_r<5>(a, s, R);
        case 6: return valu_dispatch_r<6>(a, s, R);
        case 7: return valu_dispatch_r<7>(a, s, R);
        case 8: return valu_dispatch_r<8>(a, s, R);
        default: return hipErrorInvalidValue;
    }
}

template <int OP, int NG, int QB>
hipError_t mfma_launch(const LseArgs& a, hipStream_t s) {
    constexpr int rpb = 4 * 32 * QB;
    const dim3 grid((a.n_rows + rpb - 1) / rpb, a.n_split);
    lse_mfma_kernel<OP, NG, QB><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

template <int OP>
hipError_t mfma_dispatch(int ng, const LseArgs& a, hipStream_t s) {
    if constexpr (OP == OP_F32) {
        switch (ng) {
            case 1: return mfma_launch<OP, 1, 4>(a, s);
            case 2: return mfma_launch<OP, 2, 4>(a, s);
            case 4: return mfma_launch<OP, 4, 4>(a, s);
            case 8: return mfma_launch<OP, 8, 4>(a, s);
            case 16: return mfma_launch<OP, 16, 2>(a, s);
            case 32: return mfma_launch<OP, 32, 2>(a, s);
            case 64: return mfma_launch<OP, 64, 1>(a, s);
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (ng) {
            case 1: return mfma_launch<OP, 1, 2>(a, s);
            case 2: return mfma_launch<OP, 2, 2>(a, s);
            case 4: return mfma_launch<OP, 4, 2>(a, s);
            case 8: return mfma_launch<OP, 8, 2>(a, s);
            case 16: return mfma_launch<OP, 16, 2>(a, s);
            case 32: return mfma_launch<OP, 32, 2>(a, s);
            case 64: return mfma_launch<OP, 64, 1>(a, s);
            default: return hipErrorInvalidValue;
        }
    }
}

int mfma_qb(int path, int ng) {
    if (path == PATH_MFMA_F32) return ng <= 8 ? 4 : (ng <= 32 ? 2 : 1);
    return ng <= 32 ? 2 : 1;
}

int ng_of(int path, int dp) { return path == PATH_MFMA_F32 ? dp / 8 : dp / 16; }

}  // namespace

// The vector path uses 4 rows per lane when there are enough rows to fill the
// GPU, else 1.
int valu_rows_per_lane(int n_rows) { return n_rows >= 65536 ? 4 : 1; }

int lse_rows_per_block(int path, int dp, int n_rows) {
    if (path == PATH_VALU) return 256 * valu_rows_per_lane(n_rows);
    return 4 * 32 * mfma_qb(path, ng_of(path, dp));
}

// For the vector path LseArgs::dp is the true dimension d (<= 8); operand rows
// are stored 4 (d <= 4) or 8 floats apart.  For the matrix paths it is the
// padded dimension.
hipError_t launch_lse(int path, const LseArgs& a, hipStream_t s) {
    hipError_t e;
    if (path == PATH_VALU) {
        const int R = valu_rows_per_lane(a.n_rows);
        e = valu_dispatch(a.dp, a, s, R);
    } else {
        const int ng = ng_of(path, a.dp);
        if (path == PATH_MFMA_F32)
            e = mfma_dispatch<OP_F32>(ng, a, s);
        else if (path == PATH_MFMA_BF16)
            e = mfma_dispatch<OP_BF16>(ng, a, s);
        else if (path == PATH_MFMA_F16)
            e = mfma_dispatch<OP_F16>(ng, a, s);
        else
            return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    int fin_blocks;
    if (a.n_split > 1) {
        fin_blocks = (a.n_rows + 255) / 256;
        lse_merge_kernel<<<fin_blocks, 256, 0, s>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else if (path == PATH_VALU) {
        const int R = valu_rows_per_lane(a.n_rows);
        fin_blocks = (a.n_rows + 256 * R - 1) / (256 * R);
    } else {
        const int rpb = 4 * 32 * mfma_qb(path, ng_of(path, a.dp));
        fin_blocks = (a.n_rows + rpb - 1) / rpb;
    }
    if (a.cur) {
        resid_reduce_kernel<<<1, 256, 0, s>>>(a.resid_part, fin_blocks, a.resid_out);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace fs
