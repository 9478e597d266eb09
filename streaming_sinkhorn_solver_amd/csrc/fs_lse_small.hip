// fs_lse_small.hip -- the streaming log-sum-exp pass for small dimensions
// (d <= 8) with the scores formed on the matrix cores.
//
// "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU" (gist.science
// explainer), section "Method": the update is a row-wise LSE of biased
// dot-product scores (part 1), streamed tile by tile with an exact online
// maximum/sum (part 2).  At d = 3 the contraction is a handful of products per
// pair and the pass is bound by the exponential, one per pair.  On gfx950 the
// transcendental unit, the vector ALU and the fp32 matrix instructions issue
// from the same SIMD without overlapping (their costs add), so everything
// besides the exponential has to be made cheap.  The whole score, bias
// included, is one matrix product per block of 32 keys x 32 rows, with the
// running reference in the accumulator input:
//
//   acc_ij = sum_k A_jk B_ki + C_i   with  A_j = (y~_j, beta_j, 0..),
//                                          B_i = (c_score x~_i, 1, 0..),
//                                          C_i = -R_i (every accumulator)
//          = z2_ij - R_i
//
// where z2 is the base-2 score of the vector path and R_i a per-row reference
// that plays the role of the running maximum.  The vector side is left with
// one exponential and one addition per pair.
//
// Three operand formats:
//  * fp16, d <= 4: every value v is split into fp16 parts (v = vh + vl, the
//    bias into three parts); the 16 contraction slots hold the products
//    rh*yh, rh*yl, rl*yh per coordinate and bh, bm, bl, so one
//    v_mfma_f32_32x32x16_f16 (fp16 products are exact in fp32) gives the
//    score with a relative error of a few 2^-22 per product.  A pass uses it
//    only if c_score * max_i sum_c |x_ic| * max_jc |y_jc| <= 2^9 (f then moves
//    by less than about 2e-4 eps from this error) and every bias fits fp16
//    with margin; otherwise
//  * bf16 three parts, d <= 4 (where the fp16 bound fails): every value split
//    into three bf16 parts (v = v1 + v2 + v3 exactly: 24 significant bits,
//    fp32's exponent range), the 32 contraction slots holding the six
//    products x1y1, x1y2, x2y1, x1y3, x2y2, x3y1 per coordinate (the three
//    dropped ones are below 2^-24 of x y) and b1, b2, b3: two
//    v_mfma_f32_32x32x16_bf16 per block, with the error of the fp32 products
//    and, unlike them, issued alongside the exponentials of other waves;
//  * fp32 (d > 4): A and B in fp32, ceil((d+1)/2) v_mfma_f32_32x32x2f32 per
//    block.
//
// R_i is only moved when a block's terms 2^(z2 - R) grow large (their sum
// above 2^64, checked with one compare) or on the row's first block; the move
// goes to the block maximum if that exceeds R by more than 2^8.  (The
// block-sparse form lets the sum reach 2^96 and keeps R 2^64 above the block
// maxima it starts from or moves to; see kSparseLift.)  (R, s) is
// the same base-2 (max, sum) pair as in the exact online LSE, with R a valid
// shift instead of the exact maximum: R + log2 s is unchanged, and the merge
// and finalize stages are shared with the other paths.
//
// The key records (A rows, with the bias of the current potential) are packed
// once per half-step by pack_key_records_kernel, streamed through LDS in tiles
// of TK keys (the 16-bit formats stored chunk-major, see cmaj_src), and read
// by every wave of the workgroup; three workgroups of 8 waves share a CU.
#include "fs_device.hpp"
#include "fs_internal.h"

namespace fs {

namespace {

constexpr int kSmallWaves = 8;        // waves per workgroup, 32 rows each
constexpr float kSlack = 8.f;         // R moves to a block maximum more than 2^8 above it
constexpr float kBigSum = 0x1p64f;    // common path: a block's terms sum to at most this
// The block-sparse form lets a block's terms reach 2^96 before R moves (a row
// sums at most 2^27 kept keys, so s stays below 2^123): its rows start from
// the best block's maximum, which at small eps may sit tens of bits under
// the row maximum, and should not move for that.
constexpr float kBigSumSparse = 0x1p96f;
// ... and its references sit 2^64 above the block maxima they start from or
// move to, so that a row may lie 160 bits above its start before it moves.
// Terms more than 126 - 64 = 62 bits under the row maximum may flush to zero:
// with at most 2^27 of them that is under 2^-35 of the sum.
constexpr float kSparseLift = 64.f;
constexpr float kF16Bound = 512.f;    // fp16 format: sum_c |c x_c| * max|y| <= this
constexpr float kF16Range = 16384.f;  // fp16 format: |c x|, |y| <= this, |beta| <= twice it
constexpr int kNbuf = 3;

// Keys per streamed tile (splits are whole tiles): fp32 records are 2*KP
// floats (8 KiB tiles for KP <= 2); fp16 records are 32 bytes.
constexpr int small_tile_keys(int kp) { return kp <= 2 ? 512 : 256; }
constexpr int f32_rec_bytes(int kp) { return 8 * kp; }
constexpr int kF16RecBytes = 32;
constexpr int kB3RecBytes = 64;  // bf16 three-part record: 32 slots

// Guard words written by the packing: the bits of max |y_c| over all keys,
// and nonzero if a bias or coordinate does not fit the fp16 format.
struct Guard {
    unsigned ymax_bits;
    unsigned bad;
};

// fp32 record of one key: slot k (0 <= k < 2*KP) of the contraction holds
// y~_k (k < d), beta (k == d) or 0; slot k is stored at (k & 1) * KP + (k >> 1)
// so that lane half h reads its KP values (slots h, h+2, ..) contiguously.
// fp16 record (d <= 4): slots 3c, 3c+1, 3c+2 hold yh_c, yl_c, yh_c; slots
// 3d..3d+2 the parts bh, bm, bl of beta; the rest 0.  Padding keys (j >=
// n_keys) get beta = -inf (bh = -inf, the other parts 0).
// bf16 three-part record (d <= 4): slots 6c..6c+5 hold y1, y2, y1, y3, y2,
// y1 of coordinate c (paired with the row's x1, x1, x2, x1, x2, x3), slots
// 6d..6d+2 the parts of beta (paired with 1); the rest 0; padding keys get
// b1 = -inf.
__device__ __forceinline__ void split3_bf16(float v, __bf16& v1, __bf16& v2, __bf16& v3) {
    v1 = (__bf16)v;
    const float r1 = v - (float)v1;
    v2 = (__bf16)r1;
    v3 = (__bf16)(r1 - (float)v2);
}

template <int KP>
__global__ __launch_bounds__(256) void pack_key_records_kernel(
    const float* __restrict__ keys, int stride, int d, int n_keys, int n_pad,
    const float* __restrict__ pot, const float* __restrict__ nrm, const float* __restrict__ lw2,
    float c_bias, float* __restrict__ rec32, _Float16* __restrict__ rec16,
    __bf16* __restrict__ rec3, Guard* guard) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    const bool in = j < n_pad;
    const bool real = j < n_keys;
    float y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = (real && k < d) ? keys[(int64_t)j * stride + k] : 0.f;
    const float beta = real ? fmaf(pot[j] - nrm[j], c_bias, lw2[j]) : -INFINITY;
    float ymax = 0.f;
    bool bad = false;
    if (in) {
        float v[2 * KP];
#pragma unroll
        for (int k = 0; k < 2 * KP; ++k)
            v[(k & 1) * KP + (k >> 1)] = k < d ? y[k] : (k == d ? beta : 0.f);
        float* o = rec32 + (int64_t)j * 2 * KP;
#pragma unroll
        for (int k = 0; k < 2 * KP; ++k) o[k] = v[k];
        if (rec16) {
            _Float16 hv[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) hv[k] = (_Float16)0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (c < d) {
                    const _Float16 yh = (_Float16)y[c];
                    const _Float16 yl = (_Float16)(y[c] - (float)yh);
                    hv[3 * c] = yh;
                    hv[3 * c + 1] = yl;
                    hv[3 * c + 2] = yh;
                    ymax = fmaxf(ymax, fabsf(y[c]));
                }
            }
            if (real) {
                const _Float16 bh = (_Float16)beta;
                const float r1 = beta - (float)bh;
                const _Float16 bm = (_Float16)r1;
                const _Float16 bl = (_Float16)(r1 - (float)bm);
                hv[3 * d] = bh;
                hv[3 * d + 1] = bm;
                hv[3 * d + 2] = bl;
                bad = !(fabsf(beta) <= 2.f * kF16Range) || !(ymax <= kF16Range);
            } else {
                hv[3 * d] = (_Float16)(-INFINITY);
            }
            uint4 w0, w1;
            __builtin_memcpy(&w0, &hv[0], 16);
            __builtin_memcpy(&w1, &hv[8], 16);
            uint4* o16 = (uint4*)(rec16 + (int64_t)j * 16);
            o16[0] = w0;
            o16[1] = w1;
        }
        if (rec3) {
            __bf16 bv[32];
#pragma unroll
            for (int k = 0; k < 32; ++k) bv[k] = (__bf16)0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (c < d) {
                    __bf16 v1, v2, v3;
                    split3_bf16(y[c], v1, v2, v3);
                    bv[6 * c] = v1;
                    bv[6 * c + 1] = v2;
                    bv[6 * c + 2] = v1;
                    bv[6 * c + 3] = v3;
                    bv[6 * c + 4] = v2;
                    bv[6 * c + 5] = v1;
                }
            }
            if (real) {
                split3_bf16(beta, bv[6 * d], bv[6 * d + 1], bv[6 * d + 2]);
            } else {
                bv[6 * d] = (__bf16)(-INFINITY);
            }
            uint4 w[4];
            __builtin_memcpy(&w[0], &bv[0], 64);
            uint4* o3 = (uint4*)(rec3 + (int64_t)j * 32);
#pragma unroll
            for (int q = 0; q < 4; ++q) o3[q] = w[q];
        }
    }
    if (rec16) {
        // at most one atomic per wave for each guard word, and none where the
        // word already holds as much (the maximum is the same every pass, so
        // after the first waves of a pass almost none is issued: contended
        // atomics on one word would otherwise serialise the whole grid)
        float wm = ymax;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) wm = fmaxf(wm, __shfl_xor(wm, o, 64));
        const bool wbad = __builtin_amdgcn_ballot_w64(bad) != 0;
        if ((threadIdx.x & 63) == 0) {
            const unsigned seen = __hip_atomic_load(&guard->ymax_bits, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
            if (wm > 0.f && __float_as_uint(wm) > seen)
                atomicMax(&guard->ymax_bits, __float_as_uint(wm));
            if (wbad) atomicOr(&guard->bad, 1u);
        }
    }
}

// Scalar load of N consecutive words at a wave-uniform address, waited for
// at once (the loads of the key tiles are counted by vmcnt alone).
template <int N>
__device__ __forceinline__ void sload_words(const int* p, int (&o)[N]) {
    if constexpr (N == 1) {
        int r;
        asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(r) : "s"(p) : "memory");
        o[0] = r;
    } else if constexpr (N == 2) {
        long long r;
        asm volatile("s_load_dwordx2 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(r) : "s"(p) : "memory");
        o[0] = (int)r;
        o[1] = (int)(r >> 32);
    } else {
        static_assert(N == 4, "1, 2 or 4 words");
        u32x4 r;
        asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(r) : "s"(p) : "memory");
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = (int)r[q];
    }
}

// Word at a wave-uniform address, read through the constant address space:
// a scalar load whose wait the compiler places before the first use, so it
// can be issued a tile early (the vector-memory counter still counts only
// tile copies: the kernel checks in its ISA that no vector load is emitted).
__device__ __forceinline__ int cload(const int* p) {
    return *(const __attribute__((address_space(4))) int*)p;
}

// Chunk-major LDS layout of a 32-key block of R-byte records (R / 16
// chunks of 16 bytes per key): chunk h of key k sits at byte (32 h + k) 16,
// so the matrix instruction's operand reads (lane k, chunk h) cover 16
// consecutive bytes per lane across the wave, free of bank conflicts (the
// record-major layout put the lanes R bytes apart: 4-way conflicts for
// 64-byte records, 2-way for 32-byte ones).  A copy lane that fills LDS
// position p of the block (in 16-byte units) reads chunk p / 32 of key
// p % 32; the byte offset of that source within the block:
template <int R>
__device__ __forceinline__ uint32_t cmaj_src(uint32_t p) {
    return (p & 31u) * (uint32_t)R + (p >> 5) * 16u;
}

// SPARSE: the block-sparse form.  The workgroup's keys are not a contiguous
// range but the 32-key blocks listed for its row block by the screening
// (LseArgs::bs_list, padded to whole tiles with a block of -inf records);
// a tile gathers 16 listed blocks, each wave-wide copy instruction fetching
// whole blocks at per-lane offsets.  With n_split = S the list's tiles are
// dealt round-robin to S workgroups (partials merged as for key ranges).
template <int KP, bool SPARSE = false>
__global__ __launch_bounds__(kSmallWaves * 64, 6) void lse_small_kernel(LseArgs a) {
    constexpr int W = kSmallWaves;
    constexpr bool HAS_F16 = KP <= 2;  // the fp16 format covers d <= 4
    constexpr int TK = small_tile_keys(KP);
    constexpr int F32_TILE = TK * f32_rec_bytes(KP);
    constexpr int F16_TILE = HAS_F16 ? TK * kF16RecBytes : 0;
    // The tile ring is kNbuf slots of the larger tile, cut per record
    // format in run(): the sparse form, whose
    // tiles are gathered from scattered blocks and wait longer for their
    // copies, cuts the same bytes into more slots when its tiles are fp32
    // records (6 slots; 4 slots and a conversion area for the shifted fp16
    // operands).
    constexpr int BUF_BYTES = F16_TILE > F32_TILE ? F16_TILE : F32_TILE;
    constexpr bool SHIFT = SPARSE && HAS_F16;
    // Three workgroups per CU (six waves per SIMD, 80 registers each): more
    // waves to cover the copies (gathered, in the sparse form) and the
    // start-up of short workgroups than a deeper ring would (fs2 launch 0.369
    // -> 0.329 ms, C5 half-step 5.48 -> 5.33 ms), so the ring is three slots
    // of the larger tile.
    constexpr int RING_BYTES = kNbuf * BUF_BYTES;
    static_assert(!SHIFT || TK == W * 64, "shifted conversion: one key per thread");
    __shared__ __attribute__((aligned(16))) uint4 tbuf[RING_BYTES / 16];
    // sparse: the starting block (2 KiB: a bf16 three-part block)
    __shared__ __attribute__((aligned(16))) uint4 ibuf[SPARSE ? 128 : 1];
    __shared__ float red[16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 31;
    const int h = lane >> 5;
    int row_block, split, nsp = a.n_split;
    if constexpr (SPARSE) {
        // planned (row block, split) of this workgroup: the plan's entries
        // are dealt to the 8 XCDs (workgroups go to XCD id % 8) in
        // contiguous, equal shares, so that neighbouring row blocks share an
        // L2 and every XCD has work; the grid is an upper bound of the plan
        // and the workgroups past an XCD's share have nothing to do
        const int total = *a.bs_total;
        const int id = blockIdx.x, x = id & 7, kk = id >> 3;
        const int q = total >> 3, r = total & 7;
        if (kk >= q + (x < r ? 1 : 0)) return;
        const int idx = x * q + min(x, r) + kk;
        row_block = a.bs_map[2 * idx];
        split = a.bs_map[2 * idx + 1];
        nsp = a.bs_nsplit[row_block];
    } else {
        xcd_work(row_block, split);
    }
    const int row = row_block * (W * 32) + wave * 32 + ln;  // rows are padded: always readable
    constexpr int SUB_BLOCKS = TK / 32;  // 32-key blocks per tile
    const int j0 = SPARSE ? 0 : split * a.keys_per_split;
    const int j1 = min(a.n_keys, j0 + a.keys_per_split);
    // sparse: this workgroup's tiles are list tiles split, split + S, ..
    const int* __restrict__ lst =
        SPARSE ? a.bs_list + (int64_t)row_block * a.bs_cap + split * SUB_BLOCKS : nullptr;
    const int list_step = SPARSE ? nsp * SUB_BLOCKS : 0;
    int ntiles;
    if constexpr (SPARSE) {
        const int all = (a.bs_count[row_block] + SUB_BLOCKS - 1) / SUB_BLOCKS;
        ntiles = all > split ? (all - split + nsp - 1) / nsp : 0;
    } else {
        ntiles = (j1 - j0 + TK - 1) / TK;
    }
    const int d = a.dp;
    const int stride = d <= 4 ? 4 : 8;
    const float* __restrict__ xr = (const float*)a.rows + (int64_t)row * stride;
    float r[8];  // c_score * x~ of this lane's row
#pragma unroll
    for (int k = 0; k < 8; ++k) r[k] = k < d ? a.c_score * xr[k < stride ? k : 0] : 0.f;

    // Format of this pass (the same for every workgroup, so no result depends
    // on which rows share a workgroup): fp16 if the bound holds for the
    // largest row (L1 norm, from the problem set-up) against the largest key
    // coordinate, and the packing flagged nothing.
    bool use16 = false;
    if constexpr (HAS_F16) {
        const Guard* g = (const Guard*)a.krec_guard;
        const float ymax = __uint_as_float(g->ymax_bits);
        const float rl1 = a.c_score * *a.row_l1;
        use16 = rl1 * ymax <= kF16Bound && rl1 <= kF16Range && g->bad == 0;
    }

    // Sparse form, shifted fp16 operands: with O the row block's origin
    // (o_x = O - own centre, o_y = O - key cloud's centre), the score is
    //   c x~.y~ + beta = c (x~ - o_x).(y~ - o_y) + [beta + c o_x.(y~ - o_y)] + c x~.o_y,
    // the first term a product of small vectors (rows and kept keys lie near
    // O), the bracket the key's new bias, the last a constant of the row,
    // added to its result.  Taken when the pass-wide fp16 format does not
    // hold but the screening found the shifted magnitudes within its bound for
    // this row block (and the packing flagged no key).
    bool shifted = false;
    float rowc = 0.f;
    float cox[3] = {0.f, 0.f, 0.f}, oy[3] = {0.f, 0.f, 0.f};
    if constexpr (SHIFT) {
        const float4 o0 = a.bs_org[2 * row_block], o1 = a.bs_org[2 * row_block + 1];
        shifted = !use16 && o0.w != 0.f && ((const Guard*)a.krec_guard)->bad == 0;
        if (shifted) {
            const float ox[3] = {o0.x, o0.y, o0.z};
            oy[0] = o1.x;
            oy[1] = o1.y;
            oy[2] = o1.z;
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                if (k < d) {
                    rowc = fmaf(r[k], oy[k], rowc);
                    r[k] = a.c_score * (xr[k] - ox[k]);
                    cox[k] = a.c_score * ox[k];
                }
            }
        }
    }

    float R = 0.f;      // reference: the running maximum, moved lazily
    float s = 0.f;      // sum of 2^(z2 - R) over the keys seen
    float delta = 0.f;  // R minus the reference baked into cm (moves within a tile)
    float baked = 0.f;  // sparse form: the reference baked into cm now (refreshed on a move)
    f32x16 cm;          // MFMA C operand: minus the reference, refreshed per tile
#pragma unroll
    for (int q = 0; q < 16; ++q) cm[q] = 0.f;

    auto block_max = [&](const f32x16& acc) __attribute__((always_inline)) {
        float t = fmaxf(acc[0], acc[1]);
#pragma unroll
        for (int q = 2; q < 16; ++q) t = fmaxf(t, acc[q]);
        return t;
    };
    // acc = z2 - (R - delta).  Common case -- no lane moved its reference in
    // this tile (delta = 0) and the block's terms 2^acc sum to at most
    // kBigSum (so none is large, let alone infinite): add them.  Checking the
    // sum costs one compare; the maximum is only formed on the other path,
    // which moves R, where needed, to the block maximum.  Only per-lane
    // scalars change, so the common path carries no register-tuple copies.
    // REBAKE: bk is the reference baked into cm when acc's matrix instruction
    // was issued, and a move re-bakes cm, so that the blocks after it take
    // the common path again; taken by the sparse form's formats that
    // serve small eps, whose rows move often (their start is shared by 256
    // rows).  Otherwise one baked reference per tile, R minus it in delta (a
    // loop-invariant cm keeps the common path free of register-tuple copies).
    auto epilogue = [&](const f32x16& acc, float bk, auto rebake_c) __attribute__((always_inline)) {
        constexpr bool REBAKE = decltype(rebake_c)::value;
        const float dlt = REBAKE ? R - bk : delta;
        float e[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) e[q] = ex2(acc[q]);
        // pairwise sum (short dependency chains)
#pragma unroll
        for (int w = 1; w < 16; w <<= 1)
#pragma unroll
            for (int q = 0; q < 16; q += 2 * w) e[q] += e[q + w];
        if (__builtin_amdgcn_ballot_w64(!(e[0] <= (SPARSE ? kBigSumSparse : kBigSum)) ||
                                        dlt != 0.f)) {
            const float t = block_max(acc) - dlt;  // block maximum relative to R
            const float dl = t > kSlack ? t + (SPARSE ? kSparseLift : 0.f) : 0.f;
            const float sh = dlt + dl;
#pragma unroll
            for (int q = 0; q < 16; ++q) e[q] = ex2(acc[q] - sh);
            // same summation tree as the common path: a lane that does not
            // move (dl = 0, sh = 0) gets bit-identical results on either path
#pragma unroll
            for (int w = 1; w < 16; w <<= 1)
#pragma unroll
                for (int q = 0; q < 16; q += 2 * w) e[q] += e[q + w];
            if constexpr (SPARSE) {
                // the old sum, scaled in two halves: 2^-dl alone may flush to
                // zero (dl > 126) where the scaled sum is still a normal
                // float (a lifted reference moves that far; the dense form's
                // moves stay under 2^64 + 2^8 and its sums under 2^91)
                const float hf = ex2(-0.5f * dl);
                s = s * hf * hf + e[0];
            } else {
                s = s * ex2(-dl) + e[0];
            }
            R += dl;
            if constexpr (REBAKE) {
#pragma unroll
                for (int q = 0; q < 16; ++q) cm[q] = -R;
                baked = R;
            } else {
                delta = sh;
            }
        } else {
            s += e[0];
        }
    };

    // Shifted fp16 records of nkeys fp32 records at src (one key per thread):
    // y~ - o_y split into fp16 parts, the bias beta + c o_x.(y~ - o_y) into
    // three; a -inf bias (padding) stays -inf with zero parts.  Keys 0..255 go
    // to dst0, 256..511 to dst1 (each 256 records after the other when the
    // two are contiguous).
    auto convert = [&](const char* src, int nkeys, char* dst0,
                       char* dst1) __attribute__((always_inline)) {
        const int t = threadIdx.x;
        if (t < nkeys) {
            const float* rf = (const float*)(src + (size_t)t * f32_rec_bytes(KP));
            _Float16 hv[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) hv[k] = (_Float16)0.f;
            float beta = rf[(d & 1) * KP + (d >> 1)];
            if (beta == -INFINITY) {
                hv[3 * d] = (_Float16)(-INFINITY);
            } else {
#pragma unroll
                for (int c = 0; c < 3; ++c) {
                    if (c < d) {
                        const float w = rf[(c & 1) * KP + (c >> 1)] - oy[c];
                        beta = fmaf(cox[c], w, beta);
                        const _Float16 wh = (_Float16)w;
                        const _Float16 wl = (_Float16)(w - (float)wh);
                        hv[3 * c] = wh;
                        hv[3 * c + 1] = wl;
                        hv[3 * c + 2] = wh;
                    }
                }
                const _Float16 bh = (_Float16)beta;
                const float r1 = beta - (float)bh;
                const _Float16 bm = (_Float16)r1;
                hv[3 * d] = bh;
                hv[3 * d + 1] = bm;
                hv[3 * d + 2] = (_Float16)(r1 - (float)bm);
            }
            uint4 w0, w1;
            __builtin_memcpy(&w0, &hv[0], 16);
            __builtin_memcpy(&w1, &hv[8], 16);
            // chunk-major 32-key blocks (see cmaj_src)
            const int tt = t < 256 ? t : t - 256;
            uint4* o = (uint4*)((t < 256 ? dst0 : dst1) + (tt >> 5) * 32 * kF16RecBytes +
                                (tt & 31) * 16);
            o[0] = w0;
            o[32] = w1;
        }
    };

    // The tile loop for one operand format: MODE 0 fp32 records, 1 fp16-split
    // records, 2 (sparse) fp32 records turned into shifted fp16 ones in LDS,
    // 3 bf16 three-part records.  A ring tile holds SK keys: TK, or half a
    // tile of TK keys for the 64-byte bf16 records (splits and the sparse
    // form's list tiles stay whole tiles of TK keys).
    auto run = [&](auto mode_c) __attribute__((always_inline)) {
        constexpr int MODE = decltype(mode_c)::value;
        constexpr bool F16 = MODE == 1 || MODE == 2;
        constexpr bool B3 = MODE == 3;
        constexpr bool CONV = MODE == 2;
        constexpr int REC_BYTES =  // as multiplied
            B3 ? kB3RecBytes : (F16 ? kF16RecBytes : f32_rec_bytes(KP));
        constexpr int DREC_BYTES =  // as loaded
            B3 ? kB3RecBytes : (MODE == 1 ? kF16RecBytes : f32_rec_bytes(KP));
        constexpr int SK = B3 ? TK / 2 : TK;
        constexpr int HALVES = TK / SK;
        constexpr int TILE_BYTES = SK * DREC_BYTES;
        // ring of this format: NB slots of SLOT bytes (+ the conversion area)
        constexpr int NB = !SPARSE || MODE == 1 || B3 ? kNbuf : (MODE == 0 ? 6 : 4);
        constexpr int SLOT = !SPARSE ? BUF_BYTES : TILE_BYTES;
        constexpr int CONV_BYTES = TK * kF16RecBytes;
        static_assert(NB * SLOT + (CONV ? CONV_BYTES : 0) <= RING_BYTES, "ring fits");
        char* const ring = (char*)&tbuf[0];
        char* const conv = ring + NB * SLOT;  // MODE 2: converted records of one tile
        constexpr int TILE_INSTR = TILE_BYTES / 1024;  // wave-wide 1 KiB loads per tile
        constexpr int INSTR_PER_WAVE = (TILE_INSTR + W - 1) / W;
        constexpr int MIN_INSTR = TILE_INSTR / W;
        constexpr int SUB = SK / 32;                   // 32-key blocks per ring tile
        static_assert(TILE_BYTES % 1024 == 0 && TILE_BYTES <= BUF_BYTES, "tile geometry");
        const char* __restrict__ recs =
            B3          ? (const char*)a.krec3 + (int64_t)j0 * DREC_BYTES
            : MODE == 1 ? (const char*)a.krec16 + (int64_t)j0 * DREC_BYTES
                        : (const char*)a.krec + (int64_t)j0 * DREC_BYTES;
        const int ntl = ntiles * HALVES;  // ring tiles

        // sparse: the list words of ring tile k that this wave's copies need
        // (one per instruction of 2 KiB bf16 three-part blocks, BPI per
        // instruction otherwise), read a tile ahead of their copies
        constexpr int BLK = 32 * DREC_BYTES;
        constexpr int BPI = !SPARSE || B3 ? 1 : 1024 / BLK;
        static_assert(!SPARSE || B3 || 1024 % BLK == 0, "whole blocks per instruction");
        auto tile_words = [&](int k, int (&w)[INSTR_PER_WAVE][BPI]) __attribute__((always_inline)) {
#pragma unroll
            for (int l = 0; l < INSTR_PER_WAVE; ++l) {
                const int L = l * W + wave;
#pragma unroll
                for (int q = 0; q < BPI; ++q) {
                    // B3: instruction L covers half L % 2 of block L / 2 of the
                    // ring tile, which is half k % 2 of list tile k / 2
                    const int off = B3 ? (k / HALVES) * list_step + (k % HALVES) * SUB + L / 2
                                       : k * list_step + L * BPI + q;
                    w[l][q] = (TILE_INSTR % W == 0 || L < TILE_INSTR) ? cload(lst + off) : 0;
                }
            }
        };
        // tile k -> slot (contiguous copy; records past j1 in the last tile
        // are padding records of score -inf: splits are whole tiles); the
        // sparse form's copies take the list words of their tile
        const uint32_t lane16 = (uint32_t)lane * 16u;
        auto issue_tile = [&](int k, int slot, const int (&w)[INSTR_PER_WAVE][BPI])
                              __attribute__((always_inline)) {
#pragma unroll
            for (int l = 0; l < INSTR_PER_WAVE; ++l) {
                const int L = l * W + wave;
                if (TILE_INSTR % W == 0 || L < TILE_INSTR) {
                    if constexpr (SPARSE && B3) {
                        const uint32_t Jc = min((uint32_t)w[l][0], (uint32_t)a.bs_sentinel);
                        dma_to_lds16(recs,
                                     Jc * (uint32_t)BLK +
                                         cmaj_src<DREC_BYTES>((uint32_t)(L & 1) * 64u + lane),
                                     ring + slot * SLOT + L * 1024);
                    } else if constexpr (SPARSE) {
                        // instruction L covers blocks L*BPI .. L*BPI+BPI-1 of the tile;
                        // lane `lane` fetches 16 bytes of block L*BPI + lane/LPB
                        constexpr int LPB = 64 / BPI;
                        int J = w[l][0];
#pragma unroll
                        for (int q = 1; q < BPI; ++q)
                            if (lane / LPB == q) J = w[l][q];
                        const uint32_t Jc = min((uint32_t)J, (uint32_t)a.bs_sentinel);
                        const uint32_t voff = MODE == 1 ? cmaj_src<DREC_BYTES>(lane)
                                                        : (uint32_t)(lane % LPB) * 16u;
                        dma_to_lds16(recs, Jc * (uint32_t)BLK + voff, ring + slot * SLOT + L * 1024);
                    } else {
                        if constexpr (F16 || B3) {
                            // instruction L fills 1 KiB at byte L * 1024 of the
                            // tile: part of the block (L * 1024) / BLK
                            const int64_t blk_base = (int64_t)(L * 1024 / BLK) * BLK;
                            const uint32_t p0 = (uint32_t)(L * 1024 % BLK) / 16u;
                            dma_to_lds16(recs + (int64_t)k * TILE_BYTES + blk_base,
                                         cmaj_src<DREC_BYTES>(p0 + lane),
                                         ring + slot * SLOT + L * 1024);
                        } else {
                            dma_to_lds16(recs + (int64_t)k * TILE_BYTES + L * 1024, lane16,
                                         ring + slot * SLOT + L * 1024);
                        }
                    }
                }
            }
        };
        int wnext[INSTR_PER_WAVE][BPI];  // sparse: words of the next tile to copy
        if constexpr (SPARSE) {
            // the block of largest bound, for the starting reference
            if (ntiles > 0 && wave == 0) {
                int ent[1];
                sload_words<1>(a.bs_best + row_block, ent);
                const uint32_t Jc = min((uint32_t)ent[0], (uint32_t)a.bs_sentinel);
                if constexpr (B3) {
                    dma_to_lds16(recs, Jc * (uint32_t)BLK + cmaj_src<DREC_BYTES>(lane), &ibuf[0]);
                    dma_to_lds16(recs, Jc * (uint32_t)BLK + cmaj_src<DREC_BYTES>(64u + lane),
                                 &ibuf[64]);
                } else if constexpr (MODE == 1) {
                    dma_to_lds16(recs, Jc * (uint32_t)BLK + cmaj_src<DREC_BYTES>(lane), &ibuf[0]);
                } else {
                    constexpr int LPB = 64 / (1024 / (32 * DREC_BYTES));
                    dma_to_lds16(recs,
                                 Jc * (uint32_t)(32 * DREC_BYTES) + (uint32_t)(lane % LPB) * 16u,
                                 &ibuf[0]);
                }
            }
        }
        if (ntl > 0) {
#pragma unroll
            for (int k = 0; k < NB - 1; ++k) {
                if constexpr (SPARSE) tile_words(min(k, ntl - 1), wnext);
                issue_tile(min(k, ntl - 1), k, wnext);
            }
            if constexpr (SPARSE) tile_words(min(NB - 1, ntl - 1), wnext);
        }

        // B operand of this lane: row `row`, the lane half's contraction slots
        f16x8 b16;
        float b32[KP];
        bf16x8 b3a, b3b;  // bf16 three-part: slots 8h.. of each 16-slot product
        if constexpr (B3) {
            __bf16 sl[32];
#pragma unroll
            for (int k = 0; k < 32; ++k) sl[k] = (__bf16)0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (c < d) {
                    __bf16 x1, x2, x3;
                    split3_bf16(r[c], x1, x2, x3);
                    sl[6 * c] = x1;
                    sl[6 * c + 1] = x1;
                    sl[6 * c + 2] = x2;
                    sl[6 * c + 3] = x1;
                    sl[6 * c + 4] = x2;
                    sl[6 * c + 5] = x3;
                }
            }
#pragma unroll
            for (int k = 0; k < 32; ++k)
                if (k >= 6 * d && k < 6 * d + 3) sl[k] = (__bf16)1.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                b3a[k] = h ? sl[8 + k] : sl[k];
                b3b[k] = h ? sl[24 + k] : sl[16 + k];
            }
        } else if constexpr (F16) {
            _Float16 sl[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) sl[k] = (_Float16)0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (c < d) {
                    const _Float16 rh = (_Float16)r[c];
                    const _Float16 rl = (_Float16)(r[c] - (float)rh);
                    sl[3 * c] = rh;
                    sl[3 * c + 1] = rh;
                    sl[3 * c + 2] = rl;
                }
            }
#pragma unroll
            for (int k = 0; k < 16; ++k)
                if (k >= 3 * d && k < 3 * d + 3) sl[k] = (_Float16)1.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) b16[k] = h ? sl[8 + k] : sl[k];
        } else {
#pragma unroll
            for (int p = 0; p < KP; ++p) {
                const int k = 2 * p + h;
                b32[p] = k < d ? r[k] : (k == d ? 1.f : 0.f);
            }
        }
        auto scores = [&](const char* rb, f32x16& acc) __attribute__((always_inline)) {
            if constexpr (B3) {
                const char* kr = rb + h * 512 + ln * 16;  // chunk-major block
                const bf16x8 a0 = *(const bf16x8*)kr;
                const bf16x8 a1 = *(const bf16x8*)(kr + 1024);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b3a, cm, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b3b, acc, 0, 0, 0);
            } else if constexpr (F16) {
                const f16x8 av = *(const f16x8*)(rb + h * 512 + ln * 16);  // chunk-major block
                acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, b16, cm, 0, 0, 0);
            } else {
                const float* rf = (const float*)rb + (size_t)ln * 2 * KP + h * KP;
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(rf[0], b32[0], cm, 0, 0, 0);
#pragma unroll
                for (int p = 1; p < KP; ++p)
                    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(rf[p], b32[p], acc, 0, 0, 0);
            }
        };

        // The first NB - 1 tiles are in flight.  The sparse form waits here
        // only for its starting block (issued before them), the dense form
        // for tile 0, which holds its starting block; the barriers below do
        // not fence, so the copies behind keep streaming meanwhile.
        if constexpr (MIN_INSTR == 0)
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NB - (SPARSE ? 1 : 2)) * MIN_INSTR) : "memory");
        stage_barrier();

        // R starts at the maximum of the first 32-key block (finite wherever
        // the lane sees a key at all; a lane that never does keeps s = 0, the
        // empty state); in the sparse form, kSparseLift above that of the
        // block of largest bound, whose scores are near the row maxima, so
        // that R rarely moves.
        if (ntiles > 0) {
            f32x16 acc;
            if constexpr (CONV) {
                convert((const char*)&ibuf[0], 32, conv, conv);
                stage_barrier();
                scores(conv, acc);
                stage_barrier();  // rewritten by the first tile's conversion
            } else {
                scores(SPARSE ? (const char*)&ibuf[0] : ring, acc);
            }
            const float t = block_max(acc);
            R = t > -INFINITY ? t + (SPARSE ? kSparseLift : 0.f) : 0.f;
        }
        if constexpr (SPARSE) {
            // tile 0 (tiles 1 .. NB-2 may still be in flight)
            if constexpr (MIN_INSTR == 0)
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            else
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NB - 2) * MIN_INSTR) : "memory");
            stage_barrier();
        }

        for (int t = 0; t < ntl; ++t) {
            const int slot = t % NB;
            issue_tile(min(t + NB - 1, ntl - 1), (t + NB - 1) % NB, wnext);
            if constexpr (SPARSE) tile_words(min(t + NB, ntl - 1), wnext);
            const char* tb = ring + slot * SLOT;
            if constexpr (CONV) {
                convert(tb, TK, conv, conv + (TK / 2) * kF16RecBytes);
                stage_barrier();
                tb = conv;
            }
            // 32-key block u of the tile as multiplied
            auto blk = [&](int u) __attribute__((always_inline)) { return tb + u * 32 * REC_BYTES; };
#pragma unroll
            for (int q = 0; q < 16; ++q) cm[q] = -R;
            delta = 0.f;
            baked = R;
            // one accumulator set per wave: the other waves of the SIMD hide
            // the matrix latency (six per SIMD, 80 registers each; a second
            // set spilled at that budget)
#pragma unroll
            for (int u = 0; u < SUB; ++u) {
                f32x16 acc;
                scores(blk(u), acc);
                epilogue(acc, baked, std::integral_constant<bool, SPARSE && MODE != 1>{});
            }
            // tiles issued after tile t+1: t+2 .. t+NB-1
            if constexpr (MIN_INSTR == 0)
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            else
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NB - 2) * MIN_INSTR) : "memory");
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
    if constexpr (SPARSE) {
        // the pass-wide fp16 records when they hold (no conversion), else the
        // shifted ones when this row block allows them, else bf16 three-part
        if constexpr (SHIFT) {
            if (use16) {
                run(std::integral_constant<int, 1>{});
            } else if (shifted) {
                run(std::integral_constant<int, 2>{});
            } else {
                run(std::integral_constant<int, 3>{});
            }
        } else {
            run(std::integral_constant<int, 0>{});
        }
    } else if constexpr (HAS_F16) {
        if (use16)
            run(std::integral_constant<int, 1>{});
        else
            run(std::integral_constant<int, 3>{});
    } else {
        run(std::integral_constant<int, 0>{});
    }

    // The sum's binary exponent moves into the reference (s in [1/2, 1)), so
    // that the merges below, which scale a sum by 2^(M - M_max), see M near
    // the row's log-sum: a reference far under it with a large sum (the
    // sparse form's rows that do not move) would otherwise underflow there.
    // (The dense form's sums stay under 2^91: what such a merge could lose
    // there is under 2^-35 of the row's sum.)
    if (SPARSE && s > 0.f) {
        int ex;
        s = frexpf(s, &ex);
        R += (float)ex;
    }
    // the two lane halves hold the same row over disjoint keys
    float M = s > 0.f ? R + rowc : -INFINITY;
    {
        const float M2 = __shfl_xor(M, 32, 64);
        const float S2 = __shfl_xor(s, 32, 64);
        lse_merge(M, s, M2, S2);
    }
    float resid = 0.f;
    if (h == 0 && row < a.n_rows) {
        if (a.n_split == 1) {
            const float lse2 = M + lg2(s);
            float o = a.mode == 0 ? fmaf(a.out_scale, lse2, a.row_nrm[row]) : lse2;
            if (a.cur) resid = a.row_w[row] * fabsf(ex2((a.cur[row] - o) * a.c_bias) - 1.f);
            a.out[row] = o;
        } else {
            a.part[(int64_t)split * a.n_rows + row] = make_float2(M, s);
        }
    }
    if (a.n_split == 1 && a.cur) {
        resid = block_sum(resid, red);
        if (tid == 0) a.resid_part[row_block] = resid;
    }
}

template <int KP, bool SPARSE = false>
hipError_t small_launch(const LseArgs& a, hipStream_t s, hipEvent_t ev_begin) {
    hipError_t e;
    const int n_pad_keys = a.krec_keys;
    constexpr bool f16 = KP <= 2;
    if (f16 && (e = launch_fill((float*)a.krec_guard, 2, 0.f, s)) != hipSuccess) return e;
    pack_key_records_kernel<KP><<<(n_pad_keys + 255) / 256, 256, 0, s>>>(
        (const float*)a.keys, a.dp <= 4 ? 4 : 8, a.dp, a.n_keys, n_pad_keys, a.key_pot, a.key_nrm,
        a.key_lw2, a.c_bias, a.krec, f16 ? (_Float16*)a.krec16 : nullptr,
        f16 ? (__bf16*)a.krec3 : nullptr, (Guard*)a.krec_guard);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (ev_begin && (e = hipEventRecord(ev_begin, s)) != hipSuccess) return e;
    const dim3 grid = SPARSE ? dim3(a.bs_grid, 1)
                             : dim3((a.n_rows + kSmallWaves * 32 - 1) / (kSmallWaves * 32),
                                    a.n_split);
    lse_small_kernel<KP, SPARSE><<<grid, kSmallWaves * 64, 0, s>>>(a);
    return hipGetLastError();
}

// Largest L1 norm over the points of a cloud (bits of a non-negative float,
// combined with atomicMax; *out must start at 0).
__global__ __launch_bounds__(256) void row_l1max_kernel(const float* __restrict__ ops, int64_t n,
                                                        int stride, int d, unsigned* out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    float v = 0.f;
    if (i < n)
        for (int k = 0; k < d; ++k) v += fabsf(ops[i * stride + k]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    if ((threadIdx.x & 63) == 0 && v > 0.f) atomicMax(out, __float_as_uint(v));
}

}  // namespace

hipError_t launch_row_l1max(const float* ops, int64_t n, int d, float* out, hipStream_t s) {
    hipError_t e = launch_fill(out, 1, 0.f, s);
    if (e != hipSuccess) return e;
    row_l1max_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(ops, n, d <= 4 ? 4 : 8, d,
                                                                 (unsigned*)out);
    return hipGetLastError();
}

int small_kp(int d) { return (d + 2) / 2; }
int small_tile(int d) { return small_tile_keys(small_kp(d)); }
int small_rows_per_block() { return kSmallWaves * 32; }
size_t small_f32_rec_bytes(int d) { return (size_t)f32_rec_bytes(small_kp(d)); }
size_t small_f16_rec_bytes(int d) { return small_kp(d) <= 2 ? (size_t)kF16RecBytes : 0; }
size_t small_b3_rec_bytes(int d) { return small_kp(d) <= 2 ? (size_t)kB3RecBytes : 0; }

hipError_t launch_lse_small_sparse(const LseArgs& a, hipStream_t s, hipEvent_t ev_begin) {
    if (a.n_split < 2 || !a.bs_list || !a.bs_count || !a.part || !a.bs_nsplit || !a.bs_map ||
        !a.bs_total || a.bs_grid < 1)
        return hipErrorInvalidValue;
    switch (small_kp(a.dp)) {
        case 1: return small_launch<1, true>(a, s, ev_begin);
        case 2: return small_launch<2, true>(a, s, ev_begin);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_lse_small(const LseArgs& a, hipStream_t s, hipEvent_t ev_begin) {
    switch (small_kp(a.dp)) {
        case 1: return small_launch<1>(a, s, ev_begin);
        case 2: return small_launch<2>(a, s, ev_begin);
        case 3: return small_launch<3>(a, s, ev_begin);
        case 4: return small_launch<4>(a, s, ev_begin);
        case 5: return small_launch<5>(a, s, ev_begin);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fs
