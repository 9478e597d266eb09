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
// Kernel families (the default d <= 8 path, lse_small_kernel, is in
// fs_lse_small.hip):
//  * lse_valu_kernel<D, R>: d <= 8, fp32 vector path.  Each lane owns R rows;
//    keys are wave-uniform (scalar loads), scores are D fp32 FMAs per pair.
//    The bound is the vector ALU / transcendental issue rate (one exp2 per
//    pair).
//  * lse_mfma_kernel<OP, NG, QB, WAVES>: d > 8.  The transposed score tile
//    S^T = K~ Q~^T is formed on the gfx950 matrix cores
//    (v_mfma_f32_32x32x{16_bf16,16_f16,2f32}), so every lane holds 16 scores of
//    ONE row and the row reduction stays inside the lane.  The row block
//    (WAVES x 32*QB rows x dp) lives in registers; 32-key tiles stream
//    through LDS slots in an XOR-swizzled layout.  The bound is the
//    matrix-core rate (2 n m d flops per half-step).
//  * lse_wide_kernel<OP>: two-byte scores at dp = 1024, the contraction split
//    over the two waves of each SIMD (see its comment).
// All can split the key range across workgroups (partial (max, sum) pairs
// merged afterwards in a fixed order), so results are deterministic.
#include <type_traits>

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
constexpr int kMfmaWaves = 8;    // waves per workgroup of the matrix-core kernel
constexpr int kQbMax = 2;        // cap on 32-row blocks per wave
constexpr int kAPipe = 8;        // operand fragments in flight, one wave per SIMD
constexpr int kAPipe8 = 4;       // operand fragments in flight, two waves per SIMD
constexpr int kValuPerSlot = 6;  // epilogue instructions per operand fragment (one wave per SIMD)
// Lazy reference: a tile's terms 2^(z2 - R) are summed against the running
// reference R as they come; only when some lane's tile sum is not at most
// this bound (a score more than ~64 above R, or R still -inf) does the wave
// move R to the exact running maximum and rescale.
constexpr float kLazyBound = 0x1p64f;


template <int OP, class TA, class TB>
__device__ __forceinline__ f32x16 mfma_step(const TA& av, const TB& bv, f32x16 acc) {
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

// Pipeline depth (key-tile buffers) and the largest key range per workgroup
// whose biases fit next to them in LDS (163,840 bytes on gfx950).
constexpr int kLdsBytes = 163840;
constexpr int nbuf_for(int ng) { return ng >= 64 ? 2 : 4; }
constexpr int tile_bytes_for(int ng) { return kKeyTile * 2 * ng * 16; }
// (a whole number of 256-key slices, the granule of the biases' copy to LDS)
constexpr int kps_max_for(int ng) {
    return ((kLdsBytes - nbuf_for(ng) * tile_bytes_for(ng) - 2048) / 4 / 256 * 256) < 16384
               ? (kLdsBytes - nbuf_for(ng) * tile_bytes_for(ng) - 2048) / 4 / 256 * 256
               : 16384;
}

// OP: score element type.  NG: 16-byte chunk pairs per operand row (a row is
// 2*NG chunks; dp = 16*NG for 2-byte types, 8*NG for fp32).  QB: 32-row
// blocks per wave.  WAVES: waves per workgroup.  NBUF: key-tile buffers.
//
// Software pipeline over 32-key tiles with one workgroup barrier per tile.
// Stage s:
//   (1) direct global->LDS loads (global_load_lds_dwordx4) of tile s+NBUF-1
//       into the buffer tile s-1 used, so a tile has NBUF-1 stages to arrive;
//   (2) the scores of tile s: matrix instructions with the resident row block
//       as one operand and key fragments streamed from LDS through a ring of
//       AP registers as the other;
//   (3) an online-LSE epilogue: of tile s right after (2), or of tile s-1
//       before or threaded through (2) (see below);
//   (4) wait until tile s+1 has landed (later tiles stay in flight), barrier.
// Eight waves (two per SIMD): the two halves of the workgroup run opposite
// orders -- waves 0-3 do scores then epilogue of tile s, waves 4-7 the
// epilogue of tile s-1 then the scores of tile s -- so that each SIMD's matrix
// pipe is fed by one wave while the other runs vector/transcendental work,
// and every wave has a single accumulator set live during its matrix phase.
// With tiles of at most 8 KiB the eight waves take two tiles per stage
// (TWO_TILES below).  Four waves (one per SIMD, larger row blocks): the
// epilogue of tile s-1 is threaded between the matrix instructions of tile s
// in four fenced chunks.  The key biases of the workgroup's whole key range
// are copied into LDS once, up front.  Tiles are stored XOR-swizzled (chunk c of key m at
// m*CPR + (c ^ (m & SWZ))) so that one operand fetch hits distinct banks.
template <int OP, int NG, int QB, int WAVES>
__global__ __launch_bounds__(WAVES * 64, 1) void lse_mfma_kernel(LseArgs a) {
    constexpr int CPR = 2 * NG;                      // 16-byte chunks per row
    constexpr int ROW_BYTES = CPR * 16;
    constexpr int TILE_CHUNKS = kKeyTile * CPR;      // chunks per key tile (>= 64)
    constexpr int TILE_INSTR = TILE_CHUNKS / 64;     // wave-wide 1 KiB loads per tile
    // With two waves per SIMD the tile loads are issued by the four lagging
    // waves only (whose epilogue phase has issue slots to spare), so the
    // leading waves go from the barrier straight into their matrix work.
    constexpr bool LAG_DMA = WAVES == 8;
    constexpr int DMA_WAVES = LAG_DMA ? WAVES / 2 : WAVES;
    constexpr int INSTR_PER_WAVE = (TILE_INSTR + DMA_WAVES - 1) / DMA_WAVES;
    constexpr int MIN_INSTR = TILE_INSTR / DMA_WAVES;  // loads per tile of every loading wave
    constexpr int NBUF = nbuf_for(NG);
    constexpr int KPS_MAX = kps_max_for(NG);
    constexpr int SWZ = CPR >= 16 ? 15 : CPR - 1;
    constexpr int JB = SWZ + 1 < 2 * NG ? (SWZ + 1) / 2 : NG;  // chunk-pair classes
    constexpr int APW = WAVES == 8 ? kAPipe8 : kAPipe;
    constexpr int AP = APW < NG ? APW : NG;          // operand fragments in flight
    constexpr int MF_PER_FRAG = QB * (OP == OP_F32 ? 4 : 1);
    static_assert(NBUF == 2 || NBUF == 4, "pipeline depth");
    // Tiles of at most 8 KiB (two-byte rows to 128 values, fp32 to 64) take
    // two per barrier: their stages are short, so the barrier costs more
    // than the shallower load pipeline (measured: bf16 at 64 / 128 values
    // 7.5% / 3.5% faster, fp32 at 64 2.4%; bf16 at 256 and 512 values 6.5% /
    // 5.6% slower with two per barrier).
    constexpr bool TWO_TILES = WAVES == 8 && NBUF == 4 && NG <= 8;

    constexpr int TILE_BYTES = TILE_CHUNKS * 16;
    __shared__ __attribute__((aligned(16))) uint4 kbuf[NBUF * TILE_CHUNKS];
    __shared__ __attribute__((aligned(16))) float bkeys[KPS_MAX];  // KPS_MAX: whole 1 KiB slices
    __shared__ float red[16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 31;  // query row of the B block / key row of the A block
    const int h = lane >> 5;   // lane half: contraction slots 8h..8h+7 of each 16

    int row_block, split;
    xcd_work(row_block, split);
    const int row0 = row_block * (WAVES * 32 * QB) + wave * (32 * QB);
    const int j0 = split * a.keys_per_split;
    const int j1 = min(a.n_keys, j0 + a.keys_per_split);
    const int ntiles = (j1 - j0 + kKeyTile - 1) / kKeyTile;
    const char* __restrict__ keys = (const char*)a.keys;

    // (1) tile k -> LDS buffer `dst` (64-chunk slice L of the tile per
    // wave-instruction; lane `lane` fetches the chunk that lands at position
    // L*64+lane of the swizzled layout).  For rows of >= 64 chunks a slice
    // lies in one key row m, so the source is a uniform base plus the lane's
    // swizzled chunk, (lane ^ (m & SWZ)) * 16, formed at issue time.
    const uint32_t lane16 = (uint32_t)lane * 16u;
    const int dwave = LAG_DMA ? wave - WAVES / 2 : wave;  // index among the loading waves
    auto issue_tile = [&](int k, uint4* dst) __attribute__((always_inline)) {
        const char* tbase = keys + (int64_t)(j0 + k * kKeyTile) * ROW_BYTES;
#pragma unroll
        for (int l = 0; l < INSTR_PER_WAVE; ++l) {
            const int L = l * DMA_WAVES + dwave;
            if (TILE_INSTR % DMA_WAVES == 0 || L < TILE_INSTR) {
                if constexpr (CPR >= 64) {
                    constexpr int IPR = CPR / 64;  // slices per key row
                    const int m = L / IPR;
                    uint32_t sw = (uint32_t)(m & SWZ) * 16u;
                    asm volatile("" : "+s"(sw));  // no hoisted per-lane offsets
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
    };
    auto buf = [&](int i) __attribute__((always_inline)) -> uint4* {
        return kbuf + i * TILE_CHUNKS;
    };

    // Prologue: the resident row block, tiles 0..NBUF-2 (every split holds
    // at least one key; the guard keeps an empty range from reading before
    // it) and the key biases of the whole range, all in flight at once and
    // waited for together.  The biases come from a_kbias, written once per
    // pass by key_seed_kernel in dot-product units: the base-2 score of a pair
    // is c_score * (x~.y~ + bk) with bk = (g - |y~|^2)/2 + log2(b)/(2 c_bias)
    // (c_score = 2 c_bias exactly), so bk can seed the accumulator.  They are
    // copied in 1 KiB slices (256 keys) straight into LDS; the seed array is
    // padded so that the last slice stays inside it.
    // lane (ln, h) holds chunk 2g+h of row row0+qb*32+ln.  With one wave
    // per SIMD and a block of more than 128 registers it is placed in the
    // accumulation registers (AGPRs), which the matrix instructions read
    // directly, leaving the vector registers to the accumulators, operand
    // ring and epilogue.
    constexpr bool Q_AGPR = WAVES == 4 && QB * NG * 4 > 128;
    auto issue_prologue_dma = [&]() __attribute__((always_inline)) {
        if (ntiles > 0 && (!LAG_DMA || dwave >= 0)) {
            constexpr int PRE = TWO_TILES ? 2 : NBUF - 1;
#pragma unroll
            for (int k = 0; k < PRE; ++k) issue_tile(min(k, ntiles - 1), buf(k));
        }
        const int slices = (ntiles * kKeyTile + 255) / 256;
        const char* kb = (const char*)(a.kbias + j0);
        for (int c = wave; c < slices; c += WAVES) dma_to_lds16(kb + c * 1024, lane16, bkeys + c * 256);
    };
    u32x4 q[QB][NG];
    {
        const char* __restrict__ rows = (const char*)a.rows;
        // Either way the block is consumed in the prologue, so that the
        // compiler's own waits for these loads are placed there: left to
        // their first use inside the tile loop they would be re-executed
        // every tile, and there they would also wait for the tile loads in
        // flight.  Vector-register blocks: all loads, then the copies, then
        // one wait for everything.  AGPR blocks: the copies first, then the
        // loads in batches of QLB staged in vector registers on the way.
        constexpr int QLB = Q_AGPR ? 8 : NG;
        if constexpr (Q_AGPR) issue_prologue_dma();
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const char* rp = rows + (int64_t)(row0 + qb * 32 + ln) * ROW_BYTES + h * 16;
#pragma unroll
            for (int g0 = 0; g0 < NG; g0 += QLB) {
                u32x4 v[QLB];
#pragma unroll
                for (int u = 0; u < QLB; ++u)
                    if (g0 + u < NG) v[u] = *(const u32x4*)(rp + (g0 + u) * 32);
#pragma unroll
                for (int u = 0; u < QLB; ++u) {
                    if (g0 + u >= NG) continue;
                    if constexpr (Q_AGPR)
                        asm volatile("" : "=a"(q[qb][g0 + u]) : "0"(v[u]));
                    else
                        q[qb][g0 + u] = v[u];
                }
            }
        }
        if constexpr (!Q_AGPR) {
            issue_prologue_dma();
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int g = 0; g < NG; ++g) asm volatile("" ::"v"(q[qb][g]));
        }
    }

    float M[QB], S[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        M[qb] = -INFINITY;
        S[qb] = 0.f;
    }

    // (2) scores of one tile for all QB row blocks.  Operand chunk 2g+h of key
    // ln sits at ln*CPR + ((2g+h) ^ (ln & SWZ)); with g = JB*k + j that is a
    // per-lane base for each j plus the immediate offset 2*JB*k chunks.  The
    // fragments are software-pipelined: a ring of AP operand registers keeps
    // AP LDS reads in flight ahead of the matrix instruction that consumes
    // them, and the schedule is pinned to that order (left alone, the
    // scheduler sinks each read next to its use and every matrix instruction
    // waits out a full LDS round trip).
    // An LDS read takes a 16-bit immediate offset, so slots that start at or
    // beyond 64 KiB address from a second set of bases, abase + 64 KiB.  With
    // two waves per SIMD there are registers to spare and the set is kept in
    // registers (opaque to the compiler, which would otherwise form every
    // such fragment address with a vector add in every stage); with one wave
    // per SIMD the resident block leaves none, and the adds stay.
    constexpr bool HI_BASES = WAVES == 8 && NBUF * TILE_BYTES > 0x10000;
    int abase[JB], abase_hi[JB];
#pragma unroll
    for (int j = 0; j < JB; ++j) {
        abase[j] = (ln * CPR + ((2 * j + h) ^ (ln & SWZ))) * 16;
        abase_hi[j] = abase[j] + 0x10000;
        if constexpr (HI_BASES) asm volatile("" : "+v"(abase_hi[j]));
    }
    // fragment g of the tile in slot I
    auto frag = [&](auto i_c, int g) __attribute__((always_inline)) -> uint4 {
        constexpr int OFF = decltype(i_c)::value * TILE_BYTES;
        const char* base = (const char*)kbuf;
        if constexpr (OFF >= 0x10000)
            return *(const uint4*)(base + abase_hi[g % JB] + (OFF - 0x10000) +
                                   (g / JB) * (2 * JB * 16));
        else
            return *(const uint4*)(base + abase[g % JB] + OFF + (g / JB) * (2 * JB * 16));
    };
    // Start a tile: seed the accumulators with the tile's key biases
    // (accumulator register r of lane (ln, h) holds the pair of row ln with
    // key 8*(r/4) + 4*h + (r%4) of the tile) and put the first AP fragments
    // in flight.
    auto ring_begin = [&](auto i_c, const float* bb, uint4 (&av)[AP], f32x16 (&acc)[QB])
                          __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const float4 v = *(const float4*)&bb[8 * qq + 4 * h];
                acc[qb][4 * qq + 0] = v.x;
                acc[qb][4 * qq + 1] = v.y;
                acc[qb][4 * qq + 2] = v.z;
                acc[qb][4 * qq + 3] = v.w;
            }
#pragma unroll
        for (int g = 0; g < AP; ++g) av[g] = frag(i_c, g);
    };
    // fragments [G0, G1): their matrix instructions, each followed by the
    // read that refills its ring slot with fragment g + AP
    auto ring_steps = [&](auto i_c, uint4 (&av)[AP], f32x16 (&acc)[QB], auto g0_c,
                          auto g1_c) __attribute__((always_inline)) {
        constexpr int G0 = decltype(g0_c)::value;
        constexpr int G1 = decltype(g1_c)::value;
#pragma unroll
        for (int g = G0; g < G1; ++g) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) acc[qb] = mfma_step<OP>(av[g % AP], q[qb][g], acc[qb]);
            if (g + AP < NG) av[g % AP] = frag(i_c, g + AP);
        }
    };
    // Pins the order of the current scheduling region for fragments
    // [G0, G1): (the ring's first AP reads if FIRST), then per fragment its
    // matrix instructions, its refill read and up to VPS vector instructions.
    auto pin_steps = [&](auto g0_c, auto g1_c, auto first_c, auto vps_c)
                         __attribute__((always_inline)) {
        constexpr int G0 = decltype(g0_c)::value;
        constexpr int G1 = decltype(g1_c)::value;
        constexpr bool FIRST = decltype(first_c)::value;
        constexpr int VPS = decltype(vps_c)::value;
        {
            if constexpr (FIRST) __builtin_amdgcn_sched_group_barrier(0x100, AP + 4 * QB, 0);
#pragma unroll
            for (int g = G0; g < G1; ++g) {
                __builtin_amdgcn_sched_group_barrier(0x008, MF_PER_FRAG, 0);
                if (g + AP < NG) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                if (VPS > 0) __builtin_amdgcn_sched_group_barrier(0x002, VPS, 0);
            }
        }
    };
    using Zero = std::integral_constant<int, 0>;
    using NGc = std::integral_constant<int, NG>;
    // the whole score tile (key biases `bb`) in one pinned region
    auto mfma_tile = [&](auto i_c, const float* bb, f32x16 (&acc)[QB])
                         __attribute__((always_inline)) {
        uint4 av[AP];
        ring_begin(i_c, bb, av, acc);
        ring_steps(i_c, av, acc, Zero{}, NGc{});
        pin_steps(Zero{}, NGc{}, std::true_type{}, Zero{});
    };

    // (3) online LSE of one tile from its accumulators (scores c_score*acc,
    // c_score > 0).  In parts, so it can be spread over a tile's matrix work:
    // the tile maximum and the rescaled running sum; then the exponentials
    // of scores [R0, R1); then the commit of the new state.  A lane that has
    // seen no key yet (every score -inf) keeps the empty state.
    struct EpiState {
        float Mn[QB];
        float sh[QB];
        float s[QB];
    };
    auto epi_max = [&](const f32x16 (&acc)[QB], EpiState& e) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float tmax = fmaxf(acc[qb][0], acc[qb][1]);
#pragma unroll
            for (int r = 2; r < 16; ++r) tmax = fmaxf(tmax, acc[qb][r]);
            e.Mn[qb] = fmaxf(M[qb], a.c_score * tmax);
            e.sh[qb] = e.Mn[qb] == -INFINITY ? 0.f : e.Mn[qb];
            e.s[qb] = S[qb] * ex2(M[qb] - e.sh[qb]);
        }
    };
    auto epi_exps = [&](const f32x16 (&acc)[QB], EpiState& e, auto r0_c, auto r1_c)
                        __attribute__((always_inline)) {
        constexpr int R0 = decltype(r0_c)::value;
        constexpr int R1 = decltype(r1_c)::value;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int r = R0; r < R1; ++r) e.s[qb] += ex2(fmaf(acc[qb][r], a.c_score, -e.sh[qb]));
    };
    auto epi_commit = [&](EpiState& e) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            S[qb] = e.s[qb];
            M[qb] = e.Mn[qb];
            // keep the epilogue ahead of the stage's load wait and barrier
            asm volatile("" : "+v"(S[qb]), "+v"(M[qb]));
        }
    };
    auto epilogue = [&](const f32x16 (&acc)[QB]) __attribute__((always_inline)) {
        EpiState e;
        epi_max(acc, e);
        epi_exps(acc, e, Zero{}, std::integral_constant<int, 16>{});
        epi_commit(e);
    };
    // The same state update with a lazy reference: (M, S) keeps meaning
    // M + log2(S) = LSE2 of the keys seen, but M is only a valid shift, moved
    // to the running maximum when a tile's terms against it would not stay
    // below kLazyBound (always on the first tile, when M is -inf).  Saves the
    // tile maximum and the rescale on the common path.
    auto epilogue_lazy = [&](const f32x16 (&acc)[QB]) __attribute__((always_inline)) {
        float t[QB];
        bool slow = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float e[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) e[r] = ex2(fmaf(acc[qb][r], a.c_score, -M[qb]));
#pragma unroll
            for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
                for (int r = 0; r < w; ++r) e[r] += e[r + w];
            t[qb] = e[0];
            slow = slow || !(t[qb] <= kLazyBound);
        }
        if (__builtin_amdgcn_ballot_w64(slow)) {
            EpiState x;
            epi_max(acc, x);
            epi_exps(acc, x, Zero{}, std::integral_constant<int, 16>{});
            epi_commit(x);
        } else {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                S[qb] += t[qb];
                asm volatile("" : "+v"(S[qb]), "+v"(M[qb]));
            }
        }
    };
    // One wave per SIMD: the scores of one tile (biases `bb`) into `acc` and
    // the epilogue of the previous tile (`prev`) in four fenced chunks, each
    // pinned to alternate matrix instructions, operand reads and epilogue
    // instructions.
    auto fused_chunks = [&](auto i_c, const float* bb, f32x16 (&acc)[QB],
                            const f32x16 (&prev)[QB]) __attribute__((always_inline)) {
        constexpr int C = NG >= 4 ? NG / 4 : 1;  // fragments per chunk
        using C1 = std::integral_constant<int, (C < NG ? C : NG)>;
        using C2 = std::integral_constant<int, (2 * C < NG ? 2 * C : NG)>;
        using C3 = std::integral_constant<int, (3 * C < NG ? 3 * C : NG)>;
        using V = std::integral_constant<int, kValuPerSlot>;
        uint4 av[AP];
        EpiState e;
        ring_begin(i_c, bb, av, acc);
        ring_steps(i_c, av, acc, Zero{}, C1{});
        epi_max(prev, e);
        pin_steps(Zero{}, C1{}, std::true_type{}, V{});
        __builtin_amdgcn_sched_barrier(0);
        ring_steps(i_c, av, acc, C1{}, C2{});
        epi_exps(prev, e, Zero{}, std::integral_constant<int, 6>{});
        pin_steps(C1{}, C2{}, std::false_type{}, V{});
        __builtin_amdgcn_sched_barrier(0);
        ring_steps(i_c, av, acc, C2{}, C3{});
        epi_exps(prev, e, std::integral_constant<int, 6>{}, std::integral_constant<int, 11>{});
        pin_steps(C2{}, C3{}, std::false_type{}, V{});
        __builtin_amdgcn_sched_barrier(0);
        ring_steps(i_c, av, acc, C3{}, NGc{});
        epi_exps(prev, e, std::integral_constant<int, 11>{}, std::integral_constant<int, 16>{});
        pin_steps(C3{}, NGc{}, std::false_type{}, V{});
        epi_commit(e);
    };
    // (4) wait until at most `newer` tiles' loads are outstanding for this
    // wave (loads complete in order, so the older tiles have landed).
    auto wait_tiles = [&](auto newer_c) __attribute__((always_inline)) {
        constexpr int NEWER = decltype(newer_c)::value;
        if constexpr (MIN_INSTR == 0 || NEWER <= 0)
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NEWER * MIN_INSTR) : "memory");
    };

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // waves whose epilogue runs one tile behind their scores
    const bool lagging = WAVES != 8 || wave >= 4;
    // One stage (tile s in buffer slot I = s % NBUF; the load of tile
    // s+NBUF-1 goes to slot I-1, which every wave finished reading before the
    // previous barrier).  Past the end the load is clamped to the last tile:
    // a redundant in-bounds copy into a slot that is never read again, which
    // keeps the wait count constant.
    auto stage = [&](int s, auto i_c, f32x16 (&acc)[QB], f32x16 (&prev)[QB])
                     __attribute__((always_inline)) {
        constexpr int I = decltype(i_c)::value;
        if constexpr (!LAG_DMA) {
            issue_tile(min(s + NBUF - 1, ntiles - 1), buf((I + NBUF - 1) % NBUF));
            __builtin_amdgcn_sched_barrier(0);
        }
        const float* bb = bkeys + s * kKeyTile;
        if constexpr (WAVES == 8) {
            if (!lagging) {
                mfma_tile(i_c, bb, acc);
                __builtin_amdgcn_sched_barrier(0);
                epilogue_lazy(acc);
            } else {
                if constexpr (LAG_DMA) {
                    issue_tile(min(s + NBUF - 1, ntiles - 1), buf((I + NBUF - 1) % NBUF));
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (s > 0) epilogue_lazy(prev);
                __builtin_amdgcn_sched_barrier(0);
                mfma_tile(i_c, bb, acc);
            }
        } else {
            if (s > 0)
                fused_chunks(i_c, bb, acc, prev);
            else
                mfma_tile(i_c, bb, acc);
        }
        wait_tiles(std::integral_constant<int, NBUF - 2>{});
        stage_barrier();
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    f32x16 accA[QB], accB[QB];
    if constexpr (TWO_TILES) {
        // Two tiles per stage: leading waves scores(s), epilogue(s),
        // scores(s+1), epilogue(s+1); lagging waves epilogue(s-1), scores(s),
        // epilogue(s), scores(s+1) -- the same per-wave tile order and state
        // updates as one tile per stage, with half the barriers; the tiles of
        // the next stage load during this one.
        auto dstage = [&](int s, auto i_c, auto j_c) __attribute__((always_inline)) {
            constexpr int I = decltype(i_c)::value;
            const bool two = s + 1 < ntiles;
            const float* bb = bkeys + s * kKeyTile;
            if (!lagging) {
                mfma_tile(i_c, bb, accA);
                __builtin_amdgcn_sched_barrier(0);
                epilogue_lazy(accA);
                if (two) {
                    __builtin_amdgcn_sched_barrier(0);
                    mfma_tile(j_c, bb + kKeyTile, accB);
                    __builtin_amdgcn_sched_barrier(0);
                    epilogue_lazy(accB);
                }
            } else {
                issue_tile(min(s + 2, ntiles - 1), buf((I + 2) % 4));
                issue_tile(min(s + 3, ntiles - 1), buf((I + 3) % 4));
                __builtin_amdgcn_sched_barrier(0);
                if (s > 0) epilogue_lazy(accB);
                __builtin_amdgcn_sched_barrier(0);
                mfma_tile(i_c, bb, accA);
                if (two) {
                    __builtin_amdgcn_sched_barrier(0);
                    epilogue_lazy(accA);
                    __builtin_amdgcn_sched_barrier(0);
                    mfma_tile(j_c, bb + kKeyTile, accB);
                }
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            stage_barrier();
        };
        for (int t = 0; t < ntiles; t += 4) {
            dstage(t, I0{}, I1{});
            if (t + 2 < ntiles) dstage(t + 2, I2{}, I3{});
        }
        if (lagging && ntiles > 0) {
            if (ntiles % 2 == 0)
                epilogue(accB);
            else
                epilogue(accA);
        }
    } else {
        for (int t = 0; t < ntiles; t += NBUF) {
            stage(t, I0{}, accA, accB);
            if (t + 1 < ntiles) stage(t + 1, I1{}, accB, accA);
            if constexpr (NBUF > 2) {
                if (t + 2 < ntiles) stage(t + 2, I2{}, accA, accB);
                if (t + 3 < ntiles) stage(t + 3, I3{}, accB, accA);
            }
        }
        // the lagging waves' epilogue of the last tile
        if (lagging && ntiles > 0) {
            if ((ntiles - 1) % 2 == 0)
                epilogue(accA);
            else
                epilogue(accB);
        }
    }
    // No tile load may still be writing this workgroup's LDS when it exits.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

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
        if (tid == 0) a.resid_part[row_block] = resid;
    }
}

// ------------------------------------- 1024-wide rows: split contraction
// Key biases of one pass in dot-product units (the seeds of the score
// accumulators, as in lse_mfma_kernel): kb[j] = (pot_j - nrm_j)/2 +
// log2(w_j)/(2 c_bias), -inf for the padding keys.
__global__ __launch_bounds__(256) void key_seed_kernel(LseArgs a) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= a.kbias_keys) return;
    a.kbias[j] = j < a.n_keys ? fmaf(a.key_lw2[j], 0.5f / a.c_bias,
                                     0.5f * (a.key_pot[j] - a.key_nrm[j]))
                              : -INFINITY;
}

// Rows of 1024 two-byte values are too wide for two waves per SIMD to each
// hold a 32-row block (256 registers), and one wave per SIMD that reads a
// key fragment from LDS for every matrix instruction cannot keep the matrix
// pipe busy.  So the contraction is split: the two waves of a SIMD (w and
// w+4) hold the SAME 32 rows, wave w the first 512 values of each row and
// wave w+4 the last 512, and each forms the partial scores of its half for
// all 32 keys of a tile.  Each finalises 16 of the tile's keys -- wave w keys
// 0-15 (accumulator registers 0-7), wave w+4 keys 16-31 (registers 8-15) --
// after adding the partner's partial for those keys, passed through LDS.
// The key biases seed wave w's partials only, so every score gets them once.
//
// Stage s (tile s in slot s%2; the next tile's load into the other slot):
//   wave w   : scores of tile s (its half) -> write registers 8-15 for the
//              partner -> epilogue of tile s-1 (its registers 0-7 of that
//              tile plus the partner's, written in stage s-1);
//   wave w+4 : issue the loads of tile s+1 -> epilogue of tile s-1 (registers
//              8-15 plus the partner's) -> scores of tile s -> write
//              registers 0-7 for the partner;
//   wait for the loads, barrier.
// The two waves of a SIMD thus run opposite phases (matrix / vector), and the
// exchange buffers alternate by tile parity, so a buffer is rewritten only
// two stages after it was written, one barrier after it was read.  The LSE
// state uses the lazy reference of the two-wave kernel.  At the end the two
// halves of each row's key set are merged through LDS, then the lane halves.
template <int OP>
__global__ __launch_bounds__(512, 1) void lse_wide_kernel(LseArgs a) {
    constexpr int CPR = 128;                  // 16-byte chunks per row
    constexpr int ROW_BYTES = CPR * 16;       // 2 KiB
    constexpr int TILE_CHUNKS = kKeyTile * CPR;
    constexpr int TILE_BYTES = TILE_CHUNKS * 16;  // 64 KiB
    constexpr int HG = 32;                    // fragments per half row
    constexpr int JB = 8;
    constexpr int AP = 4;
    __shared__ __attribute__((aligned(16))) uint4 kbuf[2 * TILE_CHUNKS];  // 128 KiB
    // [tile parity][row group][direction][quad][lane]: direction 0 carries
    // registers 8-15 (to the second wave), 1 registers 0-7 (to the first)
    __shared__ __attribute__((aligned(16))) float4 xbuf[2][4][2][2][64];    // 32 KiB

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rg = wave & 3, dh = wave >> 2;  // row group, contraction half
    const bool first = dh == 0;
    const int ln = lane & 31, h = lane >> 5;
    int row_block, split;
    xcd_work(row_block, split);
    const int row0 = row_block * 128 + rg * 32;
    const int j0 = split * a.keys_per_split;
    const int j1 = min(a.n_keys, j0 + a.keys_per_split);
    const int ntiles = (j1 - j0 + kKeyTile - 1) / kKeyTile;
    const char* __restrict__ keys = (const char*)a.keys;

    // Tile loads: 64 slices of 1 KiB (half a key row each); the first waves
    // issue 16 each, one after every other matrix instruction.
    constexpr int SHARE = 16;
    const bool loader = first;
    const uint32_t lane16 = (uint32_t)lane * 16u;
    auto issue_slice = [&](int k, int slot, int l) __attribute__((always_inline)) {
        const int L = l * 4 + rg;
        const char* tbase = keys + (int64_t)(j0 + k * kKeyTile) * ROW_BYTES;
        const int m = L >> 1;
        uint32_t sw = (uint32_t)(m & 15) * 16u;
        asm volatile("" : "+s"(sw));
        dma_to_lds16(tbase + m * ROW_BYTES + (L & 1) * 1024, lane16 ^ sw,
                     kbuf + slot * TILE_CHUNKS + L * 64);
    };
    auto issue_tile = [&](int k, int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int l = 0; l < SHARE; ++l) issue_slice(k, slot, l);
    };
    if (loader && ntiles > 0) issue_tile(0, 0);

    // this wave's half of the resident rows: fragment g is chunk
    // 64 dh + 2g + h of row row0 + ln
    u32x4 q[HG];
    {
        const char* rp = (const char*)a.rows + (int64_t)(row0 + ln) * ROW_BYTES + (dh * 64 + h) * 16;
#pragma unroll
        for (int g = 0; g < HG; ++g) q[g] = *(const u32x4*)(rp + g * 32);
        // consumed here, so the compiler's waits for these loads stay in the
        // prologue (all loads in flight first, then in-order waits)
#pragma unroll
        for (int g = 0; g < HG; ++g) asm volatile("" ::"v"(q[g]));
    }
    // key fragment g of this half: chunk 64 dh + 2g + h of key ln, stored at
    // ln*CPR + (chunk ^ (ln & 15)); the XOR stays inside the half's 64 chunks.
    // Slot 1 starts at 64 KiB, beyond an LDS read's immediate offset: it
    // addresses from a second, register-held set of bases.
    int abase[JB], abase_hi[JB];
#pragma unroll
    for (int j = 0; j < JB; ++j) {
        abase[j] = (ln * CPR + dh * 64 + ((2 * j + h) ^ (ln & 15))) * 16;
        abase_hi[j] = abase[j] + TILE_BYTES;
        asm volatile("" : "+v"(abase_hi[j]));
    }
    auto frag = [&](auto slot_c, int g) __attribute__((always_inline)) -> uint4 {
        const char* base = (const char*)kbuf;
        if constexpr (decltype(slot_c)::value == 1)
            return *(const uint4*)(base + abase_hi[g % JB] + (g / JB) * 256);
        else
            return *(const uint4*)(base + abase[g % JB] + (g / JB) * 256);
    };
    // key biases of tile k for this lane's accumulator order (first waves)
    const float* __restrict__ kb = a.kbias + j0;
    auto load_bias = [&](int k, float4 (&bv)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) bv[qq] = *(const float4*)(kb + k * kKeyTile + 8 * qq + 4 * h);
    };
    float4 bnext[4];
    if (first && ntiles > 0) load_bias(0, bnext);

    // partial scores of tile (slot SL) into acc; with DE > 0, slice l of tile
    // kd goes to the other slot after matrix instruction DE*l + DE-1
    auto scores = [&](auto slot_c, f32x16& acc, auto de_c, int kd) __attribute__((always_inline)) {
        constexpr int DE = decltype(de_c)::value;
        if (first) {
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                acc[4 * qq + 0] = bnext[qq].x;
                acc[4 * qq + 1] = bnext[qq].y;
                acc[4 * qq + 2] = bnext[qq].z;
                acc[4 * qq + 3] = bnext[qq].w;
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.f;
        }
        uint4 av[AP];
#pragma unroll
        for (int g = 0; g < AP; ++g) av[g] = frag(slot_c, g);
#pragma unroll
        for (int g = 0; g < HG; ++g) {
            acc = mfma_step<OP>(av[g % AP], q[g], acc);
            if (g + AP < HG) av[g % AP] = frag(slot_c, g + AP);
            if constexpr (DE > 0)
                if (g % DE == DE - 1) issue_slice(kd, 1 - decltype(slot_c)::value, g / DE);
        }
        {
            __builtin_amdgcn_sched_group_barrier(0x100, AP, 0);
#pragma unroll
            for (int g = 0; g < HG; ++g) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (g + AP < HG) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }
    };
    // the partner's registers for this wave's keys
    auto put = [&](const f32x16& acc, int par) __attribute__((always_inline)) {
        const int base = first ? 8 : 0;  // registers the partner finalises
        float4* dst = &xbuf[par][rg][first ? 0 : 1][0][0];
        dst[lane] = make_float4(acc[base + 0], acc[base + 1], acc[base + 2], acc[base + 3]);
        dst[64 + lane] = make_float4(acc[base + 4], acc[base + 5], acc[base + 6], acc[base + 7]);
    };
    // online LSE over this wave's 16 keys of a tile: own registers plus the
    // partner's (lazy reference as in lse_mfma_kernel)
    float M = -INFINITY, S = 0.f;
    auto epilogue = [&](const f32x16& acc, int par) __attribute__((always_inline)) {
        const int base = first ? 0 : 8;
        const float4* src = &xbuf[par][rg][first ? 1 : 0][0][0];
        const float4 p0 = src[lane], p1 = src[64 + lane];
        float v[8] = {acc[base + 0] + p0.x, acc[base + 1] + p0.y, acc[base + 2] + p0.z,
                      acc[base + 3] + p0.w, acc[base + 4] + p1.x, acc[base + 5] + p1.y,
                      acc[base + 6] + p1.z, acc[base + 7] + p1.w};
        float e[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) e[r] = ex2(fmaf(v[r], a.c_score, -M));
#pragma unroll
        for (int w = 4; w >= 1; w >>= 1)
#pragma unroll
            for (int r = 0; r < w; ++r) e[r] += e[r + w];
        if (__builtin_amdgcn_ballot_w64(!(e[0] <= kLazyBound))) {
            float tmax = v[0];
#pragma unroll
            for (int r = 1; r < 8; ++r) tmax = fmaxf(tmax, v[r]);
            const float Mn = fmaxf(M, a.c_score * tmax);
            const float sh = Mn == -INFINITY ? 0.f : Mn;
            float t = S * ex2(M - sh);
#pragma unroll
            for (int r = 0; r < 8; ++r) t += ex2(fmaf(v[r], a.c_score, -sh));
            S = t;
            M = Mn;
        } else {
            S += e[0];
        }
        asm volatile("" : "+v"(S), "+v"(M));
    };

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    f32x16 accA, accB;
    auto stage = [&](int s, auto slot_c, f32x16& acc, f32x16& prev) __attribute__((always_inline)) {
        using DF = std::integral_constant<int, 2>;  // a slice after every other matrix instruction
        using D0 = std::integral_constant<int, 0>;
        const int kn = min(s + 1, ntiles - 1);
        if (first) {
            scores(slot_c, acc, DF{}, kn);
            load_bias(min(s + 1, ntiles - 1), bnext);
            __builtin_amdgcn_sched_barrier(0);
            put(acc, s & 1);
            if (s > 0) epilogue(prev, (s - 1) & 1);
        } else {
            __builtin_amdgcn_sched_barrier(0);
            if (s > 0) epilogue(prev, (s - 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
            scores(slot_c, acc, D0{}, kn);
            put(acc, s & 1);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        stage_barrier();
    };
    for (int t = 0; t < ntiles; t += 2) {
        stage(t, S0{}, accA, accB);
        if (t + 1 < ntiles) stage(t + 1, S1{}, accB, accA);
    }
    // the epilogue of the last tile (its exchange landed before the last barrier)
    if (ntiles > 0) {
        if ((ntiles - 1) % 2 == 0)
            epilogue(accA, (ntiles - 1) & 1);
        else
            epilogue(accB, (ntiles - 1) & 1);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // every wave is done with the tile and exchange buffers

    // Merge the two key halves of each row (second wave -> first through
    // LDS), then the lane halves, and finish.
    float2* mrg = (float2*)kbuf;
    if (!first) mrg[rg * 64 + lane] = make_float2(M, S);
    __syncthreads();
    float resid = 0.f;
    if (first) {
        const float2 o = mrg[rg * 64 + lane];
        lse_merge(M, S, o.x, o.y);
        const float M2 = __shfl_xor(M, 32, 64);
        const float S2 = __shfl_xor(S, 32, 64);
        lse_merge(M, S, M2, S2);
        const int row = row0 + ln;
        if (h == 0 && row < a.n_rows) {
            if (a.n_split == 1)
                resid = finalize_row(a, row, M + lg2(S));
            else
                a.part[(int64_t)split * a.n_rows + row] = make_float2(M, S);
        }
    }
    if (a.n_split == 1 && a.cur) {
        // block_sum's first barrier orders the merge reads before its writes
        resid = block_sum(resid, (float*)kbuf);
        if (tid == 0) a.resid_part[row_block] = resid;
    }
}

// ----------------------------------------------------------------- merge
__global__ __launch_bounds__(256) void lse_merge_kernel(LseArgs a) {
    __shared__ float red[16];
    const int i = blockIdx.x * 256 + threadIdx.x;
    float r = 0.f;
    if (i < a.n_rows) {
        float M = -INFINITY, S = 0.f;
        const int ns = a.bs_nsplit ? a.bs_nsplit[i / 256] : a.n_split;  // block-sparse: per row block
        for (int s = 0; s < ns; ++s) {
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

constexpr int qb_cap(int qb) { return qb < kQbMax ? qb : kQbMax; }
// Eight waves (two per SIMD, 32 rows each) when a 32-row resident block fits
// in half the register file (ng * 4 <= 128 VGPRs); otherwise four.
constexpr int waves_for(int ng) { return kMfmaWaves == 8 && ng <= 32 ? 8 : 4; }
constexpr int qb_for(int op, int ng) {
    return waves_for(ng) == 8 ? 1
           : op == OP_F32      ? (ng <= 8 ? 4 : (ng <= 32 ? qb_cap(2) : 1))
                               : (ng <= 32 ? qb_cap(2) : 1);
}

template <int OP, int NG, int QB>
hipError_t mfma_launch(const LseArgs& a, hipStream_t s) {
    constexpr int W = waves_for(NG);
    constexpr int rpb = W * 32 * QB;
    const dim3 grid((a.n_rows + rpb - 1) / rpb, a.n_split);
    lse_mfma_kernel<OP, NG, QB, W><<<grid, W * 64, 0, s>>>(a);
    return hipGetLastError();
}

// 32-row blocks per wave: as many as the resident row block's registers allow
// (64 rows x 512 bf16 values = 256 VGPRs per lane), fewer for 8-wave groups.
template <int OP, int NG>
hipError_t mfma_launch_ng(const LseArgs& a, hipStream_t s) {
    return mfma_launch<OP, NG, qb_for(OP, NG)>(a, s);
}

template <int OP>
hipError_t mfma_dispatch(int ng, const LseArgs& a, hipStream_t s) {
    switch (ng) {
        case 1: return mfma_launch_ng<OP, 1>(a, s);
        case 2: return mfma_launch_ng<OP, 2>(a, s);
        case 4: return mfma_launch_ng<OP, 4>(a, s);
        case 8: return mfma_launch_ng<OP, 8>(a, s);
        case 16: return mfma_launch_ng<OP, 16>(a, s);
        case 32: return mfma_launch_ng<OP, 32>(a, s);
        case 64: return mfma_launch_ng<OP, 64>(a, s);
        default: return hipErrorInvalidValue;
    }
}

int mfma_qb(int path, int ng) {
    const int op = path == PATH_MFMA_F32 ? OP_F32 : OP_BF16;
    return qb_for(op, ng);
}

int ng_of(int path, int dp) { return path == PATH_MFMA_F32 ? dp / 8 : dp / 16; }


template <int OP>
hipError_t wide_launch(const LseArgs& a, hipStream_t s) {
    const dim3 grid((a.n_rows + 127) / 128, a.n_split);
    lse_wide_kernel<OP><<<grid, 512, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace

bool lse_wide(int path, int dp) {
    return (path == PATH_MFMA_BF16 || path == PATH_MFMA_F16) && dp == 1024;
}

// The vector path uses 4 rows per lane when there are enough rows to fill the
// GPU, else 1.
int valu_rows_per_lane(int n_rows) { return n_rows >= 65536 ? 4 : 1; }

int lse_max_keys_per_split(int path, int dp) {
    if (small_d_path(path) || lse_wide(path, dp)) return 1 << 30;
    return kps_max_for(ng_of(path, dp));
}

int lse_split_granule(int path, int dp) {
    if (path == PATH_VALU) return kValuTile;
    if (path == PATH_SMALL) return small_tile(dp);
    return kKeyTile;
}

int lse_rows_per_block(int path, int dp, int n_rows) {
    if (path == PATH_VALU) return 256 * valu_rows_per_lane(n_rows);
    if (path == PATH_SMALL) return small_rows_per_block();
    if (lse_wide(path, dp)) return 128;
    const int ng = ng_of(path, dp);
    return waves_for(ng) * 32 * mfma_qb(path, ng);
}

// For the vector path LseArgs::dp is the true dimension d (<= 8); operand rows
// are stored 4 (d <= 4) or 8 floats apart.  For the matrix paths it is the
// padded dimension.
hipError_t launch_lse(int path, const LseArgs& a, hipStream_t s, hipEvent_t ev_begin,
                      hipEvent_t ev_end) {
    hipError_t e;
    const bool wide = lse_wide(path, a.dp);
    if (!small_d_path(path)) {
        // the key seeds of the matrix-core kernels go first, outside the
        // kernel's timed bracket
        if (!a.kbias || a.kbias_keys < (a.n_keys + kKeyTile - 1) / kKeyTile * kKeyTile)
            return hipErrorInvalidValue;
        key_seed_kernel<<<(a.kbias_keys + 255) / 256, 256, 0, s>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (path == PATH_SMALL) {
        e = a.bs_list ? launch_lse_small_sparse(a, s, ev_begin) : launch_lse_small(a, s, ev_begin);
    } else if (ev_begin && (e = hipEventRecord(ev_begin, s)) != hipSuccess) {
        return e;
    } else if (wide) {
        e = path == PATH_MFMA_BF16 ? wide_launch<OP_BF16>(a, s) : wide_launch<OP_F16>(a, s);
    } else if (path == PATH_VALU) {
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
    if (ev_end && (e = hipEventRecord(ev_end, s)) != hipSuccess) return e;
    int fin_blocks;
    if (a.n_split > 1) {
        fin_blocks = (a.n_rows + 255) / 256;
        lse_merge_kernel<<<fin_blocks, 256, 0, s>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else if (path == PATH_VALU) {
        const int R = valu_rows_per_lane(a.n_rows);
        fin_blocks = (a.n_rows + 256 * R - 1) / (256 * R);
    } else {
        fin_blocks = (a.n_rows + lse_rows_per_block(path, a.dp, a.n_rows) - 1) /
                     lse_rows_per_block(path, a.dp, a.n_rows);
    }
    if (a.cur) {
        resid_reduce_kernel<<<1, 256, 0, s>>>(a.resid_part, fin_blocks, a.resid_out);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace fs
