// fs_device.hpp -- device-side helpers shared by the solver's HIP kernels.
//
// Everything is written for gfx950 (CDNA4): 64-lane wavefronts, the
// v_mfma_f32_32x32x{16_bf16,16_f16,2f32} matrix instructions, v_exp_f32 /
// v_log_f32 (base-2) transcendentals.  Log-sum-exps are carried in base 2
// (z2 = z * log2(e)); this is only a change of base of the pages' natural-log
// update ("FlashSinkhorn" explainer, "Method" part 1).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fs {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// 2^x and log2(x) on the transcendental unit (v_exp_f32 / v_log_f32).
// exp2(-inf) = 0, exp2 of very negative arguments flushes to 0.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

// One wave-wide 16-byte-per-lane global -> LDS copy (global_load_lds_dwordx4
// in its scalar-base form): lane i's 16 bytes at `gbase + voff_i` land at LDS
// byte address `lds_dst + 16*i`.  `gbase` and `lds_dst` must be wave-uniform.
// Issued as inline assembly so the compiler does not model it as an LDS
// store: the caller owns completion and waits for it explicitly (s_waitcnt
// vmcnt) before a barrier publishes it.  M0 (the LDS destination register of
// the instruction) is saved and restored around it.  The LDS address of a
// __shared__ object is the low half of its generic address.
__device__ __forceinline__ void dma_to_lds16(const char* gbase, uint32_t voff, const void* lds_dst) {
    const uint32_t lds = (uint32_t)(uintptr_t)lds_dst;
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(gbase)
        : "memory");
}

// XCD-aware work mapping of a 2-D grid (gridDim.x row blocks x gridDim.y key
// splits).  Workgroups are dispatched to the 8 XCDs round-robin by linear id,
// and each XCD has its own L2.  The linear ids of XCD x (x, x+8, ...) are
// given consecutive entries of the split-major list of (split, row block)
// pairs, so the workgroups an XCD runs at one time mostly stream the same
// key range through its L2.  A bijection: every pair is computed once,
// whatever the dispatch order.
__device__ __forceinline__ void xcd_work(int& row_block, int& split) {
    const int R = gridDim.x;
    const int total = R * gridDim.y;
    const int id = blockIdx.x + blockIdx.y * R;
    const int x = id & 7, k = id >> 3;
    const int q = total >> 3, r = total & 7;
    const int idx = x * q + min(x, r) + k;
    split = idx / R;
    row_block = idx - split * R;
}

// Combine two partial base-2 log-sum-exp states (M1, s1) and (M2, s2), each
// meaning M + log2(s).  Either may be empty (M = -inf, s = 0).
__device__ __forceinline__ void lse_merge(float& M, float& s, float M2, float s2) {
    const float Mn = fmaxf(M, M2);
    if (Mn == -INFINITY) return;  // both empty
    s = s * ex2(M - Mn) + s2 * ex2(M2 - Mn);
    M = Mn;
}

// Workgroup barrier without the memory fence of __syncthreads(): only this
// wave's LDS operations are waited for.  (The fence would also wait for every
// outstanding global->LDS tile load, serialising the load pipeline; the
// pipeline waits for exactly the tiles it needs with explicit vmcnt waits.)
__device__ __forceinline__ void stage_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Score element types of the matrix-core paths.
enum ScoreOp : int { OP_F32 = 1, OP_BF16 = 2, OP_F16 = 3 };

// Sum over the 64 lanes of a wave, in a fixed butterfly order (deterministic).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Block-wide deterministic sum (blockDim.x a multiple of 64, <= 1024).
// Returns the total on every thread.
__device__ __forceinline__ float block_sum(float v, float* lds_scratch /* >= 16 floats */) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    __syncthreads();
    if (lane == 0) lds_scratch[wid] = v;
    __syncthreads();
    float t = 0.f;
    for (int w = 0; w < nw; ++w) t += lds_scratch[w];
    return t;
}

}  // namespace fs
