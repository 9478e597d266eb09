// fs_probe.hip -- unit-throughput probe kernels behind fs_probe_peak.
//
// Each kernel keeps one execution unit busy with independent work and touches
// memory only for a store that never happens (its condition compares with a
// runtime value the caller chooses never to match), so its duration measures
// the unit's throughput at the clock the GPU holds at that moment.
//
// Launch shape: 4 workgroups of 4 waves per compute unit (four waves per SIMD),
// enough independent chains per wave to cover each instruction's latency.
#include "fs_device.hpp"
#include "fs_internal.h"

namespace fs {

namespace {

constexpr int kProbeChains = 4;   // independent matrix accumulators per wave
constexpr int kProbeIters = 512;  // loop trips; 8 instructions per chain per trip
constexpr int kExpChains = 8;     // independent exponential chains per lane
constexpr int kExpIters = 4096;   // loop trips; kExpChains exponentials per trip

template <int OP>
__global__ __launch_bounds__(256) void mfma_probe_kernel(float* sink, float never) {
    const float t = (float)threadIdx.x * (1.0f / 256.0f);
    f32x16 acc[kProbeChains];
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
    if constexpr (OP == OP_F32) {
        const float x = t, y = 1.0f - t;
        for (int it = 0; it < kProbeIters; ++it) {
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int c = 0; c < kProbeChains; ++c)
                    acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(x, y, acc[c], 0, 0, 0);
        }
    } else {
        bf16x8 ab, bb;
        f16x8 ah, bh;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ab[e] = (__bf16)(t + e);
            bb[e] = (__bf16)(1.0f - t);
            ah[e] = (_Float16)(t + e);
            bh[e] = (_Float16)(1.0f - t);
        }
        for (int it = 0; it < kProbeIters; ++it) {
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int c = 0; c < kProbeChains; ++c) {
                    if constexpr (OP == OP_BF16)
                        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, bb, acc[c], 0, 0, 0);
                    else
                        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, acc[c], 0, 0, 0);
                }
        }
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    if (s == never) sink[0] = s;
}

// x <- 2^(-x) keeps every chain in (0, 1]; one v_exp_f32 per step.
__global__ __launch_bounds__(256) void exp_probe_kernel(float* sink, float never) {
    float x[kExpChains];
#pragma unroll
    for (int c = 0; c < kExpChains; ++c) x[c] = (float)(threadIdx.x + c) * (1.0f / 512.0f);
    for (int it = 0; it < kExpIters; ++it) {
#pragma unroll
        for (int c = 0; c < kExpChains; ++c) x[c] = ex2(-x[c]);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kExpChains; ++c) s += x[c];
    if (s == never) sink[0] = s;
}

}  // namespace

int probe_blocks() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return 0;
    return 4 * cus;
}

double probe_work_per_launch(int kind, int blocks) {
    const double waves = 4.0 * blocks;
    if (kind == 4) return waves * 64.0 * kExpChains * kExpIters;
    const double mfmas = waves * kProbeChains * 8.0 * kProbeIters;
    return mfmas * (kind == 3 ? 32.0 * 32.0 * 2.0 * 2.0 : 32.0 * 32.0 * 16.0 * 2.0);
}

hipError_t launch_probe(int kind, int blocks, float* sink, hipStream_t s) {
    const float never = -1.0f;  // every probe's sum is >= 0
    switch (kind) {
        case 1: mfma_probe_kernel<OP_BF16><<<blocks, 256, 0, s>>>(sink, never); break;
        case 2: mfma_probe_kernel<OP_F16><<<blocks, 256, 0, s>>>(sink, never); break;
        case 3: mfma_probe_kernel<OP_F32><<<blocks, 256, 0, s>>>(sink, never); break;
        case 4: exp_probe_kernel<<<blocks, 256, 0, s>>>(sink, never); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace fs
