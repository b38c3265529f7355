// retro_probe.hip - the measured ceilings declared in retro_probe.h: a
// matrix-core loop with no memory traffic, the same loop beside vector FMA
// work on the same SIMDs, and a 16-byte vector copy. They share nothing with
// the OUT_PROD kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "retro_out_prod.h"
#include "retro_probe.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeBlocks = 2048;  // 8 workgroups per CU
constexpr int kProbeThreads = 256;  // 4 waves
constexpr int kChains = 4;          // independent accumulators per wave
constexpr int64_t kMaxIterations = int64_t(1) << 20;

// Operands vary by lane so that nothing folds; with |a b| about 2^-14 per
// product the accumulators stay far from overflow for any allowed count.
template <int KIND>
__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(float* sink, int iterations) {
    const int lane = threadIdx.x & 63;
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[c][v] = 0.f;
    if constexpr (KIND == RETRO_PROBE_MFMA_F32) {
        const float a = 0.0078125f * (1.f + float(lane) * 0.0009765625f);
        const float b = 0.0078125f * (1.f - float(lane) * 0.0009765625f);
        for (int i = 0; i < iterations; ++i)
#pragma unroll
            for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[c], 0, 0, 0);
    } else {
        bf16x8 a, b;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[e] = __bf16(0.0078125f * (1.f + float(lane + e) * 0.0078125f));
            b[e] = __bf16(0.0078125f * (1.f - float(lane + e) * 0.0078125f));
        }
        for (int i = 0; i < iterations; ++i)
#pragma unroll
            for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[c][v];
    sink[blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

// Matrix core beside vector ALU: a workgroup of 8 waves, two per SIMD
// (waves are placed on the SIMDs in turn). Waves 0-3 run `mfma_iterations`
// rounds of 4 independent v_mfma_f32_16x16x4_f32 chains, waves 4-7 run
// `valu_iterations` rounds of 16 v_fma_f32 over 8 independent chains.
// Timing the kernel with either count at 0 and then with both shows whether
// the two kinds of work share the SIMD's issue time or run side by side.
constexpr int kMixBlocks = 512;    // 2 workgroups per CU
constexpr int kMixThreads = 512;   // 8 waves
constexpr int kMixFmaChains = 8;
__global__ __launch_bounds__(kMixThreads) void mfma_valu_probe_kernel(float* sink, int mfma_iterations,
                                                                      int valu_iterations) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    float s = 0.f;
    if (wave < 4) {
        const float a = 0.0078125f * (1.f + float(lane) * 0.0009765625f);
        const float b = 0.0078125f * (1.f - float(lane) * 0.0009765625f);
        f32x4 acc[kChains];
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < mfma_iterations; ++i)
#pragma unroll
            for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[c], 0, 0, 0);
#pragma unroll
        for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    } else {
        // x -> x m + c then x m - c: values stay near their start for any count
        float v[kMixFmaChains];
#pragma unroll
        for (int j = 0; j < kMixFmaChains; ++j) v[j] = 1.f + float(lane) * 0.0009765625f + float(j);
        const float m = 1.0000001f, c = 1e-7f;
        for (int i = 0; i < valu_iterations; ++i) {
#pragma unroll
            for (int j = 0; j < kMixFmaChains; ++j) v[j] = __builtin_fmaf(v[j], m, c);
#pragma unroll
            for (int j = 0; j < kMixFmaChains; ++j) v[j] = __builtin_fmaf(v[j], m, -c);
        }
#pragma unroll
        for (int j = 0; j < kMixFmaChains; ++j) s += v[j];
    }
    sink[blockIdx.x * kMixThreads + threadIdx.x] = s;
}

// Copy of n 16-byte units: workgroup b copies units 1024 b .. 1024 b + 1023,
// thread i units 1024 b + 256 j + i (j = 0..3), all four loads issued before
// the stores.
constexpr int kCopyUnroll = 4;
__global__ __launch_bounds__(256) void copy_probe_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         int64_t n) {
    const int64_t base = int64_t(blockIdx.x) * (256 * kCopyUnroll) + threadIdx.x;
    u32x4 v[kCopyUnroll];
    if (base + 256 * (kCopyUnroll - 1) < n) {
#pragma unroll
        for (int j = 0; j < kCopyUnroll; ++j) v[j] = src[base + 256 * j];
#pragma unroll
        for (int j = 0; j < kCopyUnroll; ++j) dst[base + 256 * j] = v[j];
    } else {
#pragma unroll
        for (int j = 0; j < kCopyUnroll; ++j)
            if (base + 256 * j < n) dst[base + 256 * j] = src[base + 256 * j];
    }
}

int launch_status() { return hipGetLastError() == hipSuccess ? RETRO_OK : RETRO_E_HIP; }

}  // namespace

extern "C" int64_t retro_probe_sink_floats(void) { return int64_t(kProbeBlocks) * kProbeThreads; }

extern "C" int retro_probe_mfma(int kind, float* sink, int64_t iterations, double* flops, void* stream) {
    if (kind != RETRO_PROBE_MFMA_F32 && kind != RETRO_PROBE_MFMA_BF16) return RETRO_E_TYPE;
    if (iterations < 1 || iterations > kMaxIterations) return RETRO_E_SHAPE;
    if (!sink) return RETRO_E_NULL;
    if (reinterpret_cast<uintptr_t>(sink) % 4) return RETRO_E_ALIGN;
    const double per_mfma = kind == RETRO_PROBE_MFMA_F32 ? 32.0 * 32 * 2 * 2 : 32.0 * 32 * 16 * 2;
    if (flops) *flops = double(kProbeBlocks) * (kProbeThreads / 64) * double(iterations) * kChains * per_mfma;
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (kind == RETRO_PROBE_MFMA_F32)
        hipLaunchKernelGGL(mfma_probe_kernel<RETRO_PROBE_MFMA_F32>, dim3(kProbeBlocks), dim3(kProbeThreads), 0, st,
                           sink, int(iterations));
    else
        hipLaunchKernelGGL(mfma_probe_kernel<RETRO_PROBE_MFMA_BF16>, dim3(kProbeBlocks), dim3(kProbeThreads), 0, st,
                           sink, int(iterations));
    return launch_status();
}

extern "C" int retro_probe_mfma_valu(int64_t mfma_iterations, int64_t valu_iterations, float* sink, double* flops,
                                     int64_t* valu_instructions, void* stream) {
    if (mfma_iterations < 0 || mfma_iterations > kMaxIterations || valu_iterations < 0 ||
        valu_iterations > kMaxIterations)
        return RETRO_E_SHAPE;
    if (!sink) return RETRO_E_NULL;
    if (reinterpret_cast<uintptr_t>(sink) % 4) return RETRO_E_ALIGN;
    static_assert(int64_t(kMixBlocks) * kMixThreads <= int64_t(kProbeBlocks) * kProbeThreads, "sink size");
    if (flops) *flops = double(kMixBlocks) * 4 * double(mfma_iterations) * kChains * (16.0 * 16 * 4 * 2);
    if (valu_instructions) *valu_instructions = int64_t(kMixBlocks) * 4 * valu_iterations * 2 * kMixFmaChains;
    (void)hipGetLastError();
    hipLaunchKernelGGL(mfma_valu_probe_kernel, dim3(kMixBlocks), dim3(kMixThreads), 0, static_cast<hipStream_t>(stream),
                       sink, int(mfma_iterations), int(valu_iterations));
    return launch_status();
}

extern "C" int retro_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    if (bytes < 0 || bytes % 16 || bytes >= (int64_t(1) << 40)) return RETRO_E_SHAPE;
    if (bytes == 0) return RETRO_OK;
    if (!src || !dst) return RETRO_E_NULL;
    const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
    if (s % 16 || d % 16) return RETRO_E_ALIGN;
    if (s < d + uintptr_t(bytes) && d < s + uintptr_t(bytes)) return RETRO_E_ALIAS;
    const int64_t n = bytes / 16;
    const int64_t blocks = (n + 256 * kCopyUnroll - 1) / (256 * kCopyUnroll);
    (void)hipGetLastError();
    hipLaunchKernelGGL(copy_probe_kernel, dim3(unsigned(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n);
    return launch_status();
}
