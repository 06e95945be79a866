// Sustained matrix-core rate probe (a measurement aid, not part of the fused operations).
//
// The spec peaks (157.3 TFLOP/s fp32, 2516.6 TFLOP/s bf16 dense) assume every SIMD issues
// an MFMA every cycle budget at 2.4 GHz. Under load the shader clock falls with the power
// the work draws, so the rate a kernel can reach on a given part is lower. This kernel
// measures it: every wave issues only MFMAs, on four independent accumulator chains, with
// operands that alternate between two register sets of pseudo-random values so that the
// multipliers see data changing from one instruction to the next, as real work does.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace fconv {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeChains = 4;

__device__ __forceinline__ unsigned hash32(unsigned v) {
    v ^= v >> 16;
    v *= 0x7feb352dU;
    v ^= v >> 15;
    v *= 0x846ca68bU;
    v ^= v >> 16;
    return v;
}

// Two bf16 values with random signs and mantissas and magnitudes in [2^-3, 2^-1): exponent
// field 124 (0x3E00) plus a random low exponent bit.
__device__ __forceinline__ unsigned bf16_pair(unsigned h) {
    const unsigned lo = 0x3E00u | (h & 0x80FFu);
    const unsigned hi = 0x3E00u | ((h >> 16) & 0x80FFu);
    return lo | (hi << 16);
}

template <bool BF16>
__global__ void __launch_bounds__(kProbeThreads) mfma_rate_probe(int iters, float* sink) {
    const unsigned seed = hash32(blockIdx.x * kProbeThreads + threadIdx.x + 1);
    f4 acc[kProbeChains];
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) acc[c] = f4{0.f, 0.f, 0.f, 0.f};
    if constexpr (BF16) {
        u4 a0, a1, b0, b1;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            a0[k] = bf16_pair(hash32(seed + 11 * k));
            a1[k] = bf16_pair(hash32(seed + 11 * k + 3));
            b0[k] = bf16_pair(hash32(seed + 11 * k + 5));
            b1[k] = bf16_pair(hash32(seed + 11 * k + 7));
        }
        const bf16x8 A0 = __builtin_bit_cast(bf16x8, a0), A1 = __builtin_bit_cast(bf16x8, a1);
        const bf16x8 B0 = __builtin_bit_cast(bf16x8, b0), B1 = __builtin_bit_cast(bf16x8, b1);
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int c = 0; c < kProbeChains; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16((c & 1) ? A1 : A0, (c & 2) ? B1 : B0, acc[c], 0, 0,
                                                                0);
#pragma unroll
            for (int c = 0; c < kProbeChains; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16((c & 1) ? A0 : A1, (c & 2) ? B0 : B1, acc[c], 0, 0,
                                                                0);
        }
    } else {
        const float A0 = 0.25f + (hash32(seed) & 0xFFFF) * (1.0f / 65536.0f);
        const float A1 = -0.5f - (hash32(seed + 1) & 0xFFFF) * (1.0f / 65536.0f);
        const float B0 = 0.75f - (hash32(seed + 2) & 0xFFFF) * (1.0f / 131072.0f);
        const float B1 = -0.3f + (hash32(seed + 3) & 0xFFFF) * (1.0f / 65536.0f);
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int c = 0; c < kProbeChains; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32((c & 1) ? A1 : A0, (c & 2) ? B1 : B0, acc[c], 0, 0, 0);
#pragma unroll
            for (int c = 0; c < kProbeChains; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32((c & 1) ? A0 : A1, (c & 2) ? B0 : B1, acc[c], 0, 0, 0);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    // The sums are finite, so nothing is stored; the compiler cannot know that and keeps
    // every MFMA.
    if (s != s) sink[0] = s;
}

}  // namespace

long long mfma_probe_grid() { return 2048; }

double mfma_probe_flops(bool bf16, int iters) {
    const double per_mfma = bf16 ? 2.0 * 16 * 16 * 32 : 2.0 * 16 * 16 * 4;
    const double waves = (double)mfma_probe_grid() * (kProbeThreads / 64);
    return waves * iters * 2.0 * kProbeChains * per_mfma;
}

hipError_t launch_mfma_probe(bool bf16, int iters, float* sink, hipStream_t stream) {
    const dim3 grid((unsigned)mfma_probe_grid()), block(kProbeThreads);
    if (bf16)
        hipLaunchKernelGGL(mfma_rate_probe<true>, grid, block, 0, stream, iters, sink);
    else
        hipLaunchKernelGGL(mfma_rate_probe<false>, grid, block, 0, stream, iters, sink);
    return hipGetLastError();
}

}  // namespace fconv
