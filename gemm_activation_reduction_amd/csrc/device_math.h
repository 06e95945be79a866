// Device-side activation math and wave64 reductions for gfx950 (fp32).
#pragma once
#include <hip/hip_runtime.h>

namespace fconv {

enum Act { kActNone = 0, kActGelu = 1, kActMish2 = 2 };

// e^v through the hardware base-2 exponential: exp(v) = 2^(v * log2 e).
// For |v| <= 30 the relative error stays within a few 1e-6, far inside the
// 1e-4 parity tolerance.
__device__ __forceinline__ float fast_exp(float v) {
    return __builtin_amdgcn_exp2f(v * 1.4426950408889634f);
}

// Exact-form GELU, 0.5 v (1 + erf(v / sqrt 2)) ("Kimi-K2.6 l2_p67" page: PyTorch's
// default approximate='none' form, not the tanh approximation).
// erf is evaluated with the rational approximation of Abramowitz & Stegun,
// Handbook of Mathematical Functions, formula 7.1.26 (Hastings):
//   erfc(u) = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) e^{-u^2},  t = 1 / (1 + p u),  u >= 0,
// with |error| <= 1.5e-7. For v < 0 the result is formed as 0.5 v erfc(|v| / sqrt 2),
// so the negative tail keeps its absolute accuracy instead of cancelling 1 - erf.
__device__ __forceinline__ float gelu_erf(float v) {
    const float u = fabsf(v) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, u, 1.0f));
    float poly = fmaf(t, 1.061405429f, -1.453152027f);
    poly = fmaf(t, poly, 1.421413741f);
    poly = fmaf(t, poly, -0.284496736f);
    poly = fmaf(t, poly, 0.254829592f);
    const float erfc_u = t * poly * fast_exp(-u * u);
    return 0.5f * v * (v >= 0.0f ? 2.0f - erfc_u : erfc_u);
}

// Mish(v) = v tanh(softplus(v)). With t = e^v, tanh(log(1 + t)) = (t^2 + 2t) / (t^2 + 2t + 2),
// so mish(v) = v * q / (q + 2) with q = t (t + 2): one exponential and one reciprocal.
// For v > 20 the ratio is 1 to fp32 precision (2 / (q + 2) < 1e-17), so v is returned;
// for very negative v, q underflows to 0 and mish(v) -> 0 as the exact function does.
__device__ __forceinline__ float mish_f32(float v) {
    float t = fast_exp(fminf(v, 20.0f));
    float q = t * (t + 2.0f);
    float r = q * __builtin_amdgcn_rcpf(q + 2.0f);
    return v > 20.0f ? v : v * r;
}

template <int ACT>
__device__ __forceinline__ float activate(float v) {
    if constexpr (ACT == kActGelu) return gelu_erf(v);
    else if constexpr (ACT == kActMish2) return mish_f32(mish_f32(v));
    else return v;
}

// Butterfly reductions across a full wave64 (every lane ends with the result).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

}  // namespace fconv
