// Device-side activation math and wave64 reductions for gfx950 (fp32).
#pragma once
#include <hip/hip_runtime.h>

namespace fconv {

enum Act { kActNone = 0, kActGelu = 1, kActMish2 = 2, kActGeluTanh = 3 };

// e^v through the hardware base-2 exponential: exp(v) = 2^(v * log2 e).
// For |v| <= 30 the relative error stays within a few 1e-6, far inside the
// 1e-4 parity tolerance.
__device__ __forceinline__ float fast_exp(float v) {
    return __builtin_amdgcn_exp2f(v * 1.4426950408889634f);
}

// max(v, 0) as one v_med3_f32. On an MFMA accumulator fmaxf also emits a canonicalizing
// v_max_f32 v, v (the compiler cannot tell the value is not a signalling NaN), one more VALU
// instruction per output in every epilogue; with an infinite bound the compiler turns the med3
// back into that pair, so the upper bound is FLT_MAX. Equal to max(v, 0) for every finite v.
constexpr float kFltMax = 3.402823466e38f;
__device__ __forceinline__ float relu(float v) { return __builtin_amdgcn_fmed3f(v, 0.0f, kFltMax); }

// Exact-form GELU, 0.5 v (1 + erf(v / sqrt 2)) = v Phi(v) ("Kimi-K2.6 l2_p67" page:
// PyTorch's default approximate='none' form, not the tanh approximation).
// With a = |v|, v Phi(v) = max(v, 0) - a Phi(-a) for either sign of v, since
// Phi(v) = 1 - Phi(-v); so only the normal tail Phi(-a) is needed, and the negative tail
// keeps its absolute accuracy (no 1 - erf cancellation). The tail is 2^Q(a), Q a degree-5
// polynomial fitted to log2 Phi(-a) on [0, 6.5] in the weighted minimax sense that bounds
// the GELU's own error (gelu_fit.py in this package writes the coefficients): at most
// 4.3e-7 from the fit, 6.3e-7 with fp32 rounding, for every v. Q' has no real zero and the
// leading coefficient is negative, so beyond the fit Q keeps falling, 2^Q underflows to 0
// and the result is max(v, 0). Cost: 7 VALU operations and one v_exp_f32. Abramowitz &
// Stegun's formula 7.1.28 for erf, used before, took 12 and a reciprocal. In the fp32
// convolutions VALU work cannot run beside the MFMAs, so each instruction saved per output
// is kernel time saved.
__device__ __forceinline__ float gelu_erf(float v) {
    const float a = fabsf(v);
    float q = fmaf(-0.00047271855873987079f, a, 0.0070818220265209675f);
    q = fmaf(q, a, -0.051824294030666351f);
    q = fmaf(q, a, -0.45999139547348022f);
    q = fmaf(q, a, -1.1507898569107056f);
    q = fmaf(q, a, -1.0000371932983398f);
    return fmaf(-a, __builtin_amdgcn_exp2f(q), relu(v));
}

// Tanh-approximation GELU, 0.5 v (1 + tanh(u)), u = sqrt(2/pi) (v + 0.044715 v^3) (the
// l2_p67 page's approximate='tanh' form). Since 0.5 (1 + tanh(u)) = 1 / (1 + e^{-2u}), it is
// v / (1 + 2^{v (c1 + c2 v^2)}) with c1 = -2 sqrt(2/pi) log2(e) and c2 = 0.044715 c1: three
// VALU operations, an exponential and a reciprocal. For v << 0 the power overflows to +inf
// and the reciprocal to 0 (the result is -0); for v >> 0 it underflows to 0 and the result
// is v.
__device__ __forceinline__ float gelu_tanh(float v) {
    const float s = fmaf(v * v, -0.1029432395800235f, -2.302208198144325f);
    return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(v * s));
}

// Mish(v) = v tanh(softplus(v)). With t = e^v, tanh(log(1 + t)) = q / (q + 2), q = t (t + 2),
// so mish(v) = v - v r with r = 2 / (q + 2) = 1 / (1 + t (1 + t / 2)): one exponential, one
// reciprocal and four VALU operations (the product form v q / (q + 2) takes seven; in the
// fp32 convolutions, where VALU work serializes with the MFMAs, each one saved per output is
// kernel time). Large v needs no clamp: for v > 20, r < 1e-17 and v - v r rounds to v; from
// v ~ 44 on, t (1 + t / 2) overflows to +inf (and from v ~ 88 on t itself), r is 0 and the
// result is exactly v. For very negative v, t underflows to 0, r to 1 and the result to 0,
// as the exact function tends. The subtraction gives up relative (not absolute) accuracy
// where mish(v) is tiny (v << 0): the result stays within 1.3e-6 of the exact Mish for
// every finite v.
__device__ __forceinline__ float mish_f32(float v) {
    const float t = fast_exp(v);
    const float r = __builtin_amdgcn_rcpf(fmaf(t, fmaf(t, 0.5f, 1.0f), 1.0f));
    return fmaf(-v, r, v);
}

template <int ACT>
__device__ __forceinline__ float activate(float v) {
    if constexpr (ACT == kActGelu) return gelu_erf(v);
    else if constexpr (ACT == kActMish2) return mish_f32(mish_f32(v));
    else if constexpr (ACT == kActGeluTanh) return gelu_tanh(v);
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
