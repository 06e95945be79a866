/*
 * fconv -- fused dense-contraction + epilogue kernels for AMD Instinct MI355X (gfx950).
 *
 * Two fused operations, each computed in one pass so the full-resolution
 * intermediate never goes through HBM:
 *
 *   fconv_act_pool  3x3 valid stride-1 Conv2d + bias -> GELU (erf) or Mish(Mish(.))
 *                   -> optional global average pool.
 *   fgemm_lse_mish  Linear (x W^T + b) -> scale -> clamp -> row logsumexp -> z*mish(z).
 *
 * Error behaviour (all entry points): arguments are validated on the host before any
 * HIP call; a bad argument returns FCONV_EINVAL with nothing enqueued. A HIP failure
 * (allocation of the library's workspace, a launch) returns FCONV_ENOMEM / FCONV_EHIP.
 * fconv_last_error() returns a readable message for the calling thread's last non-OK
 * return. No entry point synchronizes the host with the stream.
 *
 * Ownership: every tensor pointer is a DEVICE pointer owned by the caller; outputs are
 * preallocated by the caller and must not alias any input. The library owns a small
 * device workspace per (device, stream) pair -- repacked weights and per-tile partial
 * results -- which it grows on demand (the growth path synchronizes that stream) and
 * frees in fconv_release(). Calls on one stream are ordered by the stream; calls that
 * pass the same stream from several host threads must be serialized by the caller.
 */
#ifndef FCONV_H
#define FCONV_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    FCONV_OK = 0,
    FCONV_EINVAL = -1,       /* bad argument; nothing was enqueued                   */
    FCONV_EUNSUPPORTED = -2, /* valid request the library does not implement         */
    FCONV_EHIP = -3,         /* a HIP runtime call or kernel launch failed           */
    FCONV_ENOMEM = -4        /* the workspace could not be allocated                 */
};

/* `act` argument of fconv_act_pool: bits 0..7 pick the activation, bits 8..11 the
 * element type of x and w. Every other bit must be zero. */
enum {
    FCONV_ACT_NONE = 0,   /* identity (plain conv + bias)                                 */
    FCONV_ACT_GELU = 1,   /* 0.5 v (1 + erf(v / sqrt 2)), the exact form                  */
    FCONV_ACT_MISH2 = 2,  /* mish(mish(v)), mish(v) = v tanh(log(1 + e^v))                */
    FCONV_ACT_GELU_TANH = 3, /* 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))), the tanh
                              * approximation the "Kimi-K2.6 l2_p67" page weighs against the
                              * exact form (PyTorch's approximate='tanh'); a different function,
                              * within 4.8e-4 of FCONV_ACT_GELU                               */
    FCONV_DT_F32 = 0x000, /* x, w float32                                                 */
    FCONV_DT_BF16 = 0x100 /* x, w bfloat16 (products exact in fp32, fp32 accumulation)    */
};

/*
 * Fused 3x3 convolution + bias + activation (+ global average pool).
 *
 * Computes, for 0 <= oh < H-2 and 0 <= ow < W-2 (stride 1, no padding, no kernel flip):
 *   pre[n,oc,oh,ow] = b[oc] + sum_{ic<Cin, kh<3, kw<3} w[oc,ic,kh,kw] * x[n,ic,oh+kh,ow+kw]
 *   pool == 0:  out[n,oc,oh,ow] = act(pre[n,oc,oh,ow])
 *   pool == 1:  out[n,oc]       = (1 / ((H-2)(W-2))) * sum_{oh,ow} act(pre[n,oc,oh,ow])
 * Sources: the direct-convolution sum and the Conv2d -> Mish -> Mish chain of the
 * "Kimi-K2.6 l2_p4" POPCORNBENCH page; the exact GELU and the AdaptiveAvgPool2d(1)
 * mean of the "Kimi-K2.6 l2_p67" page.
 *
 *   x     [N][Cin][H][W]      NCHW contiguous, float32 or bfloat16 (see `act`)
 *   w     [Cout][Cin][3][3]   OIHW contiguous, same element type as x
 *   b     [Cout]              float32
 *   out   pool=1: [N][Cout] float32;  pool=0: [N][Cout][H-2][W-2] float32 (NCHW)
 *   act   FCONV_ACT_* | FCONV_DT_*
 *   pool  0 or 1
 *   stream  HIP stream the work is enqueued on (0 = the null stream)
 *
 * Returns FCONV_EINVAL for a null pointer, N, Cin or Cout < 1, H or W < 3, an unknown
 * act/dtype bit, pool not in {0,1}, a tensor of 2^31 or more elements, or an output
 * that overlaps an input. The pooled result is deterministic run to run (no atomics).
 */
int fconv_act_pool(const void* x, const void* w, const float* b,
                   int N, int Cin, int H, int W, int Cout,
                   int act, int pool, float* out, hipStream_t stream);

/*
 * fconv_act_pool without any allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, results and kernels as fconv_act_pool; the caller still provides x, w,
 * b and out. Instead of the library's workspace it uses a static device array of
 * FCONV_NOALLOC_SCRATCH_BYTES (16 MiB) that each GPU the library runs on holds until the
 * process ends; it needs (repacked weights) + (pool only) N * Cout * tiles * 4 bytes, e.g.
 * 3.2 MB for x (64, 16, 224, 224) -> 64 pooled. It calls no hipMalloc, hipFree or
 * allocating library routine, and records no profiling events.
 * Every call on one GPU shares that GPU's array and leaves its contents behind (every
 * byte a call reads it has written first, so nothing needs clearing): calls that overlap
 * on one GPU -- on different streams, or from several host threads -- race and must be
 * serialized by the caller.
 * Returns the fconv_act_pool errors, and FCONV_EINVAL (nothing enqueued) when the call
 * needs more scratch than the array holds.
 */
#define FCONV_NOALLOC_SCRATCH_BYTES (16u << 20)
int fconv_act_pool_noalloc(const void* x, const void* w, const float* b,
                           int N, int Cin, int H, int W, int Cout,
                           int act, int pool, float* out, hipStream_t stream);

/*
 * The same fused operation for a K x K kernel with stride and zero padding (nn.Conv2d's
 * kernel_size, stride and padding; the pages fix K = 3, stride 1, padding 0):
 *   pre[n,oc,oh,ow] = b[oc] + sum_{ic, kh<K, kw<K} w[oc,ic,kh,kw] * xp[n, ic, oh*stride + kh - pad,
 *                                                                     ow*stride + kw - pad]
 * where xp is x with zeros outside 0 <= row < H, 0 <= col < W, and
 *   OH = (H + 2 pad - K) / stride + 1,   OW = (W + 2 pad - K) / stride + 1.
 * pool == 1 averages act(pre) over the OH x OW map (padded borders included, as
 * AdaptiveAvgPool2d(1) does on the conv output).
 *
 *   w    [Cout][Cin][K][K] OIHW, same dtype as x; all other arguments as fconv_act_pool,
 *        out [N][Cout] or [N][Cout][OH][OW].
 *
 * Supported: K in {1, 3, 5}, stride in {1, 2}, 0 <= pad < K. K = 3, stride 1, pad 0 runs
 * the same kernel as fconv_act_pool, and so does a bf16 K = 3, stride 1, pad 1 layer of 256
 * or more output channels with W % 8 == 0 and a 16-byte aligned x (the wide kernel, padded).
 * Returns FCONV_EINVAL for the fconv_act_pool errors,
 * K < 1, stride < 1, pad < 0 or a padded input smaller than the kernel;
 * FCONV_EUNSUPPORTED for another K or stride, or pad >= K.
 */
int fconv2d_act_pool(const void* x, const void* w, const float* b,
                     int N, int Cin, int H, int W, int Cout, int K, int stride, int pad,
                     int act, int pool, float* out, hipStream_t stream);

/*
 * Fused GEMM + scale + clamp + row logsumexp + z*mish(z).
 *
 *   y[m,j] = scale * (sum_k x[m,k] * w[j,k] + b[j])
 *   c[m,j] = min(max(y[m,j], cmin), cmax)
 *   z[m]   = log(sum_j exp(c[m,j]))        (evaluated max-shifted, tile by tile)
 *   out[m] = z[m] * mish(z[m])
 * Source: the Linear -> x2 -> x+x -> clamp -> logsumexp -> x*mish(x) model of the
 * "Kimi-K2.6 l2_p22" POPCORNBENCH page (its x2 then x+x is scale = 4) and the page's
 * online max / sum-of-exponentials merge rule.
 *
 *   x    [M][K] row-major float32
 *   w    [N][K] row-major float32 (nn.Linear weight layout)
 *   b    [N] float32
 *   out  [M] float32 (the (M, 1) result)
 *
 * Returns FCONV_EINVAL for a null pointer, M, K or N < 1, a non-finite scale, cmin or
 * cmax, cmin > cmax, a tensor of 2^31 or more elements, or an output overlapping an
 * input. The result is deterministic run to run (fixed-order merge, no atomics).
 */
int fgemm_lse_mish(const float* x, const float* w, const float* b,
                   int M, int K, int N, float scale, float cmin, float cmax,
                   float* out, hipStream_t stream);

/*
 * The same operation with bfloat16 operands: x [M][K] and w [N][K] row-major bfloat16
 * bit patterns, b [N] and out [M] float32. Products of bfloat16 values are exact in
 * fp32 and accumulate in fp32 (v_mfma_f32_16x16x32_bf16); bias, scale, clamp,
 * logsumexp and z * mish(z) run in fp32. The bfloat16 variant of the l2_p22 chain
 * (reduced-precision operands, the same epilogue). Errors as for fgemm_lse_mish.
 */
int fgemm_lse_mish_bf16(const void* x, const void* w, const float* b,
                        int M, int K, int N, float scale, float cmin, float cmax,
                        float* out, hipStream_t stream);

/*
 * Epilogue-only operations over an already materialized tensor: the kernels the pages
 * write for use after a separate convolution or GEMM. All float32, all HBM-bound.
 *
 * fact_pool: out[n,c] = (1 / (H W)) * sum_{h,w} act(x[n,c,h,w]), x NCHW [N][C][H][W],
 *   out [N][C]; act = FCONV_ACT_NONE, _GELU, _MISH2 or _GELU_TANH (no dtype bits).
 *   Source: the GELU + AdaptiveAvgPool2d(1) kernel of the "Kimi-K2.6 l2_p67" page.
 * fact_elementwise: out[i] = act(x[i]) for 0 <= i < count; out == x (in place) is
 *   allowed, any other overlap is not. Source: the Mish -> Mish kernel of the
 *   "Kimi-K2.6 l2_p4" page (act = FCONV_ACT_MISH2).
 * flse_mish_rows: for each row m of y [M][N] (row-major), c = min(max(scale y, cmin), cmax),
 *   z = log(sum_j exp(c[m,j])) (max-shifted), out[m] = z * mish(z). Source: the fused
 *   scale/clamp/logsumexp/mish kernel of the "Kimi-K2.6 l2_p22" page, applied to the
 *   nn.Linear output (which already includes the bias).
 * Errors: FCONV_EINVAL for a null pointer, a size < 1 (count < 0), an unknown act, a NaN
 * or infinite scale, cmin > cmax or NaN, a tensor of 2^31 or more elements (fact_pool,
 * flse_mish_rows), or a forbidden overlap; FCONV_EHIP if the launch fails. Results are
 * deterministic run to run (fixed-order reductions). No workspace is used.
 */
int fact_pool(const float* x, int N, int C, int H, int W, int act, float* out, hipStream_t stream);
int fact_elementwise(const float* x, long long count, int act, float* out, hipStream_t stream);
int flse_mish_rows(const float* y, int M, int N, float scale, float cmin, float cmax, float* out,
                   hipStream_t stream);

/* Message describing the calling thread's last non-OK return ("" if none). The
 * pointer stays valid until the next call into the library from that thread. */
const char* fconv_last_error(void);

/* Synchronizes every device that holds a workspace, frees all workspaces and
 * returns FCONV_OK (or FCONV_EHIP). Later calls allocate afresh. */
int fconv_release(void);

/*
 * Per-kernel timing, for measurement tools. fconv_profile(1) makes every later call
 * bracket each of its kernels with HIP events recorded on the call's stream (a small
 * host cost per launch); fconv_profile(0) stops it. Either call first waits for the
 * outstanding events and clears the accumulated totals.
 * fconv_profile_read(kernel, &ms, &launches) waits for the recorded events and returns
 * the summed event time in milliseconds and the number of launches of `kernel` since
 * the last fconv_profile() call. Kernel names: "pack_weights", "conv3x3_fused", "conv3x3_wide_bf16",
 * "conv_general_fused", "pool_finalize", "gemm_lse_partials", "lse_merge_mish", "act_pool_map", "act_elementwise",
 * "scale_clamp_lse", "mfma_rate_probe". Unknown names read as zero.
 * Returns FCONV_EINVAL for a null argument, FCONV_EHIP if an event wait fails.
 */
int fconv_profile(int enable);
int fconv_profile_read(const char* kernel, double* total_ms, long long* launches);

/*
 * Sustained matrix-core rate probe, for measurement tools (not a fused operation).
 * Enqueues on `stream` one kernel of a fixed grid whose waves issue only MFMAs
 * (v_mfma_f32_16x16x4_f32 for dtype FCONV_DT_F32, v_mfma_f32_16x16x32_bf16 for
 * FCONV_DT_BF16): four independent accumulator chains per wave, `iters` rounds of two
 * MFMAs per chain, operands alternating between two sets of pseudo-random values. The
 * clock a part holds under such load is set by its power draw, so the FLOP count divided
 * by the launch's duration is the dense rate the matrix cores sustain, the ceiling a
 * contraction kernel can reach on this part (the spec peaks assume 2.4 GHz throughout).
 *   sink   one float of device memory (never written for finite sums; it keeps the
 *          compiler from removing the work)
 *   flops  receives the launch's FLOP count (host pointer)
 * Timed like the other kernels under fconv_profile, as "mfma_rate_probe".
 * Returns FCONV_EINVAL for a null pointer, another dtype, or iters outside 1 .. 2^20;
 * FCONV_EHIP if the launch fails.
 */
int fconv_mfma_rate_probe(int dtype, int iters, float* sink, double* flops, hipStream_t stream);

/* Library ABI version (major * 100 + minor). */
int fconv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FCONV_H */
