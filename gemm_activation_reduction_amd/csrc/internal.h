// Internal launch interface between the C ABI (capi.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <cstddef>

namespace fconv {

// Optional per-kernel timing: when non-null, launchers bracket each kernel with
// begin(name) / end(name), which record HIP events on the launch stream.
struct KernelTimer {
    virtual void begin(const char* kernel, hipStream_t s) = 0;
    virtual void end(const char* kernel, hipStream_t s) = 0;
    virtual ~KernelTimer() = default;
};

// Conv: workspace = repacked weights followed by (pool only) per-tile partial sums.
struct ConvPlan {
    bool bf16;
    int act, pool;
    int N, Cin, H, W, Cout;
    int OH, OW;
    int KS, stride, pad;     // kernel size, stride, zero padding (3, 1, 0 on the 3x3 valid path)
    bool general;            // planned for the general-geometry kernel
    bool wide;               // 3x3 bf16: 256 oc per workgroup, weights by LDS DMA
    int TH, TW, BN, CK;      // output tile rows/cols, oc per workgroup, channels per K chunk
    int tilesH, tilesW, ocTiles, nChunk, CoutPad;
    size_t wpack_bytes;      // repacked weights [nChunk][KS * KS][CoutPad][CK]
    size_t part_bytes;       // pool partials [N][tilesH * tilesW][Cout] fp32
    size_t workspace_bytes() const { return wpack_bytes + part_bytes; }
    long long grid() const { return (long long)N * tilesH * tilesW * ocTiles; }
};

// pad 1 (a "same" 3x3 layer) only where conv3x3_same_wide holds: the wide bf16 kernel
ConvPlan plan_conv(bool bf16, int act, int pool, int N, int Cin, int H, int W, int Cout, const void* x, int pad = 0);
bool conv3x3_same_wide(bool bf16, int W, int Cout, const void* x);
hipError_t launch_conv(const ConvPlan& p, const void* x, const void* w, const float* b,
                       float* out, void* workspace, hipStream_t stream, KernelTimer* timer);

// General geometry: K x K kernel (K in {1, 3, 5}), stride 1 or 2, zero padding.
bool conv_general_supported(int K, int stride);
ConvPlan plan_conv_general(bool bf16, int act, int pool, int N, int Cin, int H, int W, int Cout, int K, int stride,
                           int pad);
hipError_t launch_conv_general(const ConvPlan& p, const void* x, const void* w, const float* b, float* out,
                               void* workspace, hipStream_t stream, KernelTimer* timer);

struct GemmPlan {
    int M, K, N;
    bool bf16;               // x, w bfloat16 (else float32)
    int BM, BN;
    int tilesM, tilesN;
    bool vec;                // K a multiple of a 16-byte group, 16-byte aligned rows: dwordx4 loads
    bool dma;                // LDS-DMA kernel (vec, K a whole even number of 64-byte stages, operands under 2 GiB)
    size_t part_bytes;       // [M][tilesN] (max, sum) pairs
    size_t workspace_bytes() const { return part_bytes; }
};

GemmPlan plan_gemm(bool bf16, int M, int K, int N, const void* x, const void* w);
hipError_t launch_gemm_lse(const GemmPlan& p, const void* x, const void* w, const float* b,
                           float scale, float cmin, float cmax, float* out, void* workspace,
                           hipStream_t stream, KernelTimer* timer);

// Epilogue-only kernels (HBM-bound streams over an already materialized tensor).
hipError_t launch_act_pool_map(const float* x, int N, int C, int H, int W, int act, float* out,
                               hipStream_t stream);
hipError_t launch_act_elementwise(const float* x, long long count, int act, float* out, hipStream_t stream);
hipError_t launch_scale_clamp_lse(const float* y, int M, int N, float scale, float cmin, float cmax, float* out,
                                  hipStream_t stream);

// Sustained matrix-core rate probe (measurement aid): a fixed grid of MFMA-only waves.
long long mfma_probe_grid();
double mfma_probe_flops(bool bf16, int iters);
hipError_t launch_mfma_probe(bool bf16, int iters, float* sink, hipStream_t stream);

}  // namespace fconv
