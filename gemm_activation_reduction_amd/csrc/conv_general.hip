// Fused K x K convolution (K = 1, 3 or 5) with stride 1 or 2 and zero padding, + bias +
// activation (+ global average pool), for gfx950: the plan, the weight repack, the dispatch
// to the per-kernel-size translation units (conv_general_k1.hip, _k3.hip, _k5.hip) and the
// pool finalize. The kernel and its design notes are in conv_general_kernel.h.
#include "conv_general_kernel.h"

namespace fconv {

bool conv_general_supported(int K, int stride) {
    return (K == 1 || K == 3 || K == 5) && (stride == 1 || stride == 2);
}

ConvPlan plan_conv_general(bool bf16, int act, int pool, int N, int Cin, int H, int W, int Cout, int K, int stride,
                           int pad) {
    ConvPlan p{};
    p.bf16 = bf16; p.act = act; p.pool = pool;
    p.N = N; p.Cin = Cin; p.H = H; p.W = W; p.Cout = Cout;
    p.KS = K; p.stride = stride; p.pad = pad; p.general = true;
    p.OH = (H + 2 * pad - K) / stride + 1;
    p.OW = (W + 2 * pad - K) / stride + 1;
    p.TH = 8; p.TW = 32;
    // 128 channels per workgroup (8 waves) where the halo traffic per MFMA is the limit
    p.BN = (bf16 || K == 1) && Cout >= 128 ? 128 : Cout <= 16 ? 16 : Cout <= 32 ? 32 : 64;
    p.CK = bf16 ? Elem<true>::CK : Elem<false>::CK;
    p.tilesH = (p.OH + p.TH - 1) / p.TH;
    p.tilesW = (p.OW + p.TW - 1) / p.TW;
    p.ocTiles = (Cout + p.BN - 1) / p.BN;
    p.CoutPad = p.ocTiles * p.BN;
    p.nChunk = (Cin + p.CK - 1) / p.CK;
    const size_t esz = bf16 ? 2 : 4;
    p.wpack_bytes = ((size_t)p.nChunk * K * K * p.CoutPad * p.CK * esz + 255) & ~(size_t)255;
    p.part_bytes = pool ? (size_t)N * Cout * p.tilesH * p.tilesW * sizeof(float) : 0;
    return p;
}

hipError_t launch_conv_general(const ConvPlan& p, const void* x, const void* w, const float* b, float* out,
                               void* workspace, hipStream_t stream, KernelTimer* timer) {
    unsigned char* ws = (unsigned char*)workspace;
    void* wpk = ws;
    float* part = (float*)(ws + p.wpack_bytes);
    const int taps = p.KS * p.KS;
    const long long total = (long long)p.nChunk * taps * p.CoutPad * p.CK;
    const unsigned pblocks = (unsigned)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
    if (timer) timer->begin("pack_weights", stream);
    if (p.bf16)
        hipLaunchKernelGGL(pack_weights<true>, dim3(pblocks), dim3(256), 0, stream, (const unsigned short*)w,
                           (unsigned short*)wpk, p.Cin, p.Cout, p.CoutPad, taps, total);
    else
        hipLaunchKernelGGL(pack_weights<false>, dim3(pblocks), dim3(256), 0, stream, (const float*)w, (float*)wpk,
                           p.Cin, p.Cout, p.CoutPad, taps, total);
    hipError_t e = hipGetLastError();
    if (timer) timer->end("pack_weights", stream);
    if (e != hipSuccess) return e;
    float* dst = p.pool ? part : out;
    if (timer) timer->begin("conv_general_fused", stream);
    e = p.KS == 1   ? launch_geo_k1(p, x, wpk, b, dst, stream)
        : p.KS == 3 ? launch_geo_k3(p, x, wpk, b, dst, stream)
        : p.KS == 5 ? launch_geo_k5(p, x, wpk, b, dst, stream)
                    : hipErrorInvalidValue;
    if (timer) timer->end("conv_general_fused", stream);
    if (e != hipSuccess || !p.pool) return e;
    if (timer) timer->begin("pool_finalize", stream);
    hipLaunchKernelGGL(pool_finalize, dim3((unsigned)p.N, (unsigned)((p.Cout + 63) / 64)), dim3(256), 0, stream,
                       (const float*)part, out, p.Cout, p.tilesH * p.tilesW, (float)((double)p.OH * (double)p.OW));
    e = hipGetLastError();
    if (timer) timer->end("pool_finalize", stream);
    return e;
}

}  // namespace fconv
