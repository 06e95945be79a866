// Pieces shared by the two fused convolution kernels (3x3 valid, general geometry):
// element traits, raw buffer resources, the XCD-contiguous workgroup order, the weight
// repack and the second level of the global average pool.
#pragma once
#include <cstdint>

#include <hip/hip_runtime.h>

namespace fconv {
namespace {  // internal linkage: each source that includes this gets its own copy

template <bool BF16> struct Elem;
template <> struct Elem<false> {
    using T = float;
    static constexpr int CK = 16;   // channels per K chunk
    static constexpr int EPG = 4;   // elements per 16-byte group
};
template <> struct Elem<true> {
    using T = unsigned short;       // bfloat16 bit pattern
    static constexpr int CK = 32;
    static constexpr int EPG = 8;
};

// All staging loads are raw buffer loads: the resource covers one image of x (or the
// repacked weights), offsets are 32-bit, and an offset past the end (kOOB) reads as zero
// without touching memory -- so padding channels, rows below the image and columns
// right of it are zero-filled without branches around the loads.
constexpr int kOOB = 0x7FFFFFF0;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Workgroups are dispatched to the 8 XCDs round-robin by blockIdx.x; renumber them so
// each XCD receives a contiguous range of logical tiles (neighbouring spatial tiles and
// all oc tiles of a spatial tile share that XCD's L2).
__device__ __forceinline__ int xcd_contiguous_index(int b, int G) {
    const int xcd = b & 7, idx = b >> 3, per = G >> 3, rem = G & 7;
    return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

// Repack OIHW weights [Cout][Cin][K][K] to [chunk][tap][CoutPad][CK] (tap = kh K + kw),
// zero-filling channels >= Cin and oc >= Cout, so a workgroup's slice for one chunk is
// `taps` = K^2 contiguous [BN][CK] blocks.
template <bool BF16>
__global__ void pack_weights(const typename Elem<BF16>::T* __restrict__ w,
                             typename Elem<BF16>::T* __restrict__ wp,
                             int Cin, int Cout, int CoutPad, int taps, long long total) {
    using T = typename Elem<BF16>::T;
    constexpr int CK = Elem<BF16>::CK;
    for (long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (long long)gridDim.x * blockDim.x) {
        int c = (int)(idx % CK);
        long long r = idx / CK;
        int oc = (int)(r % CoutPad);
        r /= CoutPad;
        int tap = (int)(r % taps);
        int chunk = (int)(r / taps);
        int ic = chunk * CK + c;
        T v = 0;
        if (oc < Cout && ic < Cin) v = w[((long long)oc * Cin + ic) * taps + tap];
        wp[idx] = v;
    }
}

// Pool level 2: out[n][oc] = (sum over tiles t of part[n][t][oc]) / area, summed in a
// fixed order. One workgroup per (image, 64 output channels); its four waves take four
// contiguous tile ranges (lanes = consecutive channels, so every load is one 256-byte
// row), and the four range sums are added in range order through LDS.
__global__ __launch_bounds__(256) void pool_finalize(const float* __restrict__ part, float* __restrict__ out,
                                                     int Cout, int nTiles, float area) {
    __shared__ float red[4][64];
    const int n = blockIdx.x, lane = threadIdx.x & 63, sl = threadIdx.x >> 6;
    const int oc = blockIdx.y * 64 + lane;
    const int per = (nTiles + 3) / 4, t0 = sl * per, t1 = min(nTiles, t0 + per);
    float s = 0.0f;
    if (oc < Cout) {
        const float* p = part + (long long)n * nTiles * Cout + oc;
#pragma unroll 8
        for (int t = t0; t < t1; ++t) s += p[(long long)t * Cout];
    }
    red[sl][lane] = s;
    __syncthreads();
    if (sl == 0 && oc < Cout) out[(long long)n * Cout + oc] = ((red[0][lane] + red[1][lane]) + red[2][lane] + red[3][lane]) / area;
}

}  // namespace
}  // namespace fconv
