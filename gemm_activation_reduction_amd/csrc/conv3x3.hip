// Fused 3x3 valid convolution + bias + activation (+ global average pool) for gfx950.
//
// The convolution is an implicit GEMM: rows = output pixels, columns = output
// channels, reduction index k = (input channel, tap). It is evaluated as nine
// shifted "tap GEMMs" over a halo tile held in LDS, on MFMA:
//   fp32:  v_mfma_f32_16x16x4_f32   (full fp32 products, fp32 accumulation)
//   bf16:  v_mfma_f32_16x16x32_bf16 (exact bf16 products, fp32 accumulation)
// The activation runs on the accumulators in registers; with pooling, each
// workgroup reduces its pixels per output channel (wave64 butterfly, then LDS
// across waves) and writes one partial per (n, oc, tile); a second kernel sums
// the partials in a fixed order, so the result is deterministic without atomics.
//
// The operation is the Conv2d -> activation (-> AdaptiveAvgPool2d(1)) chain of
// the "Kimi-K2.6 l2_p67" and "Kimi-K2.6 l2_p4" POPCORNBENCH pages; the pages'
// own kernels (shared-memory direct convolution on CUDA cores) are not followed.
//
// LDS layout. Both the halo tile and the weight slice use 80-byte rows: 64 bytes
// of channel data (16 fp32 or 32 bf16 channels, channel-minor) plus 16 bytes of
// padding. A fragment read is one 16-byte ds_read per lane at row r + lane%16,
// byte offset 16 * (lane/16); with the 20-dword row pitch the 16 rows hit
// disjoint banks, so the reads are conflict-free.
//
// Reduction-order freedom: the MFMA sums A[i][k] B[k][j] over whichever k the
// lanes supply, so lane group g supplies the 16-byte channel group g of a tap
// for both operands (fp32: channels 4g..4g+3, one per MFMA step; bf16: channels
// 8g..8g+7 in one step). A and B agree on the pairing, which is all that matters.
#include <cstdint>

#include "device_math.h"
#include "internal.h"

namespace fconv {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kRow = 80;  // bytes per LDS row (64 data + 16 pad)

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

template <int TH_, int TW_, int BN_, int WP_, int WO_>
struct Tile {
    static constexpr int TH = TH_, TW = TW_, BN = BN_, WP = WP_, WO = WO_;
    static constexpr int CB = TW / 16;          // 16-pixel blocks per tile row
    static constexpr int PB = TH * CB;          // pixel blocks per tile
    static constexpr int OB = BN / 16;          // oc blocks per tile
    static constexpr int WPB = PB / WP;         // pixel blocks per wave
    static constexpr int WOB = OB / WO;         // oc blocks per wave
    static constexpr int HR = TH + 2, HC = TW + 2, HPOS = HR * HC;
    static constexpr int LDS = HPOS * kRow + 9 * BN * kRow;
    static_assert(WP * WO == kThreads / 64, "four waves");
    static_assert(PB % WP == 0 && OB % WO == 0, "even wave split");
    static_assert(TW % 16 == 0 && BN % 16 == 0, "MFMA block multiples");
};

// Tile configurations (index = ConvPlan::tile_cfg).
using TileA = Tile<8, 32, 64, 4, 1>;   // 256 pixels x 64 oc; wave = 4 pixel blocks x 4 oc blocks

// Repack OIHW weights to [chunk][tap][CoutPad][CK], zero-filling channels >= Cin and
// oc >= Cout, so a workgroup's slice for one chunk is 9 contiguous [BN][CK] blocks.
template <bool BF16>
__global__ void pack_weights(const typename Elem<BF16>::T* __restrict__ w,
                             typename Elem<BF16>::T* __restrict__ wp,
                             int Cin, int Cout, int CoutPad, long long total) {
    using T = typename Elem<BF16>::T;
    constexpr int CK = Elem<BF16>::CK;
    for (long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (long long)gridDim.x * blockDim.x) {
        int c = (int)(idx % CK);
        long long r = idx / CK;
        int oc = (int)(r % CoutPad);
        r /= CoutPad;
        int tap = (int)(r % 9);
        int chunk = (int)(r / 9);
        int ic = chunk * CK + c;
        T v = 0;
        if (oc < Cout && ic < Cin) v = w[((long long)oc * Cin + ic) * 9 + tap];
        wp[idx] = v;
    }
}

template <bool BF16>
__device__ __forceinline__ u4 load_group(const typename Elem<BF16>::T* __restrict__ src,
                                         long long plane, int nvalid) {
    // Loads EPG consecutive channels (stride = plane) at one pixel; channels at or
    // beyond nvalid read as zero.
    if constexpr (!BF16) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = e < nvalid ? src[e * plane] : 0.0f;
        u4 r;
        r.x = __float_as_uint(v[0]); r.y = __float_as_uint(v[1]);
        r.z = __float_as_uint(v[2]); r.w = __float_as_uint(v[3]);
        return r;
    } else {
        unsigned int h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = e < nvalid ? (unsigned int)src[e * plane] : 0u;
        u4 r;
        r.x = h[0] | (h[1] << 16); r.y = h[2] | (h[3] << 16);
        r.z = h[4] | (h[5] << 16); r.w = h[6] | (h[7] << 16);
        return r;
    }
}

template <bool BF16, int ACT, bool POOL, class TL>
__global__ __launch_bounds__(kThreads) void conv3x3_fused(
    const typename Elem<BF16>::T* __restrict__ x, const typename Elem<BF16>::T* __restrict__ wp,
    const float* __restrict__ bias, float* __restrict__ dst, int Cin, int H, int W, int Cout,
    int CoutPad, int nChunk, int tilesH, int tilesW, int ocTiles, int out_align) {
    using T = typename Elem<BF16>::T;
    constexpr int CK = Elem<BF16>::CK;
    constexpr int EPG = Elem<BF16>::EPG;
    __shared__ __attribute__((aligned(16))) unsigned char smem[TL::LDS];
    unsigned char* halo = smem;
    unsigned char* wl = smem + TL::HPOS * kRow;

    int bid = blockIdx.x;
    const int ot = bid % ocTiles; bid /= ocTiles;
    const int tw = bid % tilesW; bid /= tilesW;
    const int th = bid % tilesH;
    const int n = bid / tilesH;
    const int OH = H - 2, OW = W - 2;
    const int oh0 = th * TL::TH, ow0 = tw * TL::TW, oc0 = ot * TL::BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, i = lane & 15;
    const int wpi = wave % TL::WP, woi = wave / TL::WP;

    f4 acc[TL::WPB][TL::WOB];
#pragma unroll
    for (int a = 0; a < TL::WPB; ++a)
#pragma unroll
        for (int c = 0; c < TL::WOB; ++c) acc[a][c] = f4{0.f, 0.f, 0.f, 0.f};

    const long long plane = (long long)H * W;
    const T* xn = x + (long long)n * Cin * plane;

    for (int ch = 0; ch < nChunk; ++ch) {
        if (ch) __syncthreads();
        const int c0 = ch * CK;
        // Halo tile: (TH+2) x (TW+2) positions, 4 channel groups each.
        for (int it = tid; it < TL::HPOS * 4; it += kThreads) {
            const int pos = it % TL::HPOS, q = it / TL::HPOS;
            const int ih = oh0 + pos / TL::HC, iw = ow0 + pos % TL::HC;
            const int cbase = c0 + q * EPG;
            int nvalid = (ih < H && iw < W) ? Cin - cbase : 0;
            const T* src = xn + (long long)cbase * plane + (long long)ih * W + iw;
            u4 v = load_group<BF16>(src, plane, nvalid);
            *(u4*)(halo + pos * kRow + q * 16) = v;
        }
        // Weight slice: 9 taps x BN oc x 64 bytes.
        const T* wsrc = wp + ((long long)ch * 9 * CoutPad + oc0) * CK;
        for (int it = tid; it < 9 * TL::BN * 4; it += kThreads) {
            const int q = it & 3, r = it >> 2;
            const int o = r % TL::BN, tap = r / TL::BN;
            const u4* src = (const u4*)(wsrc + ((long long)tap * CoutPad + o) * CK) + q;
            *(u4*)(wl + r * kRow + q * 16) = *src;
        }
        __syncthreads();

#pragma unroll
        for (int tap = 0; tap < 9; ++tap) {
            const int kh = tap / 3, kw = tap % 3;
            u4 a[TL::WPB], b[TL::WOB];
#pragma unroll
            for (int j = 0; j < TL::WPB; ++j) {
                const int pb = wpi * TL::WPB + j;
                const int pos = (pb / TL::CB + kh) * TL::HC + (pb % TL::CB) * 16 + i + kw;
                a[j] = *(const u4*)(halo + pos * kRow + g * 16);
            }
#pragma unroll
            for (int j = 0; j < TL::WOB; ++j) {
                const int o = (woi * TL::WOB + j) * 16 + i;
                b[j] = *(const u4*)(wl + (tap * TL::BN + o) * kRow + g * 16);
            }
            if constexpr (!BF16) {
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int jp = 0; jp < TL::WPB; ++jp)
#pragma unroll
                        for (int jo = 0; jo < TL::WOB; ++jo)
                            acc[jp][jo] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                __uint_as_float(a[jp][s]), __uint_as_float(b[jo][s]), acc[jp][jo], 0, 0, 0);
            } else {
#pragma unroll
                for (int jp = 0; jp < TL::WPB; ++jp)
#pragma unroll
                    for (int jo = 0; jo < TL::WOB; ++jo)
                        acc[jp][jo] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, a[jp]), __builtin_bit_cast(bf16x8, b[jo]),
                            acc[jp][jo], 0, 0, 0);
            }
        }
    }

    // Epilogue. Accumulator layout (16x16 MFMA output): lane (g, i) register r holds
    // pixel 4g + r of the pixel block and output channel i of the oc block.
    float bv[TL::WOB];
#pragma unroll
    for (int j = 0; j < TL::WOB; ++j) {
        const int oc = oc0 + (woi * TL::WOB + j) * 16 + i;
        bv[j] = oc < Cout ? bias[oc] : 0.0f;
    }

    if constexpr (POOL) {
        float psum[TL::WOB];
#pragma unroll
        for (int j = 0; j < TL::WOB; ++j) psum[j] = 0.0f;
#pragma unroll
        for (int jp = 0; jp < TL::WPB; ++jp) {
            const int pb = wpi * TL::WPB + jp;
            const int oh = oh0 + pb / TL::CB;
            const int owb = ow0 + (pb % TL::CB) * 16 + 4 * g;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool valid = oh < OH && owb + r < OW;
#pragma unroll
                for (int jo = 0; jo < TL::WOB; ++jo) {
                    const float v = activate<ACT>(acc[jp][jo][r] + bv[jo]);
                    psum[jo] += valid ? v : 0.0f;
                }
            }
        }
#pragma unroll
        for (int jo = 0; jo < TL::WOB; ++jo) {
            psum[jo] += __shfl_xor(psum[jo], 16, 64);
            psum[jo] += __shfl_xor(psum[jo], 32, 64);
        }
        __syncthreads();  // all waves are done with the halo / weight LDS
        float* red = (float*)smem;
        if (g == 0) {
#pragma unroll
            for (int jo = 0; jo < TL::WOB; ++jo)
                red[wpi * TL::BN + (woi * TL::WOB + jo) * 16 + i] = psum[jo];
        }
        __syncthreads();
        if (tid < TL::BN) {
            float s = 0.0f;
#pragma unroll
            for (int p = 0; p < TL::WP; ++p) s += red[p * TL::BN + tid];
            const int oc = oc0 + tid;
            const int nTiles = tilesH * tilesW;
            if (oc < Cout) dst[((long long)n * Cout + oc) * nTiles + th * tilesW + tw] = s;
        }
    } else {
#pragma unroll
        for (int jp = 0; jp < TL::WPB; ++jp) {
            const int pb = wpi * TL::WPB + jp;
            const int oh = oh0 + pb / TL::CB;
            const int owb = ow0 + (pb % TL::CB) * 16 + 4 * g;
            if (oh >= OH) continue;
#pragma unroll
            for (int jo = 0; jo < TL::WOB; ++jo) {
                const int oc = oc0 + (woi * TL::WOB + jo) * 16 + i;
                if (oc >= Cout) continue;
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = activate<ACT>(acc[jp][jo][r] + bv[jo]);
                float* o = dst + (((long long)n * Cout + oc) * OH + oh) * OW + owb;
                // out_align: 16 / 8 / 4 = byte alignment of the output base pointer
                if ((OW & 3) == 0 && out_align >= 16 && owb + 3 < OW) {
                    *(f4*)o = f4{v[0], v[1], v[2], v[3]};
                } else if ((OW & 1) == 0 && out_align >= 8) {
                    // owb is even, so each pair is in range together and 8-byte aligned
                    if (owb < OW) *(float2*)o = make_float2(v[0], v[1]);
                    if (owb + 2 < OW) *(float2*)(o + 2) = make_float2(v[2], v[3]);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (owb + r < OW) o[r] = v[r];
                }
            }
        }
    }
}

// Sum of the per-tile partials of one (n, oc) map in a fixed order, divided by the
// number of valid output positions. One wave per (n, oc).
__global__ __launch_bounds__(256) void pool_finalize(const float* __restrict__ part,
                                                     float* __restrict__ out, int NC, int nTiles,
                                                     float area) {
    const int wv = (int)(((long long)blockIdx.x * blockDim.x + threadIdx.x) >> 6);
    const int lane = threadIdx.x & 63;
    if (wv >= NC) return;
    const float* p = part + (long long)wv * nTiles;
    float s = 0.0f;
    for (int t = lane; t < nTiles; t += 64) s += p[t];
    s = wave_sum(s);
    if (lane == 0) out[wv] = s / area;
}

template <bool BF16, int ACT, bool POOL, class TL>
hipError_t launch_typed(const ConvPlan& p, const void* x, const void* wpk, const float* b,
                        float* dst, hipStream_t stream) {
    using T = typename Elem<BF16>::T;
    hipLaunchKernelGGL((conv3x3_fused<BF16, ACT, POOL, TL>), dim3((unsigned)p.grid()), dim3(kThreads), 0,
                       stream, (const T*)x, (const T*)wpk, b, dst, p.Cin, p.H, p.W, p.Cout, p.CoutPad,
                       p.nChunk, p.tilesH, p.tilesW, p.ocTiles,
                       ((uintptr_t)dst % 16 == 0) ? 16 : ((uintptr_t)dst % 8 == 0 ? 8 : 4));
    return hipGetLastError();
}

template <bool BF16, class TL>
hipError_t launch_act(const ConvPlan& p, const void* x, const void* wpk, const float* b, float* dst,
                      hipStream_t stream) {
    switch (p.act * 2 + p.pool) {
        case 0: return launch_typed<BF16, kActNone, false, TL>(p, x, wpk, b, dst, stream);
        case 1: return launch_typed<BF16, kActNone, true, TL>(p, x, wpk, b, dst, stream);
        case 2: return launch_typed<BF16, kActGelu, false, TL>(p, x, wpk, b, dst, stream);
        case 3: return launch_typed<BF16, kActGelu, true, TL>(p, x, wpk, b, dst, stream);
        case 4: return launch_typed<BF16, kActMish2, false, TL>(p, x, wpk, b, dst, stream);
        case 5: return launch_typed<BF16, kActMish2, true, TL>(p, x, wpk, b, dst, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

ConvPlan plan_conv(bool bf16, int act, int pool, int N, int Cin, int H, int W, int Cout) {
    ConvPlan p{};
    p.bf16 = bf16; p.act = act; p.pool = pool;
    p.N = N; p.Cin = Cin; p.H = H; p.W = W; p.Cout = Cout;
    p.OH = H - 2; p.OW = W - 2;
    p.tile_cfg = 0;
    p.TH = TileA::TH; p.TW = TileA::TW; p.BN = TileA::BN;
    p.CK = bf16 ? Elem<true>::CK : Elem<false>::CK;
    p.tilesH = (p.OH + p.TH - 1) / p.TH;
    p.tilesW = (p.OW + p.TW - 1) / p.TW;
    p.ocTiles = (Cout + p.BN - 1) / p.BN;
    p.CoutPad = p.ocTiles * p.BN;
    p.nChunk = (Cin + p.CK - 1) / p.CK;
    const size_t esz = bf16 ? 2 : 4;
    p.wpack_bytes = ((size_t)p.nChunk * 9 * p.CoutPad * p.CK * esz + 255) & ~(size_t)255;
    p.part_bytes = pool ? (size_t)N * Cout * p.tilesH * p.tilesW * sizeof(float) : 0;
    return p;
}

hipError_t launch_conv(const ConvPlan& p, const void* x, const void* w, const float* b, float* out,
                       void* workspace, hipStream_t stream, KernelTimer* timer) {
    unsigned char* ws = (unsigned char*)workspace;
    void* wpk = ws;
    float* part = (float*)(ws + p.wpack_bytes);
    const long long total = (long long)p.nChunk * 9 * p.CoutPad * p.CK;
    const unsigned pblocks = (unsigned)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
    if (timer) timer->begin("pack_weights", stream);
    if (p.bf16)
        hipLaunchKernelGGL(pack_weights<true>, dim3(pblocks), dim3(256), 0, stream,
                           (const unsigned short*)w, (unsigned short*)wpk, p.Cin, p.Cout, p.CoutPad, total);
    else
        hipLaunchKernelGGL(pack_weights<false>, dim3(pblocks), dim3(256), 0, stream, (const float*)w,
                           (float*)wpk, p.Cin, p.Cout, p.CoutPad, total);
    hipError_t e = hipGetLastError();
    if (timer) timer->end("pack_weights", stream);
    if (e != hipSuccess) return e;
    float* dst = p.pool ? part : out;
    if (timer) timer->begin("conv3x3_fused", stream);
    e = p.bf16 ? launch_act<true, TileA>(p, x, wpk, b, dst, stream)
               : launch_act<false, TileA>(p, x, wpk, b, dst, stream);
    if (timer) timer->end("conv3x3_fused", stream);
    if (e != hipSuccess || !p.pool) return e;
    const int NC = p.N * p.Cout;
    const unsigned fblocks = (unsigned)((NC + 3) / 4);
    if (timer) timer->begin("pool_finalize", stream);
    hipLaunchKernelGGL(pool_finalize, dim3(fblocks), dim3(256), 0, stream, (const float*)part, out, NC,
                       p.tilesH * p.tilesW, (float)((double)p.OH * (double)p.OW));
    e = hipGetLastError();
    if (timer) timer->end("pool_finalize", stream);
    return e;
}

}  // namespace fconv
