// Fused K x K convolution (K = 1, 3 or 5) with stride 1 or 2 and zero padding, + bias +
// activation (+ global average pool), for gfx950.
//
// The same implicit GEMM as the 3x3 valid kernel (rows = output pixels, columns = output
// channels, k = (input channel, kh, kw)) on the same MFMA instructions, with the geometry
// nn.Conv2d's kernel_size / stride / padding describe:
//   pre[n,oc,oh,ow] = b[oc] + sum_{ic,kh,kw} w[oc,ic,kh,kw] x[n,ic,oh S + kh - P,ow S + kw - P],
// x reading zero outside the image, OH = (H + 2P - K)/S + 1, OW = (W + 2P - K)/S + 1.
// The pages fix K = 3, S = 1, P = 0 (the direct-convolution sum of the "Kimi-K2.6 l2_p4"
// page); this kernel opens those three parameters up.
//
// K loop. One step is (channel chunk, kernel row kh): LDS holds, for the tile's TH
// output rows, the one input row each needs for this kh (TW-wide output -> (TW-1) S + K
// input columns) and the K weight taps of that kernel row. Each halo row is staged K
// times per chunk (once per kh) instead of once; in exchange the LDS footprint no longer
// grows with K^2 or with S on the row axis, so two workgroups still fit on a CU at K = 5.
//
// Channel width. A workgroup computes 64 output channels with 4 waves, or, for bf16 and for
// 1x1 kernels with at least 128 output channels, 128 channels with 8 waves (4 pixel groups
// x 2 channel halves) sharing one staged halo. The wide tile halves the halo bytes that pass
// through the vector memory path per MFMA (3x3 stride 2 bf16: TA busy 58 % -> 37 %, 24 %
// faster; 1x1 fp32: x read once per pixel tile instead of twice, 12 % faster). It runs one
// workgroup per CU (about 200 registers per lane for bf16 at 3x3).
//
// Stride 2: halo columns are stored split by parity (even columns, then odd), so the 16
// output columns of a fragment read 16 consecutive LDS rows for every tap -- the same
// conflict-free pattern as stride 1.
//
// fp32 1x1 stride-1 layers with 16-byte halo runs stage each chunk by LDS DMA into a double
// buffer instead (GeoDma below), and fp32 stride-1 3x3
// and 5x5 layers with 16-byte halo runs stage each chunk's whole halo, and each kernel row's
// weights, by LDS DMA (GeoDmaK below).
//
// Halo loads: when W is a whole number of 16-byte pixel groups and x is 16-byte aligned,
// 16-byte runs along W (ow0 S is a multiple of 32, so the misalignment (-P) mod run is
// the same for every tile and every aligned run lies wholly inside or wholly outside the
// image; outside runs read as zero), transposed to channel-minor rows in registers.
// Otherwise element-wise loads with a bounds test per element. Both zero-fill padding.
//
// This header holds the kernel and its launch templates; conv_general_k1.hip, _k3.hip and
// _k5.hip instantiate them for one kernel size each (three translation units that
// compile in parallel), and conv_general.hip plans, repacks the weights, dispatches and
// finalizes the pool.
#pragma once
#include <cstdint>
#include <type_traits>

#include "conv_common.h"
#include "device_math.h"
#include "internal.h"

namespace fconv {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kGRow = 80;  // bytes per LDS row: 64 bytes of channel data + 16 of padding

// WO = 1: 64 output channels per workgroup, 4 waves. WO = 2: 128 output channels, 8 waves
// (4 pixel groups x 2 channel halves): the staged halo of a step feeds twice the MFMAs, so
// the halo bytes moved through the vector memory path per MFMA halve. BN_ = 16 or 32 (with
// WO = 1) is the tile of layers with at most 16 or 32 output channels: 4 waves of 4 pixel
// blocks x 1 or 2 oc blocks, so a narrow layer does not spend MFMA work and weight staging
// on padding channels.
template <int KS_, int S_, int WO_ = 1, int OCC_ = 2, int BN_ = 64 * WO_>
struct GeoTile {
    static constexpr int KS = KS_, S = S_, WO = WO_;
    static constexpr int OCC = OCC_;                            // waves per SIMD the registers are fit to
    static constexpr int TH = 8, TW = 32, BN = BN_, NT = 256 * WO;
    static_assert(BN % (16 * WO) == 0 && BN <= 64 * WO, "whole oc blocks per wave");
    static constexpr int WP = 4;                                // pixel wave groups; each wave 4 pixel blocks
    static constexpr int CB = TW / 16, PB = TH * CB, OB = BN / 16, WPB = PB / WP, WOB = OB / WO;
    static constexpr int HC = (TW - 1) * S + KS;                // input columns per staged row
    static constexpr int HCS = (HC + S - 1) / S;                // positions per column-parity plane
    static constexpr int HPP0 = S * HCS;
    static constexpr int HPP = HPP0 + ((4 - HPP0 % 8) + 8) % 8;  // row pitch = 4 (mod 8) positions
    static constexpr int HPOS = TH * HPP;
    static constexpr int LDS = HPOS * kGRow + KS * BN * kGRow;
    static_assert(PB % WP == 0, "even wave split");
};

// Halo rows of one step: for each tile row r, input row (oh0 + r) S + kh - P, input
// columns ow0 S - P + j for j < HC, CK channels as 4 groups of EPG.
template <bool BF16, class TL>
struct GeoHalo {
    using T = typename Elem<BF16>::T;
    static constexpr int ESZ = (int)sizeof(T);
    static constexpr int EPG = Elem<BF16>::EPG;
    static constexpr int ITEMS = TL::TH * TL::HC * 4;  // (row, column, channel group)
    static constexpr int PER = (ITEMS + TL::NT - 1) / TL::NT;
    u4 v[PER];

    __device__ __forceinline__ void setup(int, int, int, int) {}

    __device__ __forceinline__ static bool last_used(int tid) {
        return ITEMS % TL::NT == 0 || (__builtin_amdgcn_readfirstlane(tid) & ~63) + (PER - 1) * TL::NT < ITEMS;
    }

    template <bool WITH_LAST = true>
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t xr, int H, int W, int Cin, int c0, int ih0,
                                         int iw0, int tid) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            if (!WITH_LAST && j == PER - 1) continue;  // no lane of this wave holds an item in round j
            const int it = tid + j * TL::NT;
            const int q = it & 3, pos = it >> 2;
            const int r = pos / TL::HC, col = pos % TL::HC;
            const int ih = ih0 + r * TL::S, iw = iw0 + col;
            const bool inb = it < ITEMS && ih >= 0 && ih < H && iw >= 0 && iw < W;
            const int cb = c0 + q * EPG;
            const int base = (cb * H + ih) * W + iw;
            unsigned h[EPG];
#pragma unroll
            for (int e = 0; e < EPG; ++e) {
                const int off = (inb && cb + e < Cin) ? (base + e * H * W) * ESZ : kOOB;
                if constexpr (!BF16) h[e] = __builtin_amdgcn_raw_buffer_load_b32(xr, off, 0, 0);
                else h[e] = __builtin_amdgcn_raw_buffer_load_b16(xr, off, 0, 0);
            }
            if constexpr (!BF16) v[j] = u4{h[0], h[1], h[2], h[3]};
            else v[j] = u4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        }
    }

    __device__ __forceinline__ void store(unsigned char* halo, int tid) const {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int it = tid + j * TL::NT;
            if (ITEMS % TL::NT != 0 && it >= ITEMS) continue;
            const int pos = it >> 2;
            const int r = pos / TL::HC, col = pos % TL::HC;
            const int lp = r * TL::HPP + (col % TL::S) * TL::HCS + col / TL::S;
            *(u4*)(halo + lp * kGRow + (it & 3) * 16) = v[j];
        }
    }
};

// Vector form of the halo rows: item (channel group q, aligned column group cg, row r)
// loads one 16-byte run of VW pixels from each of the EPG channels of group q, then writes
// one LDS row per pixel that falls in the staged columns. As in the 3x3 kernel, eight
// consecutive lanes store to distinct bank slots: fp32 pairs adjacent column groups,
// bf16 (whose adjacent groups share banks at stride 1) pairs adjacent rows, which the
// row pitch = 4 (mod 8) separates.
template <bool BF16, class TL>
struct GeoHaloVec {
    using T = typename Elem<BF16>::T;
    static constexpr int ESZ = (int)sizeof(T);
    static constexpr int EPG = Elem<BF16>::EPG;
    static constexpr int VW = 16 / ESZ;                       // pixels per 16-byte run
    static constexpr int NCG = (TL::HC + 2 * VW - 2) / VW;    // runs per row at any misalignment
    static constexpr int ITEMS = TL::TH * NCG * 4;
    static constexpr int PER = (ITEMS + TL::NT - 1) / TL::NT;
    static_assert(!BF16 || TL::TH % 2 == 0, "bf16 staging pairs rows");
    u4 v[PER][EPG];

    __device__ __forceinline__ static void item(int it, int& q, int& cg, int& r) {
        q = it & 3;
        if constexpr (!BF16) {
            cg = (it >> 2) % NCG;
            r = (it >> 2) / NCG;
        } else {
            cg = (it >> 3) % NCG;
            r = 2 * ((it >> 3) / NCG) + ((it >> 2) & 1);
        }
    }

    // Per-thread parts of the run addresses, fixed for the whole K loop: the element offset
    // of the item's run within the image at channel 0 and input row 0 of the step, the row
    // step r S, and whether the run's columns lie inside the image (a0: first aligned input
    // column, iw0 - mis, a multiple of VW).
    int lane_off[PER], lane_rs[PER];
    unsigned col_ok;

    __device__ __forceinline__ void setup(int H, int W, int a0, int tid) {
        col_ok = 0;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int it = tid + j * TL::NT;
            int q, cg, r;
            item(it, q, cg, r);
            const int iw = a0 + cg * VW;
            if (it < ITEMS && iw >= 0 && iw < W) col_ok |= 1u << j;
            lane_off[j] = (q * EPG * H + r * TL::S) * W + cg * VW;
            lane_rs[j] = r * TL::S;
        }
    }

    // Step (chunk at channel c0, first staged input row ih0). The step's part of every
    // offset is uniform across the workgroup; per run only a row test, a select and one add
    // per channel remain. Offsets past the image read as zero: a run outside the rows or
    // columns starts at kOOB (kOOB + e * plane stays below 2^32 because the image is under
    // 2^31 bytes), and in a chunk that runs past Cin each missing channel takes kOOB.
    // Whether any lane of this wave holds an item in the last round (j = PER - 1); only that
    // round can be short. A wave without one issues none of its loads: an out-of-range load
    // costs the texture unit as much as a real one. Uniform across the wave.
    __device__ __forceinline__ static bool last_used(int tid) {
        return ITEMS % TL::NT == 0 || (__builtin_amdgcn_readfirstlane(tid) & ~63) + (PER - 1) * TL::NT < ITEMS;
    }

    template <bool WITH_LAST = true>
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t xr, int H, int W, int Cin, int c0, int ih0, int a0,
                                         int tid) {
        (void)tid;
        const int step = (c0 * H + ih0) * W + a0;  // |step|, lane_off < 2^30 elements
        const unsigned plane_b = (unsigned)(H * W) * ESZ;
        const bool full = c0 + Elem<BF16>::CK <= Cin;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            if (!WITH_LAST && j == PER - 1) continue;
            const int ih = ih0 + lane_rs[j];
            const bool ok = ((col_ok >> j) & 1u) && (unsigned)ih < (unsigned)H;
            const unsigned b = ok ? (unsigned)(lane_off[j] + step) * ESZ : (unsigned)kOOB;
            const int cb = c0 + (((tid + j * TL::NT) & 3) * EPG);
#pragma unroll
            for (int e = 0; e < EPG; ++e) {
                const unsigned off = (full || cb + e < Cin) ? b + e * plane_b : (unsigned)kOOB;
                v[j][e] = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)off, 0, 0);
            }
        }
    }

    // mis: staged column of aligned pixel 0 is -mis
    __device__ __forceinline__ void store(unsigned char* halo, int mis, int tid) const {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int it = tid + j * TL::NT;
            if (ITEMS % TL::NT != 0 && it >= ITEMS) continue;
            int q, cg, r;
            item(it, q, cg, r);
#pragma unroll
            for (int p = 0; p < VW; ++p) {
                const int col = cg * VW + p - mis;
                if (col < 0 || col >= TL::HC) continue;
                u4 o;
                if constexpr (!BF16) {
                    o = u4{v[j][0][p], v[j][1][p], v[j][2][p], v[j][3][p]};
                } else {
                    // pixel p of channels 2k and 2k+1: one byte permute per output dword
                    const int dw = p >> 1;
                    const unsigned sel = (p & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
                    for (int k = 0; k < 4; ++k) o[k] = __builtin_amdgcn_perm(v[j][2 * k + 1][dw], v[j][2 * k][dw], sel);
                }
                const int lp = r * TL::HPP + (col % TL::S) * TL::HCS + col / TL::S;
                *(u4*)(halo + lp * kGRow + q * 16) = o;
            }
        }
    }
};

// Weights of one step: the K taps (kw) of kernel row kh, BN output channels, 64 bytes each,
// from the repacked [chunk][tap][CoutPad][CK] layout (tap = kh K + kw).
template <bool BF16, class TL>
struct GeoWeights {
    static constexpr int ITEMS = TL::KS * TL::BN * 4;  // (16 rows x 4 groups) per 64 items
    static constexpr int PER = (ITEMS + TL::NT - 1) / TL::NT;
    u4 v[PER];

    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t wr, int CoutPad, int tap0, int oc0, int tid) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int it = tid + j * TL::NT;
            const int q = (it >> 4) & 3, row = (it & 15) + 16 * (it >> 6);
            const int o = row % TL::BN, kw = row / TL::BN;
            const int off = (((tap0 + kw) * CoutPad + oc0 + o) * 4 + q) * 16;
            v[j] = __builtin_amdgcn_raw_buffer_load_b128(wr, (ITEMS % TL::NT == 0 || it < ITEMS) ? off : kOOB, 0, 0);
        }
    }

    __device__ __forceinline__ void store(unsigned char* wl, int tid) const {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int it = tid + j * TL::NT;
            const int q = (it >> 4) & 3, row = (it & 15) + 16 * (it >> 6);
            if (ITEMS % TL::NT == 0 || it < ITEMS) *(u4*)(wl + row * kGRow + q * 16) = v[j];
        }
    }
};

// fp32 1x1 stride-1 layers with 16-byte halo runs stage each chunk by LDS DMA (buffer_load
// ... lds) into one of two buffers, the next chunk's DMA flying while this chunk computes. fp32
// MFMA and VALU work serialize on a SIMD, and the register path spends VALU instructions on
// load addresses, the transpose to channel-minor rows and the LDS stores. The halo stays in
// NCHW order: channel c owns 1 KB at c * 1024 + ((c >> 2) & 3) * 64, its 8 tile rows of 32
// pixels 128 bytes apart. One DMA instruction fills one channel in lane order (lane l: row
// l / 8, 4-pixel run l % 8), so the channel is the only per-instruction part of an address.
// An fp32 fragment (channel 4g + s for lane group g, 16 consecutive pixels) is one
// ds_read_b32 per lane on 64 distinct banks: the skew puts the four groups 16 banks apart.
// The weights arrive as 64-byte rows with K group s of row r in 16-byte slot s ^ ((r >> 1) &
// 3), the layout the LDS-DMA GEMM reads conflict-free.
template <class TL>
struct GeoDma {
    static constexpr int NW = TL::NT / 64;
    static constexpr int HALO_INS = 16;  // one per channel of a chunk
    static constexpr int HALO_BYTES = 16 * 1024 + 256;
    static constexpr int W_INS = (TL::BN / 16 + NW - 1) / NW * NW;  // 16 weight rows each
    static constexpr int BUF = HALO_BYTES + W_INS * 1024;
    static constexpr int LDS = 2 * BUF;
};

// fp32 stride-1 layers with K = 3 or 5 and 16-byte halo runs stage the same way. A chunk's
// whole halo (TH + K - 1 rows, the 40 input columns from ow0 - P rounded down to a 4-pixel run)
// arrives once, as in the 3x3 valid kernel: channel c at c * 2048 + ((c >> 2) & 3) * 64, rows
// 0-5 in its first kilobyte and rows 6-11 in its second (160 bytes each), one DMA instruction
// per (channel, 6-row group) with lane l taking row l / 10, run l % 10. The weights of one
// kernel row (K taps x BN rows of 64 bytes, swizzled as above) go into one of two buffers, the
// next row's DMA flying while this row's K taps compute. At K = 5 all 25 taps of a 64-channel
// tile would not leave room for two workgroups per CU; at K = 3 staging all nine with the halo
// (one barrier per chunk) measured the same as the two row buffers.
template <class TL>
struct GeoDmaK {
    static constexpr int NW = TL::NT / 64;
    static constexpr int RG = 6;                          // halo rows per DMA instruction
    static constexpr int HR = TL::TH + TL::KS - 1;        // halo rows
    static constexpr int HALO_INS = 16 * 2;               // (channel, row group) pairs
    static constexpr int HALO_BYTES = 16 * 2048 + 256;
    static constexpr int W_ROWS = TL::KS * TL::BN;        // one kernel row's weights
    static constexpr int W_INS = (W_ROWS / 16 + NW - 1) / NW * NW;
    static constexpr int WBUF = W_INS * 1024;
    static constexpr int LDS = HALO_BYTES + 2 * WBUF;
    // byte offset of halo row r (0 <= r < 12) inside a channel block
    __device__ __forceinline__ static int row_off(int r) { return r < RG ? r * 160 : 1024 + (r - RG) * 160; }
};

// DMA: 0 = register staging, 1 = the 1x1 double-buffered DMA (GeoDma), 2 = the K x K
// stride-1 DMA (GeoDmaK).
template <bool BF16, bool VEC, int ACT, bool POOL, class TL, int DMA = 0>
__global__ __launch_bounds__(TL::NT) __attribute__((amdgpu_waves_per_eu(TL::OCC))) void conv_general_fused(
    const typename Elem<BF16>::T* __restrict__ x, const typename Elem<BF16>::T* __restrict__ wp,
    const float* __restrict__ bias, float* __restrict__ dst, int Cin, int H, int W, int Cout, int OH, int OW,
    int pad, int CoutPad, int nChunk, int tilesH, int tilesW, int ocTiles, int out_align) {
    using T = typename Elem<BF16>::T;
    constexpr int KS = TL::KS, S = TL::S;
    static_assert(DMA != 1 || (!BF16 && VEC && KS == 1 && S == 1 && TL::TH == 8 && TL::TW == 32),
                  "1x1 DMA staging: fp32 1x1 stride-1 8 x 32 tiles with 16-byte halo runs");
    static_assert(DMA != 1 || GeoDma<TL>::HALO_INS % GeoDma<TL>::NW == 0, "whole DMA instructions per wave");
    static_assert(DMA != 2 || (!BF16 && VEC && (KS == 3 || KS == 5) && S == 1 && TL::TH == 8 && TL::TW == 32),
                  "K x K DMA staging: fp32 stride-1 8 x 32 tiles with 16-byte halo runs");
    static_assert(DMA != 2 || GeoDmaK<TL>::HALO_INS % GeoDmaK<TL>::NW == 0, "whole DMA instructions per wave");
    __shared__ __attribute__((aligned(16))) unsigned char
        smem[DMA == 1 ? GeoDma<TL>::LDS : DMA == 2 ? GeoDmaK<TL>::LDS : TL::LDS];
    unsigned char* halo = smem;
    unsigned char* wl = smem + TL::HPOS * kGRow;

    int bid = xcd_contiguous_index(blockIdx.x, gridDim.x);
    const int ot = bid % ocTiles; bid /= ocTiles;
    const int tw = bid % tilesW; bid /= tilesW;
    const int th = bid % tilesH;
    const int n = bid / tilesH;
    const int oh0 = th * TL::TH, ow0 = tw * TL::TW, oc0 = ot * TL::BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, i = lane & 15;
    const int wpi = wave % TL::WP, woi = wave / TL::WP;  // pixel group, channel group
    // Pixel block pb -> (tile row, 16-column block), rows first.
    auto pb_row = [](int pb) { return pb % TL::TH; };
    auto pb_col = [](int pb) { return pb / TL::TH; };

    // The accumulators start at the bias (lane (g, i) holds output channel i of oc block c
    // in all four registers), which saves the epilogue an add per output.
    f4 acc[TL::WPB][TL::WOB];
#pragma unroll
    for (int c = 0; c < TL::WOB; ++c) {
        const int oc = oc0 + (woi * TL::WOB + c) * 16 + i;
        const float bv = oc < Cout ? bias[oc] : 0.0f;
#pragma unroll
        for (int a = 0; a < TL::WPB; ++a) acc[a][c] = f4{bv, bv, bv, bv};
    }

    const long long plane = (long long)H * W;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + (long long)n * Cin * plane, (unsigned)(Cin * plane * sizeof(T)));
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wp, (unsigned)(nChunk * KS * KS * CoutPad * 64));
    const int iw0 = ow0 * S - pad;

    // The K taps of one kernel row over the staged rows.
    // bf16 A fragments: one per-lane base (the wave's first block) plus an immediate per
    // block and tap (a wave's blocks are rows j of one block column). Written through the
    // block index wpi * WPB + j, the compiler kept a position per fragment in registers
    // (1.7 % slower at 3x3 stride 2); fp32 keeps that form, which measured 0.2-0.8 % faster
    // there.
    static_assert(TL::TH % TL::WPB == 0, "a wave's blocks share one block column");
    const unsigned char* a_base =
        halo + (((wpi * TL::WPB) % TL::TH) * TL::HPP + ((wpi * TL::WPB) / TL::TH) * 16 + i) * kGRow + g * 16;
    auto compute_step = [&]() {
#pragma unroll
        for (int kw = 0; kw < KS; ++kw) {
            u4 a[TL::WPB], b[TL::WOB];
#pragma unroll
            for (int j = 0; j < TL::WPB; ++j) {
                if constexpr (BF16) {
                    a[j] = *(const u4*)(a_base + (j * TL::HPP + (kw % S) * TL::HCS + kw / S) * kGRow);
                } else {
                    const int pb = wpi * TL::WPB + j;
                    const int pos = pb_row(pb) * TL::HPP + (kw % S) * TL::HCS + pb_col(pb) * 16 + i + kw / S;
                    a[j] = *(const u4*)(halo + pos * kGRow + g * 16);
                }
            }
#pragma unroll
            for (int j = 0; j < TL::WOB; ++j)
                b[j] = *(const u4*)(wl + (kw * TL::BN + (woi * TL::WOB + j) * 16 + i) * kGRow + g * 16);
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
                            __builtin_bit_cast(bf16x8, a[jp]), __builtin_bit_cast(bf16x8, b[jo]), acc[jp][jo], 0,
                            0, 0);
            }
        }
    };

    if constexpr (DMA == 1) {
        typedef __attribute__((address_space(3))) void lds_t;
        using DL = GeoDma<TL>;
        constexpr int NW = DL::NW;
        constexpr int CK = Elem<false>::CK;
        const int wave_u = __builtin_amdgcn_readfirstlane(wave);
        // Halo: lane l takes row l / 8, pixels ow0 + 4 (l % 8) .. + 3; a run lies wholly inside
        // or outside the image (W % 4 == 0), outside runs and channels past Cin read zero.
        const int lr = lane >> 3, lrun = lane & 7;
        const bool lane_ok = oh0 + lr < H && ow0 + 4 * lrun < W;
        const int lane_off = (lr * W + 4 * lrun) * 4;
        const int w_lane = ((lane >> 2) * 4 + ((lane & 3) ^ ((lane >> 3) & 3))) * 16;
        auto stage = [&](int ch, unsigned char* buf) {
            const int c0 = ch * CK;
#pragma unroll
            for (int k = 0; k < DL::HALO_INS / NW; ++k) {
                const int c = wave_u + NW * k;  // wave-uniform
                // unsigned: a channel past Cin (kOOB below) may lie past 2^31 bytes
                const int ubase = (int)__builtin_amdgcn_readfirstlane((((unsigned)(c0 + c) * H + oh0) * W + ow0) * 4u);
                const int off = c0 + c < Cin && lane_ok ? ubase + lane_off : kOOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_t*)(buf + c * 1024 + ((c >> 2) & 3) * 64), 16, off,
                                                         0, 0, 0);
            }
            // Weights: instruction ins fills rows 16 ins .. 16 ins + 15; lane l takes row
            // 16 ins + l / 4 and 16-byte slot l % 4, which holds K group (l % 4) ^ ((l / 4 >> 1) & 3).
            unsigned char* wb = buf + DL::HALO_BYTES;
#pragma unroll
            for (int k = 0; k < DL::W_INS / NW; ++k) {
                const int ins = wave_u + NW * k;
                const int ubase = __builtin_amdgcn_readfirstlane((ch * CoutPad + oc0 + ins * 16) * 64);
                const int off = ins * 16 < TL::BN ? ubase + w_lane : kOOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_t*)(wb + ins * 1024), 16, off, 0, 0, 0);
            }
        };
        auto compute = [&](const unsigned char* buf) {
            const unsigned char* wb = buf + DL::HALO_BYTES;
            u4 b[TL::WOB];
#pragma unroll
            for (int j = 0; j < TL::WOB; ++j) {
                const int o = (woi * TL::WOB + j) * 16 + i;
                b[j] = *(const u4*)(wb + o * 64 + 16 * (g ^ ((i >> 1) & 3)));
            }
            unsigned a[TL::WPB][4];
#pragma unroll
            for (int j = 0; j < TL::WPB; ++j) {
                const int pb = wpi * TL::WPB + j;
                const unsigned char* q =
                    buf + g * (4 * 1024 + 64) + pb_row(pb) * 128 + (pb_col(pb) * 16 + i) * 4;
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) a[j][s4] = *(const unsigned*)(q + s4 * 1024);
            }
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
                for (int jp = 0; jp < TL::WPB; ++jp)
#pragma unroll
                    for (int jo = 0; jo < TL::WOB; ++jo)
                        acc[jp][jo] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                            __uint_as_float(a[jp][s4]), __uint_as_float(b[jo][s4]), acc[jp][jo], 0, 0, 0);
        };
        // Chunk ch + 1 goes into the other buffer while chunk ch computes; one barrier per
        // chunk both publishes the landed chunk and retires the buffer read before it.
        stage(0, smem);
        for (int ch = 0; ch < nChunk; ++ch) {
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): this wave's DMA has landed
            __builtin_amdgcn_s_barrier();        // ... and every wave's; the other buffer is free
            asm volatile("" ::: "memory");
            if (ch + 1 < nChunk) stage(ch + 1, smem + ((ch + 1) & 1) * DL::BUF);
            compute(smem + (ch & 1) * DL::BUF);
        }
    } else if constexpr (DMA == 2) {
        typedef __attribute__((address_space(3))) void lds_t;
        using DL = GeoDmaK<TL>;
        constexpr int NW = DL::NW;
        constexpr int CK = Elem<false>::CK;
        const int wave_u = __builtin_amdgcn_readfirstlane(wave);
        unsigned char* const wbuf = smem + DL::HALO_BYTES;
        // Staged columns start at the 4-pixel run holding input column ow0 - P; the tile's
        // column j, tap kw reads staged column j + kw + mis.
        const int mis = ((-pad) % 4 + 4) % 4;
        const int ih0 = oh0 - pad, iwa = ow0 - pad - mis;
        // Lane l: halo row (row group) * 6 + l / 10, run l % 10. A run lies wholly inside or
        // outside the image (W % 4 == 0); rows and runs outside it, and channels past Cin, read zero.
        const int lr = lane / 10, lrun = lane - 10 * (lane / 10);
        const int lane_off = (lr * W + 4 * lrun) * 4;
        const bool lane_ok = lr < DL::RG && iwa + 4 * lrun >= 0 && iwa + 4 * lrun < W;
        const bool row_ok0 = lane_ok && lr < DL::HR && ih0 + lr >= 0 && ih0 + lr < H;
        const bool row_ok1 = lane_ok && DL::RG + lr < DL::HR && ih0 + DL::RG + lr >= 0 && ih0 + DL::RG + lr < H;
        const int w_lane = ((lane >> 2) * 4 + ((lane & 3) ^ ((lane >> 3) & 3))) * 16;
        auto stage_halo = [&](int ch) {
            const int c0 = ch * CK;
#pragma unroll
            for (int k = 0; k < DL::HALO_INS / NW; ++k) {
                const int ins = wave_u + NW * k;
                const int c = ins >> 1, rg = ins & 1;  // wave-uniform
                // unsigned, so that a channel past Cin (kOOB below) or a base row or column
                // before the image wraps instead of overflowing; in-image lanes get the
                // exact offset back
                const int ubase = (int)__builtin_amdgcn_readfirstlane(
                    (((unsigned)(c0 + c) * H + (unsigned)(ih0 + rg * DL::RG)) * W + (unsigned)iwa) * 4u);
                const bool in = c0 + c < Cin && (rg ? row_ok1 : row_ok0);
                const int off = in ? ubase + lane_off : kOOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    xr, (lds_t*)(smem + c * 2048 + ((c >> 2) & 3) * 64 + rg * 1024), 16, off, 0, 0, 0);
            }
        };
        // Weights of kernel row kh: instruction ins fills rows 16 ins .. 16 ins + 15 of [kw][BN]
        // (tap and first oc wave-uniform, BN a multiple of 16); lane l takes row 16 ins + l / 4
        // and 16-byte slot l % 4, which holds K group (l % 4) ^ ((l / 4 >> 1) & 3).
        auto stage_w = [&](int ch, int kh, unsigned char* wb) {
#pragma unroll
            for (int k = 0; k < DL::W_INS / NW; ++k) {
                const int ins = wave_u + NW * k;
                const int kw = (ins * 16) / TL::BN, o0 = (ins * 16) % TL::BN;
                const int ubase =
                    __builtin_amdgcn_readfirstlane((((ch * KS + kh) * KS + kw) * CoutPad + oc0 + o0) * 64);
                const int off = ins * 16 < DL::W_ROWS ? ubase + w_lane : kOOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_t*)(wb + ins * 1024), 16, off, 0, 0, 0);
            }
        };
        // The K taps of kernel row kh, in the register path's order (kw, channel group, pixel
        // block, oc block), so both paths round identically.
        auto compute_kh = [&](int kh, const unsigned char* wb) {
#pragma unroll
            for (int kw = 0; kw < KS; ++kw) {
                u4 b[TL::WOB];
#pragma unroll
                for (int j = 0; j < TL::WOB; ++j) {
                    const int o = (woi * TL::WOB + j) * 16 + i;
                    b[j] = *(const u4*)(wb + (kw * TL::BN + o) * 64 + 16 * (g ^ ((i >> 1) & 3)));
                }
                unsigned a[TL::WPB][4];
#pragma unroll
                for (int j = 0; j < TL::WPB; ++j) {
                    const int pb = wpi * TL::WPB + j;
                    const unsigned char* q = smem + g * (4 * 2048 + 64) + DL::row_off(pb_row(pb) + kh) +
                                             (pb_col(pb) * 16 + i + kw + mis) * 4;
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4) a[j][s4] = *(const unsigned*)(q + s4 * 2048);
                }
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
                    for (int jp = 0; jp < TL::WPB; ++jp)
#pragma unroll
                        for (int jo = 0; jo < TL::WOB; ++jo)
                            acc[jp][jo] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                __uint_as_float(a[jp][s4]), __uint_as_float(b[jo][s4]), acc[jp][jo], 0, 0, 0);
            }
        };
        for (int ch = 0; ch < nChunk; ++ch) {
            if (ch) {  // every wave is done reading the previous chunk's halo and weights
                asm volatile("" ::: "memory");
                __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
            }
            stage_halo(ch);
            stage_w(ch, 0, wbuf);
#pragma unroll
            for (int kh = 0; kh < KS; ++kh) {
                // the halo and row kh's weights have landed (this wave's, then every wave's),
                // and no wave still reads the other weight buffer (row kh - 1)
                asm volatile("" ::: "memory");
                __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
                if (kh + 1 < KS) stage_w(ch, kh + 1, wbuf + ((kh + 1) & 1) * DL::WBUF);
                compute_kh(kh, wbuf + (kh & 1) * DL::WBUF);
            }
        }
    } else {
        // Steps (chunk c, kernel row kh), kh fastest; the next step's loads fly while this
        // step computes.
        const int nStep = nChunk * KS;
        using Halo = typename std::conditional<VEC, GeoHaloVec<BF16, TL>, GeoHalo<BF16, TL>>::type;
        Halo hs;
        GeoWeights<BF16, TL> wsg;
        constexpr int CK = Elem<BF16>::CK;
        constexpr int VW = 16 / (int)sizeof(T);
        const int mis = ((-pad) % VW + VW) % VW;  // iw0 - mis is a multiple of VW
        const int hcol0 = VEC ? iw0 - mis : iw0;
        auto halo_store = [&]() {
            if constexpr (VEC) hs.store(halo, mis, tid);
            else hs.store(halo, tid);
        };
        hs.setup(H, W, hcol0, tid);
        const bool last_used = Halo::last_used(tid);
        hs.load(xr, H, W, Cin, 0, oh0 * S - pad, hcol0, tid);
        wsg.load(wr, CoutPad, 0, oc0, tid);
        // The next step's loads are spread between this step's MFMAs instead of issued as one
        // burst: the texture unit takes a 16-byte-per-lane load every ~16 cycles, so a burst from
        // every wave stalled each wave ~1.5-2.3 k cycles in issue before its first MFMA.
        constexpr int kMfmaPerStep = KS * TL::WPB * TL::WOB * (BF16 ? 1 : 4);
        constexpr int kLoadsPerStep = Halo::PER * Elem<BF16>::EPG + GeoWeights<BF16, TL>::PER;
        constexpr int kMfmaPerLoad = kMfmaPerStep / kLoadsPerStep > 0 ? kMfmaPerStep / kLoadsPerStep : 1;
        // Only the 8-wave bf16 tile with 16-byte runs and K < 5: elsewhere it made the compiler spill.
        constexpr bool kInterleave = BF16 && VEC && TL::WO == 2 && KS < 5;
        for (int st = 0; st < nStep; ++st) {
            if (st) __syncthreads();  // every wave is done reading the previous step
            halo_store();
            wsg.store(wl, tid);
            __syncthreads();
            if constexpr (kInterleave) {
                if (st + 1 < nStep) {
                    const int c = (st + 1) / KS, kh = (st + 1) % KS;
                    // loads and MFMAs in one basic block, so the scheduler can interleave them; a
                    // wave with no halo item in its last round leaves those loads out
                    auto load_and_compute = [&](auto with_last) {
                        hs.template load<decltype(with_last)::value>(xr, H, W, Cin, c * CK, oh0 * S + kh - pad, hcol0,
                                                                     tid);
                        wsg.load(wr, CoutPad, (c * KS + kh) * KS, oc0, tid);
                        compute_step();
#pragma unroll
                        for (int k = 0; k < kLoadsPerStep; ++k) {
                            __builtin_amdgcn_sched_group_barrier(0x008, kMfmaPerLoad, 0);  // MFMA
                            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);             // VMEM read
                        }
                    };
                    if (last_used) load_and_compute(std::true_type{});
                    else load_and_compute(std::false_type{});
                } else {
                    compute_step();
                }
            } else {
                if (st + 1 < nStep) {
                    const int c = (st + 1) / KS, kh = (st + 1) % KS;
                    hs.load(xr, H, W, Cin, c * CK, oh0 * S + kh - pad, hcol0, tid);
                    wsg.load(wr, CoutPad, (c * KS + kh) * KS, oc0, tid);
                }
                compute_step();
            }
        }

    }

    // Epilogue. Lane (g, i) register r holds pixel 4g + r of the pixel block and output
    // channel i of the oc block.
    const bool interior = oh0 + TL::TH <= OH && ow0 + TL::TW <= OW;  // uniform per workgroup
    if constexpr (POOL) {
        float psum[TL::WOB];
#pragma unroll
        for (int j = 0; j < TL::WOB; ++j) psum[j] = 0.0f;
        if (interior) {  // every pixel of the tile is an output: no masking
#pragma unroll
            for (int jp = 0; jp < TL::WPB; ++jp)
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int jo = 0; jo < TL::WOB; ++jo) psum[jo] += activate<ACT>(acc[jp][jo][r]);
        } else {
#pragma unroll
            for (int jp = 0; jp < TL::WPB; ++jp) {
                const int pb = wpi * TL::WPB + jp;
                const int oh = oh0 + pb_row(pb);
                const int owb = ow0 + pb_col(pb) * 16 + 4 * g;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool valid = oh < OH && owb + r < OW;
#pragma unroll
                    for (int jo = 0; jo < TL::WOB; ++jo) {
                        const float v = activate<ACT>(acc[jp][jo][r]);
                        psum[jo] += valid ? v : 0.0f;
                    }
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
            for (int jo = 0; jo < TL::WOB; ++jo) red[wpi * TL::BN + (woi * TL::WOB + jo) * 16 + i] = psum[jo];
        }
        __syncthreads();
        const int nTiles = tilesH * tilesW;
        if (tid < TL::BN) {
            float s = 0.0f;
#pragma unroll
            for (int p = 0; p < TL::WP; ++p) s += red[p * TL::BN + tid];
            const int oc = oc0 + tid;
            if (oc < Cout) dst[((long long)n * nTiles + th * tilesW + tw) * Cout + oc] = s;
        }
    } else {
        // A wave's blocks are rows oh_w + jp of one block column, so every store address is
        // the lane's base plus uniform strides (OW per block row, 16 OH OW per oc block).
        const int oh_w = oh0 + pb_row(wpi * TL::WPB);
        const int owb = ow0 + pb_col(wpi * TL::WPB) * 16 + 4 * g;
        const int oc_w = oc0 + woi * TL::WOB * 16 + i;
        float* const obase = dst + (((long long)n * Cout + oc_w) * OH + oh_w) * OW + owb;
        const long long oc_stride = 16LL * OH * OW;
#pragma unroll
        for (int jp = 0; jp < TL::WPB; ++jp) {
            if (oh_w + jp >= OH) continue;
#pragma unroll
            for (int jo = 0; jo < TL::WOB; ++jo) {
                if (oc_w + jo * 16 >= Cout) continue;
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = activate<ACT>(acc[jp][jo][r]);
                float* o = obase + jo * oc_stride + (long long)jp * OW;
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

// DMA (1 or 2): the caller has checked that the layer is fp32 with 16-byte halo runs (W % 4 ==
// 0, x 16-byte aligned), stride 1, and for the 1x1 form no padding.
template <bool BF16, int ACT, bool POOL, class TL, int DMA = 0>
hipError_t launch_geo_typed(const ConvPlan& p, const void* x, const void* wpk, const float* b, float* dst,
                            hipStream_t stream) {
    using T = typename Elem<BF16>::T;
    // 16-byte halo runs need whole runs per row and an aligned base. bf16 at K = 5, S = 2
    // keeps the element-wise path: its run registers (two 8-run items) would not fit
    // beside the accumulators without spilling.
    constexpr bool kVecOK = !(BF16 && TL::KS == 5 && TL::S == 2);
    const bool vec = kVecOK && p.W % (16 / (int)sizeof(T)) == 0 && (uintptr_t)x % 16 == 0;
    auto kern = conv_general_fused<BF16, false, ACT, POOL, TL>;
    if constexpr (DMA != 0)
        kern = conv_general_fused<false, true, ACT, POOL, TL, DMA>;
    else if constexpr (kVecOK)
        if (vec) kern = conv_general_fused<BF16, true, ACT, POOL, TL>;
    hipLaunchKernelGGL(kern, dim3((unsigned)p.grid()), dim3(TL::NT), 0, stream,
                       (const T*)x, (const T*)wpk, b, dst, p.Cin, p.H, p.W, p.Cout, p.OH, p.OW, p.pad, p.CoutPad,
                       p.nChunk, p.tilesH, p.tilesW, p.ocTiles,
                       ((uintptr_t)dst % 16 == 0) ? 16 : ((uintptr_t)dst % 8 == 0 ? 8 : 4));
    return hipGetLastError();
}

template <bool BF16, class TL, int DMA = 0>
hipError_t launch_geo_act(const ConvPlan& p, const void* x, const void* wpk, const float* b, float* dst,
                          hipStream_t stream) {
    switch (p.act * 2 + p.pool) {
        case 0: return launch_geo_typed<BF16, kActNone, false, TL, DMA>(p, x, wpk, b, dst, stream);
        case 1: return launch_geo_typed<BF16, kActNone, true, TL, DMA>(p, x, wpk, b, dst, stream);
        case 2: return launch_geo_typed<BF16, kActGelu, false, TL, DMA>(p, x, wpk, b, dst, stream);
        case 3: return launch_geo_typed<BF16, kActGelu, true, TL, DMA>(p, x, wpk, b, dst, stream);
        case 4: return launch_geo_typed<BF16, kActMish2, false, TL, DMA>(p, x, wpk, b, dst, stream);
        case 5: return launch_geo_typed<BF16, kActMish2, true, TL, DMA>(p, x, wpk, b, dst, stream);
        case 6: return launch_geo_typed<BF16, kActGeluTanh, false, TL, DMA>(p, x, wpk, b, dst, stream);
        case 7: return launch_geo_typed<BF16, kActGeluTanh, true, TL, DMA>(p, x, wpk, b, dst, stream);
        default: return hipErrorInvalidValue;
    }
}

template <class TL>
hipError_t launch_geo_dtype(const ConvPlan& p, const void* x, const void* wpk, const float* b, float* dst,
                            hipStream_t stream) {
    return p.bf16 ? launch_geo_act<true, TL>(p, x, wpk, b, dst, stream)
                  : launch_geo_act<false, TL>(p, x, wpk, b, dst, stream);
}

}  // namespace

// One kernel size per translation unit: BN 16, 32, 64 or 128 (the plan decides), stride 1 or 2,
// either dtype. Return hipErrorInvalidValue for a plan they do not cover.
hipError_t launch_geo_k1(const ConvPlan& p, const void* x, const void* wpk, const float* b, float* dst,
                         hipStream_t stream);
hipError_t launch_geo_k3(const ConvPlan& p, const void* x, const void* wpk, const float* b, float* dst,
                         hipStream_t stream);
hipError_t launch_geo_k5(const ConvPlan& p, const void* x, const void* wpk, const float* b, float* dst,
                         hipStream_t stream);

}  // namespace fconv
