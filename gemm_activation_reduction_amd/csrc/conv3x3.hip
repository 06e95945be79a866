// Fused 3x3 valid convolution + bias + activation (+ global average pool) for gfx950.
//
// The convolution is an implicit GEMM: rows = output pixels, columns = output
// channels, reduction index k = (input channel, tap). It is evaluated as nine
// shifted "tap GEMMs" over a halo tile held in LDS, on MFMA:
//   fp32:  v_mfma_f32_16x16x4_f32   (full fp32 products, fp32 accumulation)
//   bf16:  v_mfma_f32_16x16x32_bf16 (exact bf16 products, fp32 accumulation)
// The accumulators start at the bias and the activation runs on them in registers;
// with pooling, each workgroup reduces its pixels per output channel (wave64
// butterfly, then LDS across waves) and writes one partial per (n, oc, tile); a
// second kernel sums the partials in a fixed order, so the result is deterministic
// without atomics.
//
// bf16 with 256 or more output channels (and 16-byte halo loads) runs conv3x3_wide_bf16
// instead: 256 oc per workgroup, weights streamed per tap into LDS by DMA (see there); its
// PAD = 1 instantiation serves bf16 "same" 3x3 layers as well. fp32 layers with 16-byte halo
// runs stage each chunk by LDS DMA in NCHW order (DmaLayout) instead of through registers.
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
#include <type_traits>

#include "conv_common.h"
#include "device_math.h"
#include "internal.h"

namespace fconv {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kRow = 80;  // bytes per LDS row (64 data + 16 pad)


template <int TH_, int TW_, int BN_, int WP_, int WO_, int MINW_, int NT_>
struct Tile {
    static constexpr int TH = TH_, TW = TW_, BN = BN_, WP = WP_, WO = WO_;
    static constexpr int NT = NT_;              // threads per workgroup (NT / 64 waves)
    static constexpr int MINW = MINW_;          // waves per SIMD the register budget targets
    static constexpr int CB = TW / 16;          // 16-pixel blocks per tile row
    static constexpr int PB = TH * CB;          // pixel blocks per tile
    static constexpr int OB = BN / 16;          // oc blocks per tile
    static constexpr int WPB = PB / WP;         // pixel blocks per wave
    static constexpr int WOB = OB / WO;         // oc blocks per wave
    static constexpr int HR = TH + 2, HC = TW + 2;
    // Halo row pitch in positions: HP = 4 (mod 8) makes the staging stores of two
    // neighbouring halo rows land on disjoint LDS banks.
    static constexpr int HP = HC + ((4 - HC % 8) + 8) % 8, HPOS = HR * HP;
    static constexpr int LDS = HPOS * kRow + 9 * BN * kRow;
    static_assert(WP * WO == NT / 64, "one wave per (pixel group, oc group)");
    static_assert(PB % WP == 0 && OB % WO == 0, "even wave split");
    static_assert(TW % 16 == 0 && BN % 16 == 0, "MFMA block multiples");
};

// Tile configurations.
// fp32: 256 pixels x 64 oc; wave = 4 pixel blocks x 4 oc blocks; 2 workgroups per CU.
using TileA = Tile<8, 32, 64, 4, 1, 2, 256>;
// bf16: the same tile shape (measured on MI355X: a 256 x 128 tile with 8 waves and one
// workgroup per CU, or 32-oc tiles with 3 workgroups per CU, were both slower).
using TileB = Tile<8, 32, 64, 4, 1, 2, 256>;
// Layers with at most 16 or 32 output channels take a tile of that many channels (same
// pixels, same waves, one or two oc blocks per wave): a 64-channel tile would spend 4x or 2x
// the MFMA work, weight staging and latency per workgroup on padding channels.
using TileS16 = Tile<8, 32, 16, 4, 1, 2, 256>;
using TileS32 = Tile<8, 32, 32, 4, 1, 2, 256>;


// ---------------------------------------------------------------------------------
// Staging of one K chunk (CK input channels) into LDS, split into a global-load half
// (into registers, issued before the previous chunk's MFMA work so the memory latency
// overlaps it) and an LDS-store half. Trip counts are compile-time constants so all
// of a thread's loads are in flight together.
// ---------------------------------------------------------------------------------


// Halo tile, vector path (W a multiple of the 16-byte pixel group, 16-byte aligned x):
// each item loads one 16-byte run of VW pixels from each of the EPG channels of one
// channel group, then writes VW 16-byte LDS rows (one per pixel, channel-minor), i.e.
// a small register transpose. Halo columns beyond TW+2 are loaded but not stored.
template <bool BF16, class TL>
struct HaloVec {
    using T = typename Elem<BF16>::T;
    static constexpr int ESZ = (int)sizeof(T);
    static constexpr int EPG = Elem<BF16>::EPG;
    static constexpr int VW = 16 / ESZ;                      // pixels per 16-byte load
    static constexpr int NCG = (TL::HC + VW - 1) / VW;       // 16-byte column groups per row
    static constexpr int ITEMS = TL::HR * NCG * 4;           // (row, column group, channel group)
    static constexpr int PER = (ITEMS + TL::NT - 1) / TL::NT;
    u4 v[PER][EPG];

    // Item -> (channel group q, column group cg, halo row r). The LDS stores of a
    // wave are processed eight lanes at a time; each group of eight must cover eight
    // distinct 16-byte bank slots. fp32 (4-pixel runs): 4 channel groups x 2 adjacent
    // column groups. bf16 (8-pixel runs, where adjacent column groups share banks):
    // 4 channel groups x 2 adjacent rows, which the halo pitch HP = 4 (mod 8) separates.
    __device__ __forceinline__ static void item(int it, int& q, int& cg, int& r) {
        q = it & 3;
        if constexpr (!BF16) {
            cg = (it >> 2) % NCG;
            r = (it >> 2) / NCG;
        } else {
            static_assert(TL::HR % 2 == 0, "bf16 staging pairs halo rows");
            cg = (it >> 3) % NCG;
            r = 2 * ((it >> 3) / NCG) + ((it >> 2) & 1);
        }
    }

    // Per-thread part of the run addresses, fixed for the whole K loop: the byte offset of
    // the item's run at channel 0, or kOOB when its halo row or columns lie outside the
    // image (the tile's position does not change between chunks).
    unsigned lane_b[PER];

    __device__ __forceinline__ void setup(int H, int W, int oh0, int ow0, int tid) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int it = tid + j * TL::NT;
            int q, cg, r;
            item(it, q, cg, r);
            const int ih = oh0 + r, iw = ow0 + cg * VW;
            const bool inb = it < ITEMS && ih < H && iw < W;
            lane_b[j] = inb ? (unsigned)(((q * EPG) * H + ih) * W + iw) * ESZ : (unsigned)kOOB;
        }
    }

    // Chunk at channel c0: channel c of a run is lane_b + c * plane bytes. A run outside
    // the image stays at or past kOOB, and below 2^32 because the image is under 2^31
    // bytes; a channel past Cin (the last chunk only) takes kOOB.
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t xr, int H, int W, int Cin, int c0, int oh0,
                                         int ow0, int tid) {
        (void)oh0;
        (void)ow0;
        const unsigned plane_b = (unsigned)(H * W) * ESZ;
        const bool full = c0 + Elem<BF16>::CK <= Cin;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const unsigned b = lane_b[j] + (unsigned)c0 * plane_b;
            const int cb = c0 + ((tid + j * TL::NT) & 3) * EPG;
#pragma unroll
            for (int e = 0; e < EPG; ++e) {
                const unsigned off = (full || cb + e < Cin) ? b + e * plane_b : (unsigned)kOOB;
                v[j][e] = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)off, 0, 0);
            }
        }
    }

    __device__ __forceinline__ void store(unsigned char* halo, int tid) const {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int it = tid + j * TL::NT;
            if (ITEMS % TL::NT != 0 && it >= ITEMS) continue;
            int q, cg, r;
            item(it, q, cg, r);
#pragma unroll
            for (int p = 0; p < VW; ++p) {
                const int col = cg * VW + p;
                if (NCG * VW > TL::HP && col >= TL::HP) continue;
                u4 o;
                if constexpr (!BF16) {
                    o = u4{v[j][0][p], v[j][1][p], v[j][2][p], v[j][3][p]};
                } else {
                    // pixel p of channels 2k and 2k+1: one byte permute per output dword
                    const int dw = p >> 1;
                    const unsigned sel = (p & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        o[k] = __builtin_amdgcn_perm(v[j][2 * k + 1][dw], v[j][2 * k][dw], sel);
                }
                *(u4*)(halo + (r * TL::HP + col) * kRow + q * 16) = o;
            }
        }
    }
};

// Halo tile, general path (any W, any alignment of x): element loads, one (position,
// channel group) item at a time.
template <bool BF16, class TL>
struct HaloScalar {
    using T = typename Elem<BF16>::T;
    static constexpr int ESZ = (int)sizeof(T);
    static constexpr int EPG = Elem<BF16>::EPG;
    static constexpr int ITEMS = TL::HR * TL::HC * 4;
    static constexpr int PER = (ITEMS + TL::NT - 1) / TL::NT;
    u4 v[PER];

    __device__ __forceinline__ void setup(int, int, int, int, int) {}

    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t xr, int H, int W, int Cin, int c0, int oh0,
                                         int ow0, int tid) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int it = tid + j * TL::NT;
            const int q = it & 3, pos = it >> 2;
            const int ih = oh0 + pos / TL::HC, iw = ow0 + pos % TL::HC;
            const bool inb = it < ITEMS && ih < H && iw < W;
            const int base = ((c0 + q * EPG) * H + ih) * W + iw;
            unsigned h[EPG];
#pragma unroll
            for (int e = 0; e < EPG; ++e) {
                const int off = (inb && c0 + q * EPG + e < Cin) ? (base + e * H * W) * ESZ : kOOB;
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
            const int pos = it >> 2;
            if (ITEMS % TL::NT == 0 || it < ITEMS)
                *(u4*)(halo + ((pos / TL::HC) * TL::HP + pos % TL::HC) * kRow + (it & 3) * 16) = v[j];
        }
    }
};

// Weight slice of one chunk: 9 taps x BN output channels x 64 bytes, from the repacked
// [chunk][tap][CoutPad][CK] layout (16-byte loads, contiguous per tap).
template <bool BF16, class TL>
struct WeightStage {
    using T = typename Elem<BF16>::T;
    static constexpr int ITEMS = 9 * TL::BN * 4;   // (16 rows x 4 groups) per 64 items
    static constexpr int PER = (ITEMS + TL::NT - 1) / TL::NT;
    static_assert(ITEMS % 64 == 0, "BN multiple of 16");
    u4 v[PER];

    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t wr, int CoutPad, int ch, int oc0, int tid) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int it = tid + j * TL::NT;
            const int q = (it >> 4) & 3, row = (it & 15) + 16 * (it >> 6);
            const int o = row % TL::BN, tap = row / TL::BN;
            const int off = (((ch * 9 + tap) * CoutPad + oc0 + o) * 4 + q) * 16;
            v[j] = __builtin_amdgcn_raw_buffer_load_b128(wr, (ITEMS % TL::NT == 0 || it < ITEMS) ? off : kOOB, 0, 0);
        }
    }

    __device__ __forceinline__ void store(unsigned char* wl, int tid) const {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int it = tid + j * TL::NT;
            const int q = (it >> 4) & 3, row = (it & 15) + 16 * (it >> 6);
            if (ITEMS % TL::NT == 0 || it < ITEMS) *(u4*)(wl + row * kRow + q * 16) = v[j];
        }
    }
};


// fp32 layers with 16-byte halo runs (W % 4 == 0) stage each K chunk by LDS DMA
// (buffer_load ... lds) instead of through registers: fp32 MFMA and VALU work serialize on a
// SIMD, and the register path spends VALU instructions on load addresses, the halo transpose
// and LDS store addresses. The halo stays in NCHW order. Channel c occupies a 2 KB block at
// c * 2048 + ((c >> 2) & 3) * 64 bytes: rows 0-5 in its first kilobyte and rows 6-9 in its
// second, each row 10 slots of 16 bytes (40 pixels). One DMA instruction fills one such
// kilobyte in lane order, lane l taking row l / 10, run l % 10 (lanes past the rows read
// zero), so a lane's part of every load address is fixed and only the channel and the row
// group change per instruction (wave-uniform, scalar arithmetic). The 16 x 4 lanes of an
// fp32 fragment read (channel 4g + s for lane group g, 16 consecutive pixels) land on 64
// distinct banks: the skew puts the four groups 16 banks apart. The weights arrive as 64-byte
// rows (tap, oc) with K group s of row r in 16-byte slot s ^ ((r >> 1) & 3), the layout the
// LDS-DMA GEMM reads conflict-free.
template <class TL>
struct DmaLayout {
    static constexpr int RG = 6;                        // halo rows per DMA instruction
    static constexpr int HALO_INS = 16 * 2;             // (channel, row group) pairs
    static constexpr int HALO_BYTES = 16 * 2048 + 3 * 64 + 64;
    static constexpr int W_ROWS = 9 * TL::BN;
    static constexpr int W_INS = (W_ROWS / 16 + (TL::NT / 64) - 1) / (TL::NT / 64) * (TL::NT / 64);
    static constexpr int LDS = HALO_BYTES + W_INS * 1024;
    static_assert(TL::HR <= 2 * RG && TL::HC <= 40, "the halo fits two 6-row groups of 40 pixels");
    static_assert(HALO_INS % (TL::NT / 64) == 0, "whole DMA instructions per wave");
    static_assert(W_ROWS % 16 == 0, "whole 16-row weight blocks");
    // byte offset of halo row r (0 <= r < 12) inside a channel block
    __device__ __forceinline__ static int row_off(int r) { return r < RG ? r * 160 : 1024 + (r - RG) * 160; }
};

template <bool BF16, bool VEC, int ACT, bool POOL, class TL, int DMA = 0>
__global__ __launch_bounds__(TL::NT) __attribute__((amdgpu_waves_per_eu(TL::MINW))) void conv3x3_fused(
    const typename Elem<BF16>::T* __restrict__ x, const typename Elem<BF16>::T* __restrict__ wp,
    const float* __restrict__ bias, float* __restrict__ dst, int Cin, int H, int W, int Cout,
    int CoutPad, int nChunk, int tilesH, int tilesW, int ocTiles, int out_align) {
    using T = typename Elem<BF16>::T;
    constexpr int CK = Elem<BF16>::CK;
    static_assert(!DMA || (!BF16 && VEC), "DMA staging: fp32 with 16-byte halo runs");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[DMA ? DmaLayout<TL>::LDS : TL::LDS];
    unsigned char* halo = smem;
    unsigned char* wl = smem + (DMA ? DmaLayout<TL>::HALO_BYTES : TL::HPOS * kRow);

    int bid = xcd_contiguous_index(blockIdx.x, gridDim.x);
    const int ot = bid % ocTiles; bid /= ocTiles;
    const int tw = bid % tilesW; bid /= tilesW;
    const int th = bid % tilesH;
    const int n = bid / tilesH;
    const int OH = H - 2, OW = W - 2;
    const int oh0 = th * TL::TH, ow0 = tw * TL::TW, oc0 = ot * TL::BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, i = lane & 15;
    const int wpi = wave % TL::WP, woi = wave / TL::WP;
    // Pixel block pb -> (tile row, 16-column block). fp32 enumerates rows first, so a
    // wave's blocks are one column of rows and A fragments repeat across kh taps (fewer
    // LDS reads); bf16 uses 2 x 2 blocks, which needs fewer live registers.
    auto pb_row = [](int pb) { return BF16 ? pb / TL::CB : pb % TL::TH; };
    auto pb_col = [](int pb) { return BF16 ? pb % TL::CB : pb / TL::TH; };

    // The accumulators start at the bias: lane (g, i) holds output channel i of each oc
    // block in all four of its accumulator registers, so one value per oc block does, and
    // the epilogue saves an add per output (VALU work here is not hidden under the MFMAs).
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
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wp, (unsigned)(nChunk * 9 * CoutPad * 64));

    // Nine shifted tap GEMMs over the chunk held in LDS.
    // bf16 A fragments: the wave's blocks are 2 x 2 blocks from row wpi * WPB / CB, so each
    // fragment address is one per-lane base plus an immediate. (Written through the block
    // index wpi * WPB + j, the compiler kept a position per fragment in registers and
    // multiplied it out per tap: 1.8 % slower. fp32 keeps that form: there the compiler
    // already used one base per block, and the rewrite changed its register allocation
    // for the worse.)
    static_assert(TL::WPB % TL::CB == 0, "bf16: a wave's blocks are whole block rows");
    const unsigned char* a_base = halo + (wpi * (TL::WPB / TL::CB) * TL::HP + i) * kRow + g * 16;
    auto compute_chunk = [&]() {
    #pragma unroll
        for (int tap = 0; tap < 9; ++tap) {
            const int kh = tap / 3, kw = tap % 3;
            u4 a[TL::WPB], b[TL::WOB];
    #pragma unroll
            for (int j = 0; j < TL::WPB; ++j) {
                if constexpr (BF16) {
                    a[j] = *(const u4*)(a_base + ((j / TL::CB + kh) * TL::HP + (j % TL::CB) * 16 + kw) * kRow);
                } else if constexpr (DMA) {
                    // channel 4g + s of pixel (row + kh, col + i + kw), s = 0..3: channel block
                    // (4g + s) * 2048 + g * 64, then the row, then the pixel
                    const int pb = wpi * TL::WPB + j;
                    const unsigned char* q = halo + g * (4 * 2048 + 64) + DmaLayout<TL>::row_off(pb_row(pb) + kh) +
                                             (pb_col(pb) * 16 + i + kw) * 4;
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4) a[j][s4] = *(const unsigned*)(q + s4 * 2048);
                } else {
                    const int pb = wpi * TL::WPB + j;
                    const int pos = (pb_row(pb) + kh) * TL::HP + pb_col(pb) * 16 + i + kw;
                    a[j] = *(const u4*)(halo + pos * kRow + g * 16);
                }
            }
    #pragma unroll
            for (int j = 0; j < TL::WOB; ++j) {
                const int o = (woi * TL::WOB + j) * 16 + i;
                if constexpr (DMA)
                    b[j] = *(const u4*)(wl + (tap * TL::BN + o) * 64 + 16 * (g ^ ((i >> 1) & 3)));
                else
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
    };

    if constexpr (DMA) {
        typedef __attribute__((address_space(3))) void lds_t;
        using DL = DmaLayout<TL>;
        constexpr int NW = TL::NT / 64;
        const int wave_u = __builtin_amdgcn_readfirstlane(wave);
        // Halo. Lane l: halo row (row group) * 6 + l / 10, pixels ow0 + 4 (l % 10) .. + 3. The lane's
        // offset and its bounds test for each row group are computed once; the channel and row
        // group of an instruction are wave-uniform and go through scalar registers.
        const int lr = lane / 10, lrun = lane - 10 * (lane / 10);
        const int lane_off = (lr * W + 4 * lrun) * 4;
        const bool lane_ok = lr < DL::RG && ow0 + 4 * lrun < W;
        const bool row_ok0 = lane_ok && lr < TL::HR && oh0 + lr < H;
        const bool row_ok1 = lane_ok && DL::RG + lr < TL::HR && oh0 + DL::RG + lr < H;
        if constexpr (DMA == 1) {  // the only chunk: its halo and weights, then the MFMA work
#pragma unroll
            for (int k = 0; k < DL::HALO_INS / NW; ++k) {
                const int ins = wave_u + NW * k;
                const int c = ins >> 1, rg = ins & 1;  // wave-uniform
                // unsigned: a channel past Cin (kOOB below) may lie past 2^31 bytes
                const int ubase = (int)__builtin_amdgcn_readfirstlane((((unsigned)c * H + oh0 + rg * DL::RG) * W + ow0) * 4u);
                const bool in = c < Cin && (rg ? row_ok1 : row_ok0);
                const int off = in ? ubase + lane_off : kOOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_t*)(halo + c * 2048 + ((c >> 2) & 3) * 64 + rg * 1024), 16,
                                                         off, 0, 0, 0);
            }
            // Weights. Instruction ins fills rows 16 ins .. 16 ins + 15 of [tap][BN]: since BN is a
            // multiple of 16 the tap and the first oc are wave-uniform; lane l takes row 16 ins + l / 4
            // and 16-byte slot l % 4, which holds K group (l % 4) ^ ((l / 4 >> 1) & 3).
            const int w_lane = ((lane >> 2) * 4 + ((lane & 3) ^ ((lane >> 3) & 3))) * 16;
#pragma unroll
            for (int k = 0; k < DL::W_INS / NW; ++k) {
                const int ins = wave_u + NW * k;
                const int tap = (ins * 16) / TL::BN, o0 = (ins * 16) % TL::BN;  // wave-uniform
                const int ubase = __builtin_amdgcn_readfirstlane((tap * CoutPad + oc0 + o0) * 64);
                const int off = ins * 16 < DL::W_ROWS ? ubase + w_lane : kOOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_t*)(wl + ins * 1024), 16, off, 0, 0, 0);
            }
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): this wave's DMA has landed
            __builtin_amdgcn_s_barrier();        // ... and every wave's
            asm volatile("" ::: "memory");
            compute_chunk();
        } else {  // the same staging for chunk after chunk, in one LDS buffer
            // One chunk at a time: the co-resident workgroup's MFMA work covers this one's DMA
            // latency (the register path overlaps it inside the workgroup instead).
            const int w_lane = ((lane >> 2) * 4 + ((lane & 3) ^ ((lane >> 3) & 3))) * 16;
            for (int ch = 0; ch < nChunk; ++ch) {
                const int c0 = ch * CK;
                if (ch) {  // every wave is done reading the previous chunk
                    asm volatile("" ::: "memory");
                    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
                    __builtin_amdgcn_s_barrier();
                    asm volatile("" ::: "memory");
                }
#pragma unroll
                for (int k = 0; k < DL::HALO_INS / NW; ++k) {
                    const int ins = wave_u + NW * k;
                    const int c = ins >> 1, rg = ins & 1;
                    // unsigned: a channel past Cin (kOOB below) may lie past 2^31 bytes
                    const int ubase = (int)__builtin_amdgcn_readfirstlane(
                        (((unsigned)(c0 + c) * H + oh0 + rg * DL::RG) * W + ow0) * 4u);
                    const bool in = c0 + c < Cin && (rg ? row_ok1 : row_ok0);
                    const int off = in ? ubase + lane_off : kOOB;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        xr, (lds_t*)(halo + c * 2048 + ((c >> 2) & 3) * 64 + rg * 1024), 16, off, 0, 0, 0);
                }
#pragma unroll
                for (int k = 0; k < DL::W_INS / NW; ++k) {
                    const int ins = wave_u + NW * k;
                    const int tap = (ins * 16) / TL::BN, o0 = (ins * 16) % TL::BN;
                    const int ubase = __builtin_amdgcn_readfirstlane(((ch * 9 + tap) * CoutPad + oc0 + o0) * 64);
                    const int off = ins * 16 < DL::W_ROWS ? ubase + w_lane : kOOB;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_t*)(wl + ins * 1024), 16, off, 0, 0, 0);
                }
                asm volatile("" ::: "memory");
                __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
                compute_chunk();
            }
        }
    } else {
    using Halo = typename std::conditional<VEC, HaloVec<BF16, TL>, HaloScalar<BF16, TL>>::type;
    WeightStage<BF16, TL> wsg;
    // One chunk ahead: the next chunk's loads fly while this chunk computes.
    Halo hs;
    hs.setup(H, W, oh0, ow0, tid);
    hs.load(xr, H, W, Cin, 0, oh0, ow0, tid);
    wsg.load(wr, CoutPad, 0, oc0, tid);
    for (int ch = 0; ch < nChunk; ++ch) {
        if (ch) __syncthreads();  // every wave is done reading the previous chunk
        hs.store(halo, tid);
        wsg.store(wl, tid);
        __syncthreads();
        if (ch + 1 < nChunk) {
            hs.load(xr, H, W, Cin, (ch + 1) * CK, oh0, ow0, tid);
            wsg.load(wr, CoutPad, ch + 1, oc0, tid);
        }
        // bf16: while computing, this wave issues ahead of the co-resident workgroup's
        // staging and epilogue VALU work on the same SIMD (measured +2 %; fp32, whose
        // MFMAs are 8x longer, loses 2-3 % with it)
        if constexpr (BF16) __builtin_amdgcn_s_setprio(1);
        compute_chunk();
        if constexpr (BF16) __builtin_amdgcn_s_setprio(0);
    }
    }

    // Epilogue. Accumulator layout (16x16 MFMA output): lane (g, i) register r holds
    // pixel 4g + r of the pixel block and output channel i of the oc block.
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
            for (int jo = 0; jo < TL::WOB; ++jo)
                red[wpi * TL::BN + (woi * TL::WOB + jo) * 16 + i] = psum[jo];
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
        // Every store address is the lane's base plus uniform offsets: block jp sits
        // pb_row(pb) - pb_row(pb0) rows and pb_col(pb) - pb_col(pb0) column blocks from the
        // wave's first block pb0, and oc block jo 16 OH OW elements on.
        const int pb0 = wpi * TL::WPB;
        const int oc_w = oc0 + woi * TL::WOB * 16 + i;
        float* const obase = dst + (((long long)n * Cout + oc_w) * OH + oh0 + pb_row(pb0)) * OW + ow0 +
                             pb_col(pb0) * 16 + 4 * g;
        const long long oc_stride = 16LL * OH * OW;
#pragma unroll
        for (int jp = 0; jp < TL::WPB; ++jp) {
            const int pb = wpi * TL::WPB + jp;
            const int oh = oh0 + pb_row(pb);
            const int owb = ow0 + pb_col(pb) * 16 + 4 * g;
            if (oh >= OH) continue;
#pragma unroll
            for (int jo = 0; jo < TL::WOB; ++jo) {
                if (oc_w + jo * 16 >= Cout) continue;
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = activate<ACT>(acc[jp][jo][r]);
                float* o = obase + jo * oc_stride + (long long)(pb_row(pb) - pb_row(pb0)) * OW +
                           (pb_col(pb) - pb_col(pb0)) * 16;
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


// ---------------------------------------------------------------------------------
// bf16, all of 256 output channels per workgroup ("wide"). The input halo of a pixel tile
// is staged once for 256 channels instead of once per 64, and the weights stream tap by
// tap from HBM/L2 into a ring of LDS slots by LDS DMA (buffer_load_dwordx4 ... lds), so
// they take no registers, no LDS store instructions and no address arithmetic per chunk.
// Tile: 4 output rows x 32 columns x 256 oc; 4 waves, each 2 x 2 pixel blocks x 8 oc
// blocks (128 accumulator registers). A K step is one tap of one 32-channel chunk:
// 32 MFMAs per wave. LDS: the halo (6 rows x 40 positions of 64 bytes: 32 bf16 channels)
// and kWideSlots tap slots of 256 rows x 64 bytes. Both are read 16 rows x 4 16-byte groups
// per fragment, and both keep group s of row (or halo position) r in 16-byte slot
// s ^ f(r), f(r) = (r >> 1) & 3. Measured with SQ_LDS_BANK_CONFLICT on gfx950, that pattern
// reads without bank conflicts at every row offset the kernel uses. An unswizzled
// 80-byte-row halo, and the slot swizzle ((r >> 1) ^ (r >> 3)) & 3, each cost four conflict
// cycles per ds_read_b128. A wave's DMA fills 1 KB of a tap slot in lane order (16 rows x
// 4 slots). With a halo row of 40 positions (a multiple of 8), f of a position depends only
// on the lane and the tap column, so the A fragment reads take three per-lane bases (one
// per tap column) plus immediate offsets. The next chunk's halo also arrives by LDS DMA, into a raw
// staging area, and is transposed LDS to LDS at the chunk boundary. So every vector memory
// operation in the main loop is a DMA at a fixed place in program order, and the vmcnt waits
// below, which count them, hold whatever the compiler does with other loads. (Counting
// ordinary halo loads was not safe: the compiler may move a load from the read-only input
// across the barriers, which left the last DMA instruction of a step unwaited.)
// ---------------------------------------------------------------------------------
using TileW = Tile<4, 32, 256, 2, 2, 2, 256>;
constexpr int kWideSlots = 3;                  // tap slots: the DMA runs two taps ahead
constexpr int kWideSlot = TileW::BN * 64;      // bytes per tap slot
// Raw (NCHW-order) staging of the next chunk's halo, filled by LDS DMA: 16-byte runs of 8
// pixels for (channel, halo row, column group 0-3), then 4-byte runs for halo columns 32-33
// of each (channel, halo row), padded to one 256-lane block.
constexpr int kRawA = 12 * 1024;
constexpr int kRawB = 1024;
constexpr int kWHP = 40;                                    // halo positions per row (>= 34, multiple of 8)
constexpr int kWideHalo = TileW::HR * kWHP * 64;            // 6 rows x 40 positions x 64 bytes
constexpr int kWideLds = kWideSlots * kWideSlot + kWideHalo + kRawA + kRawB;
static_assert(TileW::HR == 6 && TileW::HC == 34 && Elem<true>::CK == 32, "raw halo staging covers 32 x 6 x 34");
static_assert(2 * (kWideLds + 1024) <= 160 * 1024, "two wide workgroups per CU");

// PAD = 1 is the zero-padded ("same") 3x3 layer: the halo starts one row and one column
// before the tile, so halo column 0 comes from a third set of 4-byte runs (input columns
// ow0 - 2, ow0 - 1), the 16-byte runs land one position to the right, and halo column 33
// is the first pixel of the 4-byte run at ow0 + 32. Rows and columns outside x read zero.
template <int ACT, bool POOL, int PAD = 0>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void conv3x3_wide_bf16(
    const unsigned short* __restrict__ x, const unsigned short* __restrict__ wp, const float* __restrict__ bias,
    float* __restrict__ dst, int Cin, int H, int W, int Cout, int CoutPad, int nChunk, int tilesH, int tilesW,
    int ocTiles, int out_align) {
    using TL = TileW;
    constexpr int CK = Elem<true>::CK;
    static_assert(TL::NT == 256 && TL::WPB == 4 && TL::WOB == 8 && TL::CB == 2, "wide tile shape");
    static_assert(PAD == 0 || PAD == 1, "valid or one-pixel zero padding");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kWideLds + PAD * 1024];
    unsigned char* ring = smem;
    unsigned char* halo = smem + kWideSlots * kWideSlot;
    unsigned char* raw = halo + kWideHalo;

    int bid = xcd_contiguous_index(blockIdx.x, gridDim.x);
    const int ot = bid % ocTiles; bid /= ocTiles;
    const int tw = bid % tilesW; bid /= tilesW;
    const int th = bid % tilesH;
    const int n = bid / tilesH;
    const int OH = H - 2 + 2 * PAD, OW = W - 2 + 2 * PAD;
    const int oh0 = th * TL::TH, ow0 = tw * TL::TW, oc0 = ot * TL::BN;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar DMA choices
    const int g = lane >> 4, i = lane & 15;
    const int wpi = wave % TL::WP, woi = wave / TL::WP;
    const int row0 = wpi * (TL::WPB / TL::CB);  // the wave's blocks: rows row0, row0 + 1, two block columns

    f4 acc[TL::WPB][TL::WOB];
#pragma unroll
    for (int c = 0; c < TL::WOB; ++c) {
        const int oc = oc0 + (woi * TL::WOB + c) * 16 + i;
        const float bv = oc < Cout ? bias[oc] : 0.0f;
#pragma unroll
        for (int a = 0; a < TL::WPB; ++a) acc[a][c] = f4{bv, bv, bv, bv};
    }

    const long long plane = (long long)H * W;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + (long long)n * Cin * plane, (unsigned)(Cin * plane * 2));
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wp, (unsigned)(nChunk * 9 * CoutPad * 64));

    // DMA of K step s (chunk s / 9, tap s % 9) into slot s % kWideSlots: 16 instructions of
    // 16 rows, 4 per wave. Lane l covers row l >> 2 of its block, physical slot l & 3, which
    // holds K group (l & 3) ^ f(l >> 2).
    const int dma_r = lane >> 2;
    const int dma_grp = (lane & 3) ^ ((dma_r >> 1) & 3);
    auto issue = [&](int s) {
        const int slot = s % kWideSlots;
        const int rowbase = s * CoutPad + oc0;  // [chunk][tap] row index: (chunk * 9 + tap) * CoutPad
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int ins = wave + 4 * q;
            typedef __attribute__((address_space(3))) void lds_t;
            lds_t* d = (lds_t*)(ring + slot * kWideSlot + ins * 1024);
            const int off = ((rowbase + ins * 16 + dma_r) * 4 + dma_grp) * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, d, 16, off, 0, 0, 0);
        }
    };
    // fragment offsets: A from the halo as in the narrow bf16 kernel, B from a tap slot
    // A: halo position p = (row0 + row) * kWHP + block * 16 + i + kw keeps its group g in slot
    // g ^ ((p >> 1) & 3) = g ^ (((i + kw) >> 1) & 3), since every other term of p is a
    // multiple of 8: one base per tap column kw
    const unsigned char* a_base[3];
#pragma unroll
    for (int kw = 0; kw < 3; ++kw)
        a_base[kw] = halo + (row0 * kWHP + i + kw) * 64 + 16 * (g ^ (((i + kw) >> 1) & 3));
    const int b_off = (woi * TL::WOB * 16 + i) * 64 + 16 * (g ^ ((i >> 1) & 3));

    // Halo DMA of the chunk starting at channel c0 into the raw staging area: 12 instructions
    // of 16-byte runs and 4 of 4-byte runs, 4 per wave (3 + 1). Raw 16-byte entry
    // e * 96 + (r * 4 + cg) * 4 + q holds channel c0 + 8q + e, halo row r, pixels 8cg..8cg+7;
    // 4-byte entry e * 24 + r * 4 + q holds its pixels 32-33. Channels, rows and 8-pixel groups
    // outside x read as zero (W is a multiple of 8, so a group is wholly in or out).
    auto halo_issue = [&](int c0) {
        typedef __attribute__((address_space(3))) void lds_t;
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const int ia = wave + 4 * k;
            const int ei = ia * 64 + lane;
            const int e = ei / 96, rem = ei % 96;
            const int q = rem & 3, cg = (rem >> 2) & 3, r = rem >> 4;
            if constexpr (PAD == 0) {
                const int ch = c0 + 8 * q + e, ih = oh0 + r, iw = ow0 + 8 * cg;
                const int off = (ch < Cin && ih < H && iw < W) ? ((ch * H + ih) * W + iw) * 2 : kOOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_t*)(raw + ia * 1024), 16, off, 0, 0, 0);
            } else {
                const int ch = c0 + 8 * q + e, ih = oh0 - 1 + r, iw = ow0 + 8 * cg;
                const int off = (ch < Cin && (unsigned)ih < (unsigned)H && iw < W) ? ((ch * H + ih) * W + iw) * 2 : kOOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_t*)(raw + ia * 1024), 16, off, 0, 0, 0);
            }
        }
        if constexpr (PAD == 0) {
            const int ei = wave * 64 + lane;  // 192 entries; lanes 192-255 pad
            const int e = ei / 24, rem = ei % 24;
            const int q = rem & 3, r = rem >> 2;
            const int ch = c0 + 8 * q + e, ih = oh0 + r, iw = ow0 + 32;
            const int off = (ei < 192 && ch < Cin && ih < H && iw < W) ? ((ch * H + ih) * W + iw) * 2 : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_t*)(raw + kRawA + wave * 256), 4, off, 0, 0, 0);
        } else {
            // the right 4-byte runs (ow0 + 32) and the left ones (ow0 - 2) of one entry share
            // its channel and row: one base, 68 bytes apart
            const int ei = wave * 64 + lane;  // 192 entries; lanes 192-255 pad
            const int e = ei / 24, rem = ei % 24;
            const int q = rem & 3, r = rem >> 2;
            const int ch = c0 + 8 * q + e, ih = oh0 - 1 + r;
            const bool in = ei < 192 && ch < Cin && (unsigned)ih < (unsigned)H;
            // unsigned: a channel past Cin or a row before x (both kOOB below) wraps harmlessly
            const int base = (int)(((unsigned)(ch * H + ih) * (unsigned)W + (unsigned)(ow0 + 32)) * 2u);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_t*)(raw + kRawA + wave * 256), 4,
                                                     in && ow0 + 32 < W ? base : kOOB, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_t*)(raw + kRawA + 1024 + wave * 256), 4,
                                                     in && ow0 > 0 ? base - 68 : kOOB, 0, 0, 0);
        }
    };
    constexpr int kHaloDma = 4 + PAD;  // halo DMA instructions per wave
    // Raw staging -> channel-minor halo positions (the layout the A fragments read): item
    // (channel group q, column group cg, halo row r) gathers its 8 channels' runs and writes
    // pixel p of them as one 16-byte group (a byte permute per output dword) to halo position
    // r * kWHP + 8 cg + p, slot q ^ f(position). Columns 34-39 receive zeros.
    auto halo_transpose = [&]() {
        int q, cg, r;
        HaloVec<true, TL>::item(tid, q, cg, r);
        if (tid < HaloVec<true, TL>::ITEMS) {
            u4 v[8];
            if (cg < 4) {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = *(const u4*)(raw + (e * 96 + (r * 4 + cg) * 4 + q) * 16);
            } else {
                // PAD: dword 1 holds the left run (its pixel 1 is halo column 0)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[e] = u4{*(const unsigned*)(raw + kRawA + (e * 24 + r * 4 + q) * 4),
                              PAD ? *(const unsigned*)(raw + kRawA + 1024 + (e * 24 + r * 4 + q) * 4) : 0u, 0u, 0u};
            }
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const int dw = p >> 1;
                const unsigned sel = (p & 1) ? 0x07060302u : 0x05040100u;
                u4 o;
#pragma unroll
                for (int k = 0; k < 4; ++k) o[k] = __builtin_amdgcn_perm(v[2 * k + 1][dw], v[2 * k][dw], sel);
                // PAD, 4-byte item: pixel 0 is halo column 33 and pixel 3 (the left run's second
                // pixel) column 0; the other six land in columns 34-39, which no fragment reads
                constexpr int kEdge[8] = {33, 34, 35, 0, 37, 38, 39, 36};
                const int col = (PAD && cg == 4) ? kEdge[p] : cg * 8 + p + PAD;
                const int pos = r * kWHP + col;
                *(u4*)(halo + pos * 64 + 16 * (q ^ ((pos >> 1) & 3))) = o;
            }
        }
    };
    static_assert(HaloVec<true, TL>::PER == 1 && HaloVec<true, TL>::NCG == 5 && 8 * 5 == kWHP,
                  "one transpose item per thread; five 8-pixel column groups fill a halo row");

    const int nsteps = nChunk * 9;
    halo_issue(0);
    issue(0);
    if (nsteps > 1) issue(1);
    // the halo and step 0 have landed for this wave (step 1's DMA may fly)
    asm volatile("" ::: "memory");
    if (nsteps > 1) __builtin_amdgcn_s_waitcnt(0x0074);  // vmcnt(4) lgkmcnt(0)
    else __builtin_amdgcn_s_waitcnt(0x0070);             // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    halo_transpose();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the halo stores are done
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    // One K chunk (9 tap steps). NEXT: a later chunk follows, so its halo DMA is sent in tap 0
    // and transposed after tap 8. Chunks before the last take NEXT = true and the last
    // NEXT = false, which keeps every wait below a compile-time count.
    auto chunk = [&](const int c, auto next_tag) {
        constexpr bool NEXT = decltype(next_tag)::value;
#pragma unroll
        for (int t = 0; t < 9; ++t) {
            const int s = c * 9 + t;
            // step s + 2 exists: always when a chunk follows; in the last chunk for taps 0-6
            const bool ahead = NEXT || t + 2 < 9;
            if (ahead) issue(s + 2);
            if (NEXT && t == 0) halo_issue((c + 1) * CK);
            const int kh = t / 3, kw = t % 3;
            const unsigned char* bslot = ring + (s % kWideSlots) * kWideSlot + b_off;
            u4 a[TL::WPB], b[TL::WOB];
#pragma unroll
            for (int j = 0; j < TL::WPB; ++j)
                a[j] = *(const u4*)(a_base[kw] + ((j / TL::CB + kh) * kWHP + (j % TL::CB) * 16) * 64);
#pragma unroll
            for (int j = 0; j < TL::WOB; ++j) b[j] = *(const u4*)(bslot + j * 16 * 64);
#pragma unroll
            for (int jp = 0; jp < TL::WPB; ++jp)
#pragma unroll
                for (int jo = 0; jo < TL::WOB; ++jo)
                    acc[jp][jo] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, a[jp]), __builtin_bit_cast(bf16x8, b[jo]), acc[jp][jo], 0, 0, 0);
            // Before the barrier: this wave's reads of this step are done (the next step's DMA
            // reuses the slot read here) and its DMA of step s + 1 has landed. Vector memory
            // operations complete in order; the DMA instructions sent after step s + 1's may stay
            // in flight: step s + 2's (4) and, in taps 0 and 1, the next chunk's halo (kHaloDma).
            // The halo has landed by the end of tap 2, long before its transpose after tap 8.
            const int after = (ahead ? 4 : 0) + ((NEXT && t <= 1) ? kHaloDma : 0);
            asm volatile("" ::: "memory");
            if (after == 9) __builtin_amdgcn_s_waitcnt(0x0079);       // vmcnt(9) lgkmcnt(0)
            else if (after == 8) __builtin_amdgcn_s_waitcnt(0x0078);  // vmcnt(8) lgkmcnt(0)
            else if (after == 5) __builtin_amdgcn_s_waitcnt(0x0075);  // vmcnt(5) lgkmcnt(0)
            else if (after == 4) __builtin_amdgcn_s_waitcnt(0x0074);  // vmcnt(4) lgkmcnt(0)
            else __builtin_amdgcn_s_waitcnt(0x0070);                  // vmcnt(0) lgkmcnt(0)
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
        if constexpr (NEXT) {
            halo_transpose();  // every wave is past the chunk's last tap: the halo is free
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the raw reads and halo stores are done
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
    };
    for (int c = 0; c + 1 < nChunk; ++c) chunk(c, std::true_type{});
    chunk(nChunk - 1, std::false_type{});

    // Epilogue (accumulator layout: lane (g, i) register r holds pixel 4g + r of the pixel
    // block and output channel i of the oc block).
    const bool interior = oh0 + TL::TH <= OH && ow0 + TL::TW <= OW;  // uniform per workgroup
    if constexpr (POOL) {
        float psum[TL::WOB];
#pragma unroll
        for (int j = 0; j < TL::WOB; ++j) psum[j] = 0.0f;
        if (interior) {
#pragma unroll
            for (int jp = 0; jp < TL::WPB; ++jp)
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int jo = 0; jo < TL::WOB; ++jo) psum[jo] += activate<ACT>(acc[jp][jo][r]);
        } else {
#pragma unroll
            for (int jp = 0; jp < TL::WPB; ++jp) {
                const int oh = oh0 + row0 + jp / TL::CB;
                const int owb = ow0 + (jp % TL::CB) * 16 + 4 * g;
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
        float* red = (float*)smem;  // the ring is free: the last step ended with a barrier
        if (g == 0) {
#pragma unroll
            for (int jo = 0; jo < TL::WOB; ++jo) red[wpi * TL::BN + (woi * TL::WOB + jo) * 16 + i] = psum[jo];
        }
        __syncthreads();
        const int nTiles = tilesH * tilesW;
        {
            float sum = 0.0f;
#pragma unroll
            for (int p = 0; p < TL::WP; ++p) sum += red[p * TL::BN + tid];
            const int oc = oc0 + tid;
            if (oc < Cout) dst[((long long)n * nTiles + th * tilesW + tw) * Cout + oc] = sum;
        }
    } else {
#pragma unroll
        for (int jp = 0; jp < TL::WPB; ++jp) {
            const int oh = oh0 + row0 + jp / TL::CB;
            const int owb = ow0 + (jp % TL::CB) * 16 + 4 * g;
            if (oh >= OH) continue;
#pragma unroll
            for (int jo = 0; jo < TL::WOB; ++jo) {
                const int oc = oc0 + (woi * TL::WOB + jo) * 16 + i;
                if (oc >= Cout) continue;
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = activate<ACT>(acc[jp][jo][r]);
                float* o = dst + (((long long)n * Cout + oc) * OH + oh) * OW + owb;
                if ((OW & 3) == 0 && out_align >= 16 && owb + 3 < OW) {
                    *(f4*)o = f4{v[0], v[1], v[2], v[3]};
                } else if ((OW & 1) == 0 && out_align >= 8) {
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


template <bool BF16, int ACT, bool POOL, class TL>
hipError_t launch_typed(const ConvPlan& p, const void* x, const void* wpk, const float* b,
                        float* dst, hipStream_t stream) {
    using T = typename Elem<BF16>::T;
    // Vector halo loads need whole 16-byte pixel groups per row and an aligned base.
    const int vw = 16 / (int)sizeof(T);
    const bool vec = p.W % vw == 0 && (uintptr_t)x % 16 == 0;
    auto kern = vec ? conv3x3_fused<BF16, true, ACT, POOL, TL> : conv3x3_fused<BF16, false, ACT, POOL, TL>;
    if constexpr (!BF16)
        if (vec) kern = p.nChunk == 1 ? conv3x3_fused<false, true, ACT, POOL, TL, 1> : conv3x3_fused<false, true, ACT, POOL, TL, 2>;
    hipLaunchKernelGGL(kern, dim3((unsigned)p.grid()), dim3(TL::NT), 0,
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
        case 6: return launch_typed<BF16, kActGeluTanh, false, TL>(p, x, wpk, b, dst, stream);
        case 7: return launch_typed<BF16, kActGeluTanh, true, TL>(p, x, wpk, b, dst, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int ACT, bool POOL>
hipError_t launch_wide_typed(const ConvPlan& p, const void* x, const void* wpk, const float* b, float* dst,
                             hipStream_t stream) {
    auto kern = p.pad ? conv3x3_wide_bf16<ACT, POOL, 1> : conv3x3_wide_bf16<ACT, POOL, 0>;
    hipLaunchKernelGGL(kern, dim3((unsigned)p.grid()), dim3(TileW::NT), 0, stream,
                       (const unsigned short*)x, (const unsigned short*)wpk, b, dst, p.Cin, p.H, p.W, p.Cout,
                       p.CoutPad, p.nChunk, p.tilesH, p.tilesW, p.ocTiles,
                       ((uintptr_t)dst % 16 == 0) ? 16 : ((uintptr_t)dst % 8 == 0 ? 8 : 4));
    return hipGetLastError();
}

hipError_t launch_wide(const ConvPlan& p, const void* x, const void* wpk, const float* b, float* dst,
                       hipStream_t stream) {
    switch (p.act * 2 + p.pool) {
        case 0: return launch_wide_typed<kActNone, false>(p, x, wpk, b, dst, stream);
        case 1: return launch_wide_typed<kActNone, true>(p, x, wpk, b, dst, stream);
        case 2: return launch_wide_typed<kActGelu, false>(p, x, wpk, b, dst, stream);
        case 3: return launch_wide_typed<kActGelu, true>(p, x, wpk, b, dst, stream);
        case 4: return launch_wide_typed<kActMish2, false>(p, x, wpk, b, dst, stream);
        case 5: return launch_wide_typed<kActMish2, true>(p, x, wpk, b, dst, stream);
        case 6: return launch_wide_typed<kActGeluTanh, false>(p, x, wpk, b, dst, stream);
        case 7: return launch_wide_typed<kActGeluTanh, true>(p, x, wpk, b, dst, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool conv3x3_same_wide(bool bf16, int W, int Cout, const void* x) {
    return bf16 && W % 8 == 0 && (uintptr_t)x % 16 == 0 && Cout >= TileW::BN;
}

ConvPlan plan_conv(bool bf16, int act, int pool, int N, int Cin, int H, int W, int Cout, const void* x, int pad) {
    ConvPlan p{};
    p.bf16 = bf16; p.act = act; p.pool = pool;
    p.N = N; p.Cin = Cin; p.H = H; p.W = W; p.Cout = Cout;
    p.OH = H - 2 + 2 * pad; p.OW = W - 2 + 2 * pad;
    p.KS = 3; p.stride = 1; p.pad = pad; p.general = false;
    // bf16 with 256 or more output channels and 16-byte halo loads: the wide kernel
    const bool vec = W % 8 == 0 && (uintptr_t)x % 16 == 0;
    p.wide = bf16 && vec && Cout >= TileW::BN;
    p.TH = p.wide ? TileW::TH : bf16 ? TileB::TH : TileA::TH;
    p.TW = p.wide ? TileW::TW : bf16 ? TileB::TW : TileA::TW;
    p.BN = p.wide ? TileW::BN : Cout <= TileS16::BN ? TileS16::BN : Cout <= TileS32::BN ? TileS32::BN
                                                                 : bf16 ? TileB::BN : TileA::BN;
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
    if (p.pad != 0 && !p.wide) return hipErrorInvalidValue;  // only the wide kernel pads
    unsigned char* ws = (unsigned char*)workspace;
    void* wpk = ws;
    float* part = (float*)(ws + p.wpack_bytes);
    const long long total = (long long)p.nChunk * 9 * p.CoutPad * p.CK;
    const unsigned pblocks = (unsigned)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
    if (timer) timer->begin("pack_weights", stream);
    if (p.bf16)
        hipLaunchKernelGGL(pack_weights<true>, dim3(pblocks), dim3(256), 0, stream,
                           (const unsigned short*)w, (unsigned short*)wpk, p.Cin, p.Cout, p.CoutPad, 9, total);
    else
        hipLaunchKernelGGL(pack_weights<false>, dim3(pblocks), dim3(256), 0, stream, (const float*)w,
                           (float*)wpk, p.Cin, p.Cout, p.CoutPad, 9, total);
    hipError_t e = hipGetLastError();
    if (timer) timer->end("pack_weights", stream);
    if (e != hipSuccess) return e;
    float* dst = p.pool ? part : out;
    const char* kname = p.wide ? "conv3x3_wide_bf16" : "conv3x3_fused";
    if (timer) timer->begin(kname, stream);
    if (p.wide)
        e = launch_wide(p, x, wpk, b, dst, stream);
    else if (p.BN == TileS16::BN)
        e = p.bf16 ? launch_act<true, TileS16>(p, x, wpk, b, dst, stream)
                   : launch_act<false, TileS16>(p, x, wpk, b, dst, stream);
    else if (p.BN == TileS32::BN)
        e = p.bf16 ? launch_act<true, TileS32>(p, x, wpk, b, dst, stream)
                   : launch_act<false, TileS32>(p, x, wpk, b, dst, stream);
    else
        e = p.bf16 ? launch_act<true, TileB>(p, x, wpk, b, dst, stream)
                   : launch_act<false, TileA>(p, x, wpk, b, dst, stream);
    if (timer) timer->end(kname, stream);
    if (e != hipSuccess || !p.pool) return e;
    if (timer) timer->begin("pool_finalize", stream);
    hipLaunchKernelGGL(pool_finalize, dim3((unsigned)p.N, (unsigned)((p.Cout + 63) / 64)), dim3(256), 0, stream,
                       (const float*)part, out, p.Cout, p.tilesH * p.tilesW, (float)((double)p.OH * (double)p.OW));
    e = hipGetLastError();
    if (timer) timer->end("pool_finalize", stream);
    return e;
}

}  // namespace fconv
