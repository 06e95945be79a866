// Fused GEMM + scale + clamp + row logsumexp + z*mish(z) for gfx950.
//
// Source: the Linear -> x2 -> x+x -> clamp -> logsumexp -> x*mish(x) model of the
// "Kimi-K2.6 l2_p22" POPCORNBENCH page. The page materializes the GEMM output and
// reduces it row by row; here the (M x N) product never leaves the chip:
//   kernel 1 (gemm_lse_partials): one workgroup per BM x BN output tile computes
//     the tile on MFMA (fp32: v_mfma_f32_16x16x4_f32; bf16: v_mfma_f32_16x16x32_bf16
//     with fp32 accumulation; LDS double-buffered over K),
//     applies bias, scale and clamp in registers and reduces each of its rows to a
//     (max, sum exp(c - max)) pair, written to part[m][tile_n];
//   kernel 2 (lse_merge_mish): one wave per row merges the pairs with the page's
//     online logsumexp rule, M = max m_t, S = sum s_t e^(m_t - M), in a fixed
//     order, then writes z * mish(z) with z = M + log S.
// Both operands are K-contiguous (x [M][K], w [N][K]); an LDS row holds BK elements of
// K (four 16-byte groups) plus one 16-byte group of padding, so the fragment reads (16
// rows x 4 groups per wave) and the staging stores (8 rows per 8 lanes) are conflict-free.
// Lane group g of a wave supplies the same K positions of both operands, so any order of
// K inside a 16-byte group is a valid MFMA operand order.
#include "device_math.h"
#include "internal.h"

namespace fconv {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <bool BF16>
struct GElem;
template <>
struct GElem<false> {
    using T = float;
    static constexpr int PER16 = 4;  // elements per 16-byte group
};
template <>
struct GElem<true> {
    using T = unsigned short;  // bfloat16 bit patterns
    static constexpr int PER16 = 8;
};

template <int BM_, int BN_, int WM_, int WN_, int BK_, int NT_, bool BF16_>
struct GTile {
    static constexpr bool BF16 = BF16_;
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int NT = NT_;             // threads per workgroup
    static constexpr int BK = BK_;             // K elements per LDS stage (4 or more 16-byte groups)
    static constexpr int KG = BK / GElem<BF16>::PER16;  // 16-byte K groups per row
    static constexpr int PITCH = KG + 1;       // 16-byte units per LDS row (one of padding)
    static constexpr int MB = BM / WM / 16;   // 16-row blocks per wave
    static constexpr int NB = BN / WN / 16;   // 16-col blocks per wave
    static constexpr int IA = BM * KG, IB = BN * KG;  // float4 items per stage
    static constexpr int LA = (IA + NT - 1) / NT;      // float4 loads per thread (A)
    static constexpr int LB = (IB + NT - 1) / NT;      // float4 loads per thread (B)
    static_assert(WM * WN == NT / 64, "one wave per (row group, column group)");
    static_assert(KG % 4 == 0, "whole MFMA K steps per stage");
};

// Tile order. The dispatcher deals workgroups to the eight XCDs round-robin (workgroup b
// runs on XCD b % 8), and each XCD has its own L2. When the tile count is a multiple of 8,
// workgroup b is renumbered to logical tile (b % 8) * (T / 8) + b / 8, so each XCD holds a
// contiguous run of T / 8 logical tiles; logical tiles are then walked in groups of
// kGroupM tile rows (column by column inside a group), so one XCD's run is a block of
// kGroupM x (T / 8 / kGroupM) tiles that shares kGroupM strips of x and the W strips of
// its columns in that XCD's L2.
constexpr int kGroupM = 4;

__device__ __forceinline__ void tile_coords(int b, int tilesM, int tilesN, int& tm, int& tn) {
    const int T = tilesM * tilesN, per = T >> 3;
    const int L = b < (per << 3) ? (b & 7) * per + (b >> 3) : b;
    const int span = kGroupM * tilesN, first = (L / span) * kGroupM;
    const int rows = min(kGroupM, tilesM - first), r = L - (L / span) * span;
    tm = first + r % rows;
    tn = r / rows;
}

// 256 x 192 tiles: 2048 x 6144 is exactly 256 tiles, one per CU; 8 waves of 64 x 96.
using GTileF = GTile<256, 192, 4, 2, 32, 512, false>;
using GTileH = GTile<256, 192, 4, 2, 64, 512, true>;
// LDS-DMA path: the same tile with 64-byte K stages (32 bf16 / 16 fp32 values), four
// stages in flight.
using GTileD = GTile<256, 192, 4, 2, 32, 512, true>;
using GTileDF = GTile<256, 192, 4, 2, 16, 512, false>;
constexpr int kDmaStages = 4;

// One 16-byte group of K elements of one row (PER16 elements from k on); out-of-range
// rows and elements read as zero.
template <bool BF16, bool VEC>
__device__ __forceinline__ f4 load16(const typename GElem<BF16>::T* __restrict__ base, int rows, int K, int row,
                                     int k) {
    constexpr int P = GElem<BF16>::PER16;
    if (row >= rows) return f4{0.f, 0.f, 0.f, 0.f};
    const auto* p = base + (long long)row * K + k;
    if constexpr (VEC) {
        if (k < K) return *(const f4*)p;  // K % P == 0: the group is all in or all out
        return f4{0.f, 0.f, 0.f, 0.f};
    } else if constexpr (!BF16) {
        f4 v;
        v.x = k < K ? p[0] : 0.f;
        v.y = k + 1 < K ? p[1] : 0.f;
        v.z = k + 2 < K ? p[2] : 0.f;
        v.w = k + 3 < K ? p[3] : 0.f;
        return v;
    } else {
        unsigned d[4];
#pragma unroll
        for (int e = 0; e < P / 2; ++e) {
            const unsigned lo = k + 2 * e < K ? p[2 * e] : 0u;
            const unsigned hi = k + 2 * e + 1 < K ? p[2 * e + 1] : 0u;
            d[e] = lo | (hi << 16);
        }
        return __builtin_bit_cast(f4, d);
    }
}

// Tile epilogue shared by both GEMM kernels. Lane (g, i) register r of acc[jm][jn] holds
// row rm0 + 16 jm + 4g + r, column rn0 + 16 jn + i of the tile. Applies bias, scale and
// clamp, reduces each row to (max, sum exp(c - max)) (16-lane butterflies, then the WN
// column slices through `red`, LDS the caller no longer needs) and writes part[m][tn].
template <class TL>
__device__ __forceinline__ void tile_epilogue(f4 (&acc)[TL::MB][TL::NB], float2* red, const float* __restrict__ bias,
                                              float2* __restrict__ part, int m0, int n0, int M, int N, int tn,
                                              int tilesN, float scale, float cmin, float cmax, int tid, int g, int i,
                                              int wn, int rm0, int rn0) {
    // Epilogue: lane (g, i) register r holds row rm0 + 16 jm + 4g + r, column rn0 + 16 jn + i.
    float bv[TL::NB];
    bool cv[TL::NB];
#pragma unroll
    for (int jn = 0; jn < TL::NB; ++jn) {
        const int n = n0 + rn0 + jn * 16 + i;
        cv[jn] = n < N;
        bv[jn] = cv[jn] ? bias[n] : 0.0f;
    }
    float rmax[TL::MB][4], rsum[TL::MB][4];
#pragma unroll
    for (int jm = 0; jm < TL::MB; ++jm) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float mx = -INFINITY;
#pragma unroll
            for (int jn = 0; jn < TL::NB; ++jn) {
                const float c = fminf(fmaxf(scale * (acc[jm][jn][r] + bv[jn]), cmin), cmax);
                acc[jm][jn][r] = c;
                mx = cv[jn] ? fmaxf(mx, c) : mx;
            }
#pragma unroll
            for (int off = 8; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
            float s = 0.0f;
#pragma unroll
            for (int jn = 0; jn < TL::NB; ++jn) s += cv[jn] ? fast_exp(acc[jm][jn][r] - mx) : 0.0f;
#pragma unroll
            for (int off = 8; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
            rmax[jm][r] = mx;
            rsum[jm][r] = s;
        }
    }
    // Merge the WN column slices of each row through LDS (the caller ended on a barrier).
    if (i == 0) {
#pragma unroll
        for (int jm = 0; jm < TL::MB; ++jm)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                red[wn * TL::BM + rm0 + jm * 16 + 4 * g + r] = make_float2(rmax[jm][r], rsum[jm][r]);
    }
    __syncthreads();
    if (tid < TL::BM && m0 + tid < M) {
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < TL::WN; ++w) mx = fmaxf(mx, red[w * TL::BM + tid].x);
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < TL::WN; ++w) {
            const float2 p = red[w * TL::BM + tid];
            s += p.y > 0.0f ? p.y * fast_exp(p.x - mx) : 0.0f;
        }
        part[(long long)(m0 + tid) * tilesN + tn] = make_float2(mx, s);
    }
}

template <class TL, bool VEC>
__global__ __launch_bounds__(TL::NT) void gemm_lse_partials(
    const typename GElem<TL::BF16>::T* __restrict__ X, const typename GElem<TL::BF16>::T* __restrict__ Wt,
    const float* __restrict__ bias, float2* __restrict__ part, int M, int K, int N, float scale, float cmin,
    float cmax, int tilesN) {
    constexpr int BK = TL::BK, kPitch = TL::PITCH, P16 = GElem<TL::BF16>::PER16;
    __shared__ f4 As[2][TL::BM * kPitch];
    __shared__ f4 Bs[2][TL::BN * kPitch];

    int tm, tn;
    tile_coords(blockIdx.x, (int)gridDim.x / tilesN, tilesN, tm, tn);
    const int m0 = tm * TL::BM, n0 = tn * TL::BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, i = lane & 15;
    const int wm = wave % TL::WM, wn = wave / TL::WM;
    const int rm0 = wm * TL::MB * 16, rn0 = wn * TL::NB * 16;

    f4 acc[TL::MB][TL::NB];
#pragma unroll
    for (int a = 0; a < TL::MB; ++a)
#pragma unroll
        for (int b = 0; b < TL::NB; ++b) acc[a][b] = f4{0.f, 0.f, 0.f, 0.f};

    f4 ra[TL::LA], rb[TL::LB];
    // Item it -> (row, 16-byte K group). With 8 or more groups a row's stage is whole
    // 128-byte lines: groups go fastest, so eight lanes read one line and store to eight
    // consecutive LDS slots. With 4 groups (64 bytes) each 16 * KG items are 16 rows x KG
    // groups with rows fastest, so eight consecutive lanes still hit distinct bank slots.
    auto row_of = [](int it) { return TL::KG >= 8 ? it / TL::KG : (it & 15) + 16 * (it / (16 * TL::KG)); };
    auto grp_of = [](int it) { return TL::KG >= 8 ? it % TL::KG : (it >> 4) % TL::KG; };
    auto gload = [&](int k0) {
#pragma unroll
        for (int j = 0; j < TL::LA; ++j) {
            const int it = tid + j * TL::NT;
            if (TL::IA % TL::NT == 0 || it < TL::IA)
                ra[j] = load16<TL::BF16, VEC>(X, M, K, m0 + row_of(it), k0 + grp_of(it) * P16);
        }
#pragma unroll
        for (int j = 0; j < TL::LB; ++j) {
            const int it = tid + j * TL::NT;
            if (TL::IB % TL::NT == 0 || it < TL::IB)
                rb[j] = load16<TL::BF16, VEC>(Wt, N, K, n0 + row_of(it), k0 + grp_of(it) * P16);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int j = 0; j < TL::LA; ++j) {
            const int it = tid + j * TL::NT;
            if (TL::IA % TL::NT == 0 || it < TL::IA) As[buf][row_of(it) * kPitch + grp_of(it)] = ra[j];
        }
#pragma unroll
        for (int j = 0; j < TL::LB; ++j) {
            const int it = tid + j * TL::NT;
            if (TL::IB % TL::NT == 0 || it < TL::IB) Bs[buf][row_of(it) * kPitch + grp_of(it)] = rb[j];
        }
    };

    const int nk = (K + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
        for (int kk = 0; kk < TL::KG / 4; ++kk) {
            // lane (g, i): 16-byte group 4 kk + g of row i of each 16-row block
            f4 a[TL::MB], b[TL::NB];
#pragma unroll
            for (int j = 0; j < TL::MB; ++j) a[j] = As[cur][(rm0 + j * 16 + i) * kPitch + kk * 4 + g];
#pragma unroll
            for (int j = 0; j < TL::NB; ++j) b[j] = Bs[cur][(rn0 + j * 16 + i) * kPitch + kk * 4 + g];
            if constexpr (TL::BF16) {
#pragma unroll
                for (int jm = 0; jm < TL::MB; ++jm)
#pragma unroll
                    for (int jn = 0; jn < TL::NB; ++jn)
                        acc[jm][jn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, a[jm]), __builtin_bit_cast(bf16x8, b[jn]), acc[jm][jn], 0, 0,
                            0);
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int jm = 0; jm < TL::MB; ++jm)
#pragma unroll
                        for (int jn = 0; jn < TL::NB; ++jn)
                            acc[jm][jn] =
                                __builtin_amdgcn_mfma_f32_16x16x4f32(a[jm][s], b[jn][s], acc[jm][jn], 0, 0, 0);
            }
        }
        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
    }

    tile_epilogue<TL>(acc, (float2*)&As[0][0], bias, part, m0, n0, M, N, tn, tilesN, scale, cmin, cmax, tid, g, i,
                      wn, rm0, rn0);
}

// LDS-DMA path (bf16 or fp32 operands): each K stage is 64 bytes (32 bf16 or 16 fp32
// values) of every tile row, loaded by buffer_load_dwordx4 ... lds straight into one of
// STAGES LDS buffers,
// STAGES-1 stages ahead of the MFMA work (no registers, no LDS store instructions). A
// wave's DMA instruction fills 1 KB of LDS in lane order: 16 rows x 4 slots. Rows carry
// no padding; instead slot s of a row whose index within its 16-row block is r holds
// K group s ^ f(r), f(r) = ((r >> 1) ^ (r >> 3)) & 3, which keeps the fragment reads
// (16 rows x 4 groups per wave) on distinct banks. Out-of-range rows and K groups read
// zero through the buffer resource. Taken when K is a whole even number of stages
// (bf16: K % 64 == 0, fp32: K % 32 == 0) and operands are under 2 GiB. A lane's
// 16-byte group feeds one bf16 16x16x32 MFMA or, element by element, four fp32
// 16x16x4 MFMAs (the reduction order within the stage is free).
// On gfx950 the VALU work of staging through registers (global loads, LDS stores,
// address arithmetic) does not overlap fp32 MFMA work, so the DMA path pays off for
// fp32 as well.
// Instruction order of one DMA step (READS fragment reads of the next stage, MFMAS of this
// one): two MFMAs, then one read, until the reads are issued, then the remaining MFMAs, so
// the reads go out early and their latency hides under the MFMA work (measured: 1-2 %
// faster than the compiler's own order, which issued them after most of the MFMAs).
template <int READS, int MFMAS>
__device__ __forceinline__ void dma_step_schedule() {
    static_assert(MFMAS >= 2 * READS, "two MFMAs per fragment read");
    // sched_group_barrier masks: 0x008 MFMA, 0x100 LDS read
#pragma unroll
    for (int r = 0; r < READS; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, MFMAS - 2 * READS, 0);
}

template <class TL, int STAGES>
__global__ __launch_bounds__(TL::NT) void gemm_lse_partials_dma(
    const typename GElem<TL::BF16>::T* __restrict__ X, const typename GElem<TL::BF16>::T* __restrict__ Wt,
    const float* __restrict__ bias, float2* __restrict__ part, int M, int K, int N, float scale, float cmin,
    float cmax, int tilesN) {
    static_assert(TL::KG == 4, "64-byte K stages");
    constexpr int ESZ = (int)sizeof(typename GElem<TL::BF16>::T), EPG = 16 / ESZ;  // bytes, values per group
    constexpr int BK = TL::BK, ROWS = TL::BM + TL::BN, SB = ROWS * 64;  // bytes per stage
    constexpr int NI = ROWS / 16, NW = TL::NT / 64;                       // DMA instructions per stage, waves
    static_assert(ROWS % 16 == 0 && TL::BM % 16 == 0, "whole 16-row DMA blocks");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[STAGES * SB + 1024];  // + junk DMA target

    int tm, tn;
    tile_coords(blockIdx.x, (int)gridDim.x / tilesN, tilesN, tm, tn);
    const int m0 = tm * TL::BM, n0 = tn * TL::BN;
    const int tid = threadIdx.x, lane = tid & 63;
    // The wave index is the same in every lane; readfirstlane makes that visible to the
    // compiler, so the per-wave DMA choices below are scalar branches and the buffer
    // resource stays in scalar registers.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, i = lane & 15;
    const int wm = wave % TL::WM, wn = wave / TL::WM;
    const int rm0 = wm * TL::MB * 16, rn0 = wn * TL::NB * 16;

    f4 acc[TL::MB][TL::NB];
#pragma unroll
    for (int a = 0; a < TL::MB; ++a)
#pragma unroll
        for (int b = 0; b < TL::NB; ++b) acc[a][b] = f4{0.f, 0.f, 0.f, 0.f};

    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void*)X, (short)0, M * K * ESZ, 0x00020000);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc((void*)Wt, (short)0, N * K * ESZ, 0x00020000);
    constexpr int kOOB = 0x7FFFFFF0;
    // DMA lane -> (row within the 16-row block, K group): physical slot lane & 3 holds
    // group (lane & 3) ^ f(lane >> 2).
    const int dma_r = lane >> 2;
    const int dma_grp = (lane & 3) ^ ((dma_r >> 1) & 3);
    // Every wave sends exactly IPW DMA instructions per stage, so the per-stage DMA code has no
    // branches and every wave's vmcnt counts are the same: instruction q of wave w fills
    // 16-row block w + NW q. The X blocks come first (BM / 16 = 2 NW of them: q = 0, 1, fixed
    // at compile time), then the W blocks; a block index past the last (wave w + NW q >= NI)
    // sends an out-of-range load into a junk kilobyte past the ring. K stages are whole
    // (K is a multiple of 2 BK on this path), so only the row needs a bound.
    constexpr int IPW = (NI + NW - 1) / NW;
    static_assert(TL::BM / 16 == 2 * NW && IPW == 4, "X blocks are instructions q = 0, 1; W blocks q = 2, 3");
    int dma_off[IPW];  // byte offset of this lane's first K group in its row, or kOOB past the operand
#pragma unroll
    for (int q = 0; q < IPW; ++q) {
        const int ins = wave + NW * q;
        const int row = ins * 16 + dma_r;
        if (q < 2) {
            const int r = m0 + row;
            dma_off[q] = r < M ? (r * K + EPG * dma_grp) * ESZ : kOOB;
        } else {
            const int r = n0 + row - TL::BM;
            dma_off[q] = (ins < NI && r < N) ? (r * K + EPG * dma_grp) * ESZ : kOOB;
        }
    }
    auto issue = [&](int buf, int k0) {
        typedef __attribute__((address_space(3))) void lds_t;
#pragma unroll
        for (int q = 0; q < IPW; ++q) {
            const int ins = wave + NW * q;  // wave-uniform
            lds_t* dst = (lds_t*)(lds + (ins < NI ? buf * SB + ins * 1024 : STAGES * SB));
            const int off = dma_off[q] == kOOB ? kOOB : dma_off[q] + k0 * ESZ;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(q < 2 ? xr : wr, dst, 16, off, 0, 0, 0);
        }
    };
    // this wave's DMA instructions per stage
    constexpr int per_stage = IPW;
    // fragment read offset of lane (g, i): group g of row i sits in slot g ^ f(i),
    // f(i) = (i >> 1) & 3, the pattern SQ_LDS_BANK_CONFLICT measured conflict-free for these
    // 16-row x 4-group ds_read_b128 reads on gfx950 (f = ((i >> 1) ^ (i >> 3)) & 3 cost four
    // conflict cycles per read: 22.6 % of the CU's cycles in the bf16 GEMM)
    const int frag_off = i * 64 + 16 * (g ^ ((i >> 1) & 3));

    // Waits until this wave's DMA of stage `st` has landed, allowing its DMA of the stages
    // issued after it (up to `last`) to stay in flight, then a bare barrier (not
    // __syncthreads, whose release fence would wait for every DMA in flight): afterwards
    // stage st is in LDS for every wave. s_waitcnt immediates (gfx9 encoding: vmcnt bits
    // [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]; a field at its maximum is not waited
    // on): vmcnt(n) only. Issued through the builtin so the compiler's own wait insertion
    // knows the counter drained.
    auto stage_ready = [&](int st, int last) {
        const int inflight = (last > st ? last - st : 0) * per_stage;
        __asm__ volatile("" ::: "memory");  // the LDS reads issued above stay above the wait
        // The fragment reads of the next stage are not waited for here: they stay in flight
        // across the barrier, and the compiler waits for each register at its first MFMA.
        // (Their buffer is next overwritten by the DMA issued two barriers later, after the
        // MFMAs that consumed them; measured 1.8 % faster for bf16 than waiting here.)
        if (inflight >= 8) __builtin_amdgcn_s_waitcnt(0x0F78);
        else if (inflight >= 6) __builtin_amdgcn_s_waitcnt(0x0F76);
        else if (inflight >= 4) __builtin_amdgcn_s_waitcnt(0x0F74);
        else if (inflight >= 3) __builtin_amdgcn_s_waitcnt(0x0F73);
        else __builtin_amdgcn_s_waitcnt(0x0F70);
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
    };
    // lane (g, i) fragment of stage st for 16-row block j of the A rows / B rows
    auto frag_a = [&](int st, int j) { return *(const f4*)(lds + (st % STAGES) * SB + (rm0 + j * 16) * 64 + frag_off); };
    auto frag_b = [&](int st, int j) {
        return *(const f4*)(lds + (st % STAGES) * SB + (TL::BM + rn0 + j * 16) * 64 + frag_off);
    };

    // Pipeline. Step kt: read stage kt+1's fragments (into the other register set), the
    // MFMA work of stage kt, the DMA of stage kt+STAGES-1 into the buffer stage kt-1 used,
    // then wait for stage kt+2 and the barrier. The LDS reads of the next stage overlap
    // this stage's MFMA work.
    const int nk = (K + BK - 1) / BK;
    const int lastIssued0 = (nk < STAGES - 1 ? nk : STAGES - 1) - 1;
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
        if (st < nk) issue(st, st * BK);
    f4 a0[TL::MB], b0[TL::NB], a1[TL::MB], b1[TL::NB];
    stage_ready(0, lastIssued0);
#pragma unroll
    for (int j = 0; j < TL::MB; ++j) a0[j] = frag_a(0, j);
#pragma unroll
    for (int j = 0; j < TL::NB; ++j) b0[j] = frag_b(0, j);
    stage_ready(1, lastIssued0);
#define FCONV_DMA_STEP(KT, AC, BC, AN, BN_)                                                                      \
    {                                                                                                            \
        const int kt_ = (KT);                                                                                    \
        /* the last step reads a stale ring slot it never uses: no branch around the reads */                    \
        _Pragma("unroll") for (int j = 0; j < TL::MB; ++j) AN[j] = frag_a(kt_ + 1, j);                           \
        _Pragma("unroll") for (int j = 0; j < TL::NB; ++j) BN_[j] = frag_b(kt_ + 1, j);                          \
        if constexpr (TL::BF16) {                                                                                \
            _Pragma("unroll") for (int jm = 0; jm < TL::MB; ++jm)                                                \
                _Pragma("unroll") for (int jn = 0; jn < TL::NB; ++jn)                                            \
                    acc[jm][jn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, AC[jm]),     \
                        __builtin_bit_cast(bf16x8, BC[jn]), acc[jm][jn], 0, 0, 0);                                \
        } else {                                                                                                 \
            _Pragma("unroll") for (int s_ = 0; s_ < 4; ++s_)                                                     \
                _Pragma("unroll") for (int jm = 0; jm < TL::MB; ++jm)                                            \
                    _Pragma("unroll") for (int jn = 0; jn < TL::NB; ++jn)                                        \
                        acc[jm][jn] = __builtin_amdgcn_mfma_f32_16x16x4f32(AC[jm][s_], BC[jn][s_], acc[jm][jn],  \
                            0, 0, 0);                                                                            \
        }                                                                                                        \
        dma_step_schedule<TL::MB + TL::NB, TL::MB * TL::NB * (TL::BF16 ? 1 : 4)>();                              \
        if (kt_ + STAGES - 1 < nk) issue((kt_ + STAGES - 1) % STAGES, (kt_ + STAGES - 1) * BK);                  \
        stage_ready(kt_ + 2, nk - 1 < kt_ + STAGES - 1 ? nk - 1 : kt_ + STAGES - 1);                            \
    }
    // Steady state (every step sends a DMA and waits for the stage two ahead with one stage in
    // flight behind it): the DMA goes first, then this stage's MFMA work with the next stage's
    // fragment reads, then a fixed vmcnt and the barrier -- no branches in the step. Stage
    // kt + STAGES - 1 goes into the buffer of stage kt - 1, whose fragments were read during
    // step kt - 2 and consumed by step kt - 1's MFMAs, before the last barrier.
#define FCONV_DMA_STEADY(KT, AC, BC, AN, BN_)                                                                    \
    {                                                                                                            \
        const int kt_ = (KT);                                                                                    \
        issue((kt_ + STAGES - 1) % STAGES, (kt_ + STAGES - 1) * BK);                                             \
        _Pragma("unroll") for (int j = 0; j < TL::MB; ++j) AN[j] = frag_a(kt_ + 1, j);                           \
        _Pragma("unroll") for (int j = 0; j < TL::NB; ++j) BN_[j] = frag_b(kt_ + 1, j);                          \
        if constexpr (TL::BF16) {                                                                                \
            _Pragma("unroll") for (int jm = 0; jm < TL::MB; ++jm)                                                \
                _Pragma("unroll") for (int jn = 0; jn < TL::NB; ++jn)                                            \
                    acc[jm][jn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, AC[jm]),     \
                        __builtin_bit_cast(bf16x8, BC[jn]), acc[jm][jn], 0, 0, 0);                                \
        } else {                                                                                                 \
            _Pragma("unroll") for (int s_ = 0; s_ < 4; ++s_)                                                     \
                _Pragma("unroll") for (int jm = 0; jm < TL::MB; ++jm)                                            \
                    _Pragma("unroll") for (int jn = 0; jn < TL::NB; ++jn)                                        \
                        acc[jm][jn] = __builtin_amdgcn_mfma_f32_16x16x4f32(AC[jm][s_], BC[jn][s_], acc[jm][jn],  \
                            0, 0, 0);                                                                            \
        }                                                                                                        \
        dma_step_schedule<TL::MB + TL::NB, TL::MB * TL::NB * (TL::BF16 ? 1 : 4)>();                              \
        __asm__ volatile("" ::: "memory");                                                                       \
        __builtin_amdgcn_s_waitcnt(0x0F70 | per_stage);  /* vmcnt(per_stage): stage kt + 2 landed */            \
        __builtin_amdgcn_s_barrier();                                                                            \
        __asm__ volatile("" ::: "memory");                                                                       \
    }
    static_assert(STAGES == 4, "steady-state waits count one stage in flight");
    int kt = 0;
    for (; kt + 2 * (STAGES - 1) <= nk; kt += 2) {  // both steps send a DMA (nk is even on this path)
        FCONV_DMA_STEADY(kt, a0, b0, a1, b1)
        FCONV_DMA_STEADY(kt + 1, a1, b1, a0, b0)
    }
    for (; kt < nk; kt += 2) {  // the last steps: fewer DMAs, shrinking waits
        FCONV_DMA_STEP(kt, a0, b0, a1, b1)
        FCONV_DMA_STEP(kt + 1, a1, b1, a0, b0)
    }
#undef FCONV_DMA_STEADY
#undef FCONV_DMA_STEP
    __syncthreads();  // every wave is done with the stage buffers (the epilogue reuses them)
    tile_epilogue<TL>(acc, (float2*)lds, bias, part, m0, n0, M, N, tn, tilesN, scale, cmin, cmax, tid, g, i, wn, rm0,
                      rn0);
}

// One wave per row: fixed-order online-logsumexp merge of the tile partials, then
// out = z * mish(z) with the overflow-free softplus max(z,0) + log1p(e^-|z|).
__global__ __launch_bounds__(256) void lse_merge_mish(const float2* __restrict__ part,
                                                      float* __restrict__ out, int M, int tilesN) {
    const int row = (int)(((long long)blockIdx.x * blockDim.x + threadIdx.x) >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= M) return;
    const float2* p = part + (long long)row * tilesN;
    float mx = -INFINITY;
    for (int t = lane; t < tilesN; t += 64) mx = fmaxf(mx, p[t].x);
    mx = wave_max(mx);
    float s = 0.0f;
    for (int t = lane; t < tilesN; t += 64) {
        const float2 q = p[t];
        s += q.y > 0.0f ? q.y * expf(q.x - mx) : 0.0f;
    }
    s = wave_sum(s);
    if (lane == 0) {
        const float z = mx + logf(s);
        const float sp = fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z)));
        out[row] = z * (z * tanhf(sp));
    }
}

template <class TL>
hipError_t launch_partials(const GemmPlan& p, const void* x, const void* w, const float* b, float scale, float cmin,
                           float cmax, float2* part, hipStream_t stream) {
    using T = typename GElem<TL::BF16>::T;
    const unsigned grid = (unsigned)(p.tilesM * p.tilesN);
    if (p.vec)
        hipLaunchKernelGGL((gemm_lse_partials<TL, true>), dim3(grid), dim3(TL::NT), 0, stream, (const T*)x,
                           (const T*)w, b, part, p.M, p.K, p.N, scale, cmin, cmax, p.tilesN);
    else
        hipLaunchKernelGGL((gemm_lse_partials<TL, false>), dim3(grid), dim3(TL::NT), 0, stream, (const T*)x,
                           (const T*)w, b, part, p.M, p.K, p.N, scale, cmin, cmax, p.tilesN);
    return hipGetLastError();
}

}  // namespace

GemmPlan plan_gemm(bool bf16, int M, int K, int N, const void* x, const void* w) {
    GemmPlan p{};
    p.M = M; p.K = K; p.N = N;
    p.bf16 = bf16;
    p.BM = bf16 ? GTileH::BM : GTileF::BM;
    p.BN = bf16 ? GTileH::BN : GTileF::BN;
    p.tilesM = (M + p.BM - 1) / p.BM;
    p.tilesN = (N + p.BN - 1) / p.BN;
    p.vec = (K % (bf16 ? 8 : 4) == 0) && (((size_t)x | (size_t)w) % 16 == 0);
    // LDS-DMA path: bf16, whole 16-byte K groups, each operand addressable with 31-bit
    // byte offsets (the buffer resource's out-of-range offset must lie past its end).
    const long long esz = bf16 ? 2 : 4;
    p.dma = p.vec && K % (bf16 ? 64 : 32) == 0 && (long long)M * K * esz < 0x7FFF0000LL &&
            (long long)N * K * esz < 0x7FFF0000LL;
    p.part_bytes = (size_t)M * p.tilesN * sizeof(float2);
    return p;
}

hipError_t launch_gemm_lse(const GemmPlan& p, const void* x, const void* w, const float* b, float scale,
                           float cmin, float cmax, float* out, void* workspace, hipStream_t stream,
                           KernelTimer* timer) {
    float2* part = (float2*)workspace;
    if (timer) timer->begin("gemm_lse_partials", stream);
    hipError_t e;
    if (p.dma && p.bf16) {
        hipLaunchKernelGGL((gemm_lse_partials_dma<GTileD, kDmaStages>), dim3((unsigned)(p.tilesM * p.tilesN)),
                           dim3(GTileD::NT), 0, stream, (const unsigned short*)x, (const unsigned short*)w, b, part,
                           p.M, p.K, p.N, scale, cmin, cmax, p.tilesN);
        e = hipGetLastError();
    } else if (p.dma) {
        hipLaunchKernelGGL((gemm_lse_partials_dma<GTileDF, kDmaStages>), dim3((unsigned)(p.tilesM * p.tilesN)),
                           dim3(GTileDF::NT), 0, stream, (const float*)x, (const float*)w, b, part, p.M, p.K, p.N,
                           scale, cmin, cmax, p.tilesN);
        e = hipGetLastError();
    } else {
        e = p.bf16 ? launch_partials<GTileH>(p, x, w, b, scale, cmin, cmax, part, stream)
                   : launch_partials<GTileF>(p, x, w, b, scale, cmin, cmax, part, stream);
    }
    if (timer) timer->end("gemm_lse_partials", stream);
    if (e != hipSuccess) return e;
    if (timer) timer->begin("lse_merge_mish", stream);
    hipLaunchKernelGGL(lse_merge_mish, dim3((unsigned)((p.M + 3) / 4)), dim3(256), 0, stream,
                       (const float2*)part, out, p.M, p.tilesN);
    e = hipGetLastError();
    if (timer) timer->end("lse_merge_mish", stream);
    return e;
}

}  // namespace fconv
