// mfma_pipe.hip -- grouped bf16 expert GEMMs on the matrix cores with a
// multi-stage global->LDS pipeline (groups of more than 8 rows; prefill).
//
// [P1] "GLM-5.2 multi-GPU: expert-parallel sharding + the resident-fit
// benchmark": per-expert expertSwiGLU; its lever table: one batched call over
// all picked experts.  [P5] "GLM-5.3-Flash and full GLM-5.3 on the native CUDA
// engine (tracker) #593": fused gate/up rows 2w wide; grouped experts on
// prompt rows.
//
// A block owns a BM x BN output tile of one group (256 x 256 with 8 waves for
// groups of more than 128 rows, the last tile partial; 128, 64 or 32 x 128
// with 4 waves for a group that one such tile covers) and walks K in steps of
// 64.  Tiles of A
// (the group's rows) and B (weight rows) go straight from global memory into
// LDS with global_load_lds_dwordx4 (16 bytes per lane, a wave filling 1 KiB =
// 8 rows of 128 bytes), S steps in flight.  In LDS a row's eight 16-byte
// chunks are XOR-swizzled by the row index so the MFMA operand reads of 16
// consecutive rows hit different banks.  16x16x32 bf16 MFMAs; gate/up tiles
// hold 64 gate and the matching 64 up columns so the SwiGLU epilogue stays in
// registers.  Blocks are persistent over (tile, column tile) items; with a
// column-tile count that is a multiple of 8 and a grid that is too, a weight
// column tile always runs on the same XCD, whose L2 then serves its re-reads
// by the group's other row tiles.
#include "common.h"

#include <type_traits>

namespace moe {

typedef __bf16 bf16x8_p __attribute__((ext_vector_type(8)));
typedef float f32x4_p __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_p __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) const bf16x8_p lds_bf16x8;

// BM x BN tiles.  256 x 256: 8 waves of 128 x 64 (fewer LDS operand bytes
// per MFMA than 64 x 64 wave tiles; LDS bandwidth bounds the 64 x 64 layout
// at full MFMA rate), two 64 KiB stages, one block per CU.  256 x 128 (when
// there are too few 256 x 256 items to fill the chip): 8 waves of 64 x 64,
// three stages.  128, 64, 32 x 128: 4 waves, two blocks per CU.
template <int BM, int BN_ = (BM == 256 ? 256 : 128)>
struct PipeCfg {
    static constexpr int BN = BN_;                                // columns per tile
    static constexpr int NW = BM == 256 ? 8 : 4;                  // waves per block
    static constexpr int WM = BM == 256 ? (BN == 256 ? 2 : 4) : (BM == 128 ? 2 : 1);  // waves along M
    static constexpr int WN = NW / WM;                            // waves along N
    static constexpr int MT = BM / WM / 16;                       // 16-row subtiles per wave
    static constexpr int NT = BN / WN / 16;                       // 16-column subtiles per wave
    static constexpr int S = BM == 256 ? (BN == 256 ? 2 : 3) : (BM == 128 ? 2 : (BM == 64 ? 3 : 4));  // stages
    static constexpr int ALoads = BM / 8;                         // A wave-loads per stage
    static constexpr int LA = ALoads / NW;                        // A loads per wave per stage
    static constexpr int LB = BN / 8 / NW;                        // B loads per wave per stage
    static constexpr int L = LA + LB;                             // all loads per wave per stage
    static constexpr int ATile = BM * kBK * 2;
    static constexpr int BTile = BN * kBK * 2;
    static constexpr int Stage = ATile + BTile;
    // 128 x 128: separate rings, A two slots deep and B (the weights, read
    // from HBM) three, so B is issued two steps ahead within 80 KiB
    static constexpr bool Split = BM == 128;
    static constexpr int SA = Split ? 2 : S;
    static constexpr int SB = Split ? 3 : S;
    static constexpr int Lds = Split ? SA * ATile + SB * BTile : S * Stage;
    static constexpr int PerCU = Lds <= 80 * 1024 ? 2 : 1;
    static constexpr int Threads = 64 * NW;
    static_assert(ALoads % NW == 0, "A loads per wave");
    // column tiles of a gate/up (width w: BN / 2 gate + BN / 2 up columns) or
    // down projection
    static __host__ __device__ int col_tiles(bool gateup, int w, int H) {
        return gateup ? (w + BN / 2 - 1) / (BN / 2) : H / BN;
    }
};

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xf) | (0x7 << 4) | (0xf << 8) | ((N >> 4) << 14));
}

// Walk of (tile, column tile) items for tile lists whose tiles mostly belong
// to different experts.  Workgroups are dealt to the 8 XCDs round-robin by
// index; here XCD x takes tiles x, x + 8, ... with all their column tiles, in
// tile-major order over its own blocks, so a tile's A rows are fetched into
// one XCD's L2 once and then served to every column tile from there (the
// weights, read once per item either way, are not shared across tiles).
struct XcdWalk {
    int x, l, g8, NT, ntiles, j;
    __device__ XcdWalk(int ntiles_, int NT_) : NT(NT_), ntiles(ntiles_) {
        x = blockIdx.x & 7;
        l = blockIdx.x >> 3;
        g8 = gridDim.x >> 3;
        j = l;
    }
    // next item of this block: false when its XCD has none left
    __device__ bool next(int* tile, int* nt) {
        const int t = x + 8 * (j / NT);
        if (t >= ntiles) return false;
        *tile = t;
        *nt = j % NT;
        j += g8;
        return true;
    }
};

template <bool GATEUP, int BM, int BN>
__device__ void pipe_tile(const ExpertArgs& a, lds_u8* smem, const Group& g, int m0, int nt) {
    using C = PipeCfg<BM, BN>;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int wm = wave / C::WN, wn = wave % C::WN;
    const bool shared = g.expert < 0;
    const int Ig = shared ? a.Is : a.I;
    const int H = a.H;
    const int K = GATEUP ? H : Ig;
    const int rows = min(BM, g.n - m0);
    const int KT = K / kBK;
    // The small tiles start their K walk at step nt mod KT and wrap around:
    // neighbouring column tiles, which run at the same time, then read
    // different 128-byte columns of their weight rows instead of all
    // starting at column 0 (bands 3.34 -> 3.27 ms).  Only the fp32 summation
    // order over K changes, the same on every call.
    const int rot = BM < 256 ? nt % KT : 0;

    // Load sources.  Load j of this wave fills tile rows 8 (wave + NW j) .. +7;
    // lane l writes physical chunk l % 8 of row 8 (wave + NW j) + l / 8, which
    // holds logical chunk (l % 8) ^ (row % 8).
    const uint16_t* asrc[C::LA];
    const uint16_t* bsrc[C::LB];
    const uint16_t* wbase = GATEUP ? (shared ? a.swgu : a.wgu + (size_t)g.expert * 2 * Ig * H)
                                   : (shared ? a.swd : a.wd + (size_t)g.expert * H * Ig);
#pragma unroll
    for (int j = 0; j < C::LA; ++j) {
        const int r = 8 * (wave + C::NW * j) + (lane >> 3);
        const int c = (lane & 7) ^ (r & 7);
        const int rr = r < rows ? r : 0;  // rows past the group reload row 0 (never stored)
        const uint16_t* arow;
        if (GATEUP) {
            const int tok = shared ? m0 + rr : a.perm[g.row0 + m0 + rr] / a.topk;
            arow = a.x + (size_t)tok * H;
        } else {
            arow = shared ? a.h_s + (size_t)(m0 + rr) * a.Is : a.h_r + (size_t)(g.row0 + m0 + rr) * a.I;
        }
        asrc[j] = arow + 8 * c;
    }
#pragma unroll
    for (int j = 0; j < C::LB; ++j) {
        const int r = 8 * (wave + C::NW * j) + (lane >> 3);
        const int c = (lane & 7) ^ (r & 7);
        int brow;
        if (GATEUP) {
            constexpr int hb = C::BN / 2;
            const int col = nt * hb + (r < hb ? r : r - hb);
            // columns past the width (I not a multiple of BN / 2) reload
            // column 0 and are never stored
            brow = (col < Ig ? col : 0) + (r < hb ? 0 : Ig);
        } else {
            brow = nt * C::BN + r;
        }
        bsrc[j] = wbase + (size_t)brow * K + 8 * c;
    }

    // A and B slots of step kt: one ring of [A | B] stages, or (Split) an A
    // ring followed by a B ring
    auto a_slot = [&](int kt) -> lds_u8* {
        return C::Split ? smem + (kt % C::SA) * C::ATile : smem + (kt % C::S) * C::Stage;
    };
    auto b_slot = [&](int kt) -> lds_u8* {
        return C::Split ? smem + C::SA * C::ATile + (kt % C::SB) * C::BTile
                        : smem + (kt % C::S) * C::Stage + C::ATile;
    };
    auto issue_a = [&](int kt) {
        lds_u8* st = a_slot(kt);
        const int k0 = (kt + rot < KT ? kt + rot : kt + rot - KT) * kBK;
#pragma unroll
        for (int j = 0; j < C::LA; ++j)
            __builtin_amdgcn_global_load_lds(asrc[j] + k0, st + (wave + C::NW * j) * 1024, 16, 0, 0);
    };
    // Weight tiles of the small-tile lists are read by one tile each: loaded
    // non-temporal (the `nt` cache-policy bit, 2), they do not displace the
    // A rows that the group's column tiles share (prefill -2.7%, bands
    // -7.7%).  The 256-row tiles' weight columns are shared by the row tiles
    // of a group through L2, so they load with the default policy.
    constexpr int kBPolicy = BM == 256 ? 0 : 2;
    auto issue_b = [&](int kt) {
        lds_u8* st = b_slot(kt);
        const int k0 = (kt + rot < KT ? kt + rot : kt + rot - KT) * kBK;
#pragma unroll
        for (int j = 0; j < C::LB; ++j)
            __builtin_amdgcn_global_load_lds(bsrc[j] + k0, st + (wave + C::NW * j) * 1024, 16, 0, kBPolicy);
    };
    auto issue = [&](int kt) {
        issue_a(kt);
        issue_b(kt);
    };

    f32x4_p acc[C::MT][C::NT];
#pragma unroll
    for (int i = 0; i < C::MT; ++i)
#pragma unroll
        for (int j = 0; j < C::NT; ++j) acc[i][j] = f32x4_p{0.f, 0.f, 0.f, 0.f};

    // Tile rows of this wave's operand subtiles (A: 16-row blocks; B: 16-row
    // blocks of weight rows; for gate/up the first half are gate columns and
    // the second half the matching up columns).
    int aoff[C::MT], ax[C::MT], boff[C::NT], bx[C::NT];
#pragma unroll
    for (int i = 0; i < C::MT; ++i) {
        const int r = wm * (BM / C::WM) + 16 * i + (lane & 15);
        aoff[i] = r * 128;
        ax[i] = r & 7;
    }
#pragma unroll
    for (int j = 0; j < C::NT; ++j) {
        int rb;
        if (GATEUP) {
            constexpr int half = C::NT / 2;
            rb = (j < half ? 0 : C::BN / 2) + wn * (C::BN / 2 / C::WN) + 16 * (j % half);
        } else {
            rb = wn * (C::BN / C::WN) + 16 * j;
        }
        rb += lane & 15;
        boff[j] = rb * 128;
        bx[j] = rb & 7;
    }

    // Plain s_barrier, not __syncthreads(): the latter's release fence would
    // wait for every load in flight and undo the pipeline.  LDS reads are
    // complete before the barrier because the MFMAs consumed them.
    __builtin_amdgcn_s_barrier();  // every wave is done with the previous tile's stages
    if (C::Split) {
        // issue order A_0, B_0, B_1, then per step kt: A_{kt+1}, B_{kt+2}
        if (KT > 0) issue(0);
        if (KT > 1) issue_b(1);
    } else {
#pragma unroll
        for (int s = 0; s < C::S - 1; ++s)
            if (s < KT) issue(s);
    }

    // The step loop, compiled twice: with every 16-row subtile of this wave
    // live (no branches: the compiler schedules the LDS reads among the
    // MFMAs) and with the per-subtile checks of a partial last tile.
    auto steps = [&](auto all_live) {
    for (int kt = 0; kt < KT; ++kt) {
        if (C::Split) {
            // loads return in issue order: A_kt and B_kt have landed once at
            // most the loads of B_{kt+1} (issued after A_kt) are in flight
            if (kt + 1 < KT)
                wait_vmcnt<C::LB>();
            else
                wait_vmcnt<0>();
        } else {
            // Stage kt is complete once at most (stages issued after it) x L
            // of this wave's loads are still in flight.
            const int after = min(C::S - 2, KT - 1 - kt);
            if (after >= 4)
                wait_vmcnt<4 * C::L>();
            else if (after == 3)
                wait_vmcnt<3 * C::L>();
            else if (after == 2)
                wait_vmcnt<2 * C::L>();
            else if (after == 1)
                wait_vmcnt<C::L>();
            else
                wait_vmcnt<0>();
        }
        __builtin_amdgcn_s_barrier();  // step kt visible to all waves; step kt-1's slots free
        if (C::Split) {
            if (kt + 1 < KT) issue_a(kt + 1);
            if (kt + 2 < KT) issue_b(kt + 2);
        } else if (kt + C::S - 1 < KT) {
            issue(kt + C::S - 1);
        }
        const lds_u8* sa = a_slot(kt);
        const lds_u8* sb = b_slot(kt);
        // 16-row subtiles wholly past the group's rows do no MFMA work
        // (wave-uniform: a partial last tile of a large group)
        bool live[C::MT];
#pragma unroll
        for (int i = 0; i < C::MT; ++i) live[i] = decltype(all_live)::value || wm * (BM / C::WM) + 16 * i < rows;
        // the operand reads of both halves of the step first, then their
        // MFMAs (one half at a time for the 128 x 64 wave tile: registers)
        if constexpr (decltype(all_live)::value && BM == 256) {
            // Every subtile live: the step's MFMAs in groups of two 16-row
            // subtiles x all column subtiles, each group's A fragments (and a
            // new 32-deep half's B fragments) read from LDS while the
            // previous group's MFMAs run (two register sets each).
            constexpr int KS = kBK / 32, NP = C::MT / 2, NG = KS * NP;
            bf16x8_p ga[2][2], gb[2][C::NT];
            auto read_a = [&](int g, bf16x8_p* dst) {
                const int q = (g / NP) * 4 + (lane >> 4);
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const int i = 2 * (g % NP) + m;
                    dst[m] = *(lds_bf16x8*)(sa + aoff[i] + ((q ^ ax[i]) << 4));
                }
            };
            auto read_b = [&](int h, bf16x8_p* dst) {
                const int q = h * 4 + (lane >> 4);
#pragma unroll
                for (int j = 0; j < C::NT; ++j) dst[j] = *(lds_bf16x8*)(sb + boff[j] + ((q ^ bx[j]) << 4));
            };
            read_b(0, gb[0]);
            read_a(0, ga[0]);
            // the scheduler keeps this order: each group's LDS reads ahead of
            // the previous group's MFMAs (sched_group_barrier masks: 0x100 LDS
            // reads, 0x8 MFMA)
            __builtin_amdgcn_sched_group_barrier(0x100, 2 + C::NT, 0);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                if (g + 1 < NG) {
                    read_a(g + 1, ga[(g + 1) & 1]);
                    if ((g + 1) % NP == 0) {
                        read_b((g + 1) / NP, gb[((g + 1) / NP) & 1]);
                        __builtin_amdgcn_sched_group_barrier(0x100, 2 + C::NT, 0);
                    } else {
                        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                    }
                }
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const int i = 2 * (g % NP) + m;
#pragma unroll
                    for (int j = 0; j < C::NT; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ga[g & 1][m], gb[(g / NP) & 1][j],
                                                                            acc[i][j], 0, 0, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x8, 2 * C::NT, 0);
            }
            continue;
        }
        constexpr int KH = C::MT + C::NT <= 8 ? 2 : 1;
#pragma unroll
        for (int k0 = 0; k0 < kBK / 32; k0 += KH) {
            bf16x8_p af[KH][C::MT], bfr[KH][C::NT];
#pragma unroll
            for (int kh = 0; kh < KH; ++kh) {
                const int q = (k0 + kh) * 4 + (lane >> 4);  // logical 16-byte chunk of the operand
#pragma unroll
                for (int i = 0; i < C::MT; ++i)
                    if (live[i]) af[kh][i] = *(lds_bf16x8*)(sa + aoff[i] + ((q ^ ax[i]) << 4));
#pragma unroll
                for (int j = 0; j < C::NT; ++j) bfr[kh][j] = *(lds_bf16x8*)(sb + boff[j] + ((q ^ bx[j]) << 4));
            }
#pragma unroll
            for (int kh = 0; kh < KH; ++kh)
#pragma unroll
                for (int i = 0; i < C::MT; ++i)
                    if (live[i]) {
#pragma unroll
                        for (int j = 0; j < C::NT; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[kh][i], bfr[kh][j], acc[i][j], 0,
                                                                                0, 0);
                    }
        }
    }
    };
    if (wm * (BM / C::WM) + 16 * (C::MT - 1) < rows)
        steps(std::true_type{});
    else
        steps(std::false_type{});

    // Epilogue.  Lane holds D[4 (lane >> 4) + v][lane & 15] of each 16x16 subtile.
    if (GATEUP) {
        constexpr int half = C::NT / 2;
        uint16_t* hout = shared ? a.h_s + (size_t)m0 * a.Is : a.h_r + (size_t)(g.row0 + m0) * a.I;
#pragma unroll
        for (int i = 0; i < C::MT; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = wm * (BM / C::WM) + 16 * i + 4 * (lane >> 4) + v;
                if (r >= rows) continue;
#pragma unroll
                for (int j = 0; j < half; ++j) {
                    const int c = nt * (C::BN / 2) + wn * (C::BN / 2 / C::WN) + 16 * j + (lane & 15);
                    if (c < Ig)
                        hout[(size_t)r * Ig + c] =
                            f32_to_bf16_bits(silu_mul(acc[i][j][v], acc[i][j + half][v]));
                }
            }
    } else {
        float* yout = shared ? a.y_s + (size_t)m0 * H : a.y_r + (size_t)(g.row0 + m0) * H;
#pragma unroll
        for (int i = 0; i < C::MT; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = wm * (BM / C::WM) + 16 * i + 4 * (lane >> 4) + v;
                if (r >= rows) continue;
#pragma unroll
                for (int j = 0; j < C::NT; ++j) {
                    const int c = nt * C::BN + wn * (C::BN / C::WN) + 16 * j + (lane & 15);
                    yout[(size_t)r * H + c] = acc[i][j][v];
                }
            }
    }
}

// The 256-row list.  A large group has several 256-row tiles: column tile nt
// of all of them runs on XCD nt mod 8 (NT and the grid are multiples of 8 at
// the usual widths), whose L2 then serves the shared weight rows.  Every tile
// gets the same number of column tiles (the larger of the routed and shared
// widths); items past a group's width are skipped.
template <bool GATEUP, int BM>
__global__ __launch_bounds__(PipeCfg<BM>::Threads) void expert_mfma_pipe_kernel(ExpertArgs a) {
    static_assert(BM == 256, "the 128-, 64- and 32-row lists run in expert_mfma_small_kernel");
    using C = PipeCfg<BM>;
    using CN = PipeCfg<BM, 128>;  // 256 x 128 items when 256 x 256 ones are too few
    constexpr int kLds = C::Lds > CN::Lds ? C::Lds : CN::Lds;
    __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[kLds];
    lds_u8* smem = (lds_u8*)smem_raw;
    const int ntiles = a.plan_counts[4];
    const int32_t* tl = a.mfma_list + 2 * (size_t)3 * a.mfma_cap;
    const bool narrow = (long long)ntiles * C::col_tiles(GATEUP, a.I > a.Is ? a.I : a.Is, a.H) < gridDim.x;
    const int NTr = narrow ? CN::col_tiles(GATEUP, a.I, a.H) : C::col_tiles(GATEUP, a.I, a.H);
    const int NTs = narrow ? CN::col_tiles(GATEUP, a.Is, a.H) : C::col_tiles(GATEUP, a.Is, a.H);
    const int NT = NTr > NTs ? NTr : NTs;
    const int total = ntiles * NT;
    // Items in rounds of g8 (the blocks of one XCD), round r on XCD r mod 8.
    // Within a group the items run column chunk by column chunk (kChunk
    // column tiles wide), all of the group's row tiles per chunk, so the
    // blocks of a round share a few A tiles and a few weight column tiles in
    // their XCD's L2.
    constexpr int kChunk = 4;
    const int g8 = gridDim.x >> 3, x = blockIdx.x & 7, l = blockIdx.x >> 3;
    for (int rd = x;; rd += 8) {
        const int item = rd * g8 + l;
        if (item >= total) break;
        // the group of the item: its tiles are consecutive in the list and
        // own items NT * first tile .. NT * (first tile + tiles) - 1
        const int t = item / NT;
        const Group g = a.groups[tl[2 * t]];
        const int tf = t - tl[2 * t + 1] / 256;
        const int R = (g.n + 255) / 256;
        const int j = item - tf * NT;
        const int cc = j / (R * kChunk);
        const int c0 = cc * kChunk;
        const int wd = NT - c0 < kChunk ? NT - c0 : kChunk;
        const int rem = j - cc * R * kChunk;
        const int tile = tf + rem / wd, nt = c0 + rem % wd;
        if (nt >= (g.expert < 0 ? NTs : NTr)) continue;
        if (a.fmt != 0 && g.expert >= 0) continue;  // 4-bit experts: expert_mfma_w4_kernel
        if (narrow)
            pipe_tile<GATEUP, BM, 128>(a, smem, g, tl[2 * tile + 1], nt);
        else
            pipe_tile<GATEUP, BM, C::BN>(a, smem, g, tl[2 * tile + 1], nt);
    }
}

template <bool GATEUP, int BM>
static void launch_pipe_bm(const ExpertArgs& a, int num_cu, hipStream_t st) {
    using C = PipeCfg<BM>;
    const int NT = PipeCfg<BM, 128>::col_tiles(GATEUP, a.I > a.Is ? a.I : a.Is, a.H);
    long long grid = (long long)num_cu * C::PerCU;
    const long long ub = (long long)a.mfma_cap * NT;
    if (ub < grid) grid = ub;
    grid = grid < 8 ? 8 : grid & ~7LL;  // the XCD walk deals blocks in groups of 8
    expert_mfma_pipe_kernel<GATEUP, BM><<<(int)grid, C::Threads, 0, st>>>(a);
}

// The 128-, 64- and 32-row lists in one launch: the same block shape (4
// waves, 128 columns, at most 80 KiB of LDS, two blocks per CU), walked as
// one list, so the launch has one tail instead of three.
constexpr int kSmallLds = PipeCfg<128>::Lds > PipeCfg<64>::Lds
                              ? (PipeCfg<128>::Lds > PipeCfg<32>::Lds ? PipeCfg<128>::Lds : PipeCfg<32>::Lds)
                              : (PipeCfg<64>::Lds > PipeCfg<32>::Lds ? PipeCfg<64>::Lds : PipeCfg<32>::Lds);

// It is the only caller of the 128-, 64- and 32-row tile functions (the
// host compilation pass rejects a second kernel calling a specialization of
// pipe_tile that another kernel already instantiated).
template <bool GATEUP>
__global__ __launch_bounds__(256) void expert_mfma_small_kernel(ExpertArgs a) {
    using C = PipeCfg<128>;  // column tiling (128 columns) is the same for all three
    __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[kSmallLds];
    lds_u8* smem = (lds_u8*)smem_raw;
    const int n128 = a.plan_counts[1], n64 = a.plan_counts[2], n32 = a.plan_counts[3];
    const int NTr = C::col_tiles(GATEUP, a.I, a.H);
    const int NTs = C::col_tiles(GATEUP, a.Is, a.H);
    const int NT = NTr > NTs ? NTr : NTs;
    XcdWalk w(n128 + n64 + n32, NT);
    int v, nt;
    while (w.next(&v, &nt)) {
        const int list = v < n128 ? 0 : (v < n128 + n64 ? 1 : 2);
        const int tile = v - (list == 0 ? 0 : (list == 1 ? n128 : n128 + n64));
        const int32_t* tl = a.mfma_list + 2 * (size_t)list * a.mfma_cap;
        const Group g = a.groups[tl[2 * tile]];
        if (nt >= (g.expert < 0 ? NTs : NTr)) continue;
        if (a.fmt != 0 && g.expert >= 0) continue;  // 4-bit experts: expert_mfma_w4_kernel
        if (list == 0)
            pipe_tile<GATEUP, 128, 128>(a, smem, g, tl[2 * tile + 1], nt);
        else if (list == 1)
            pipe_tile<GATEUP, 64, 128>(a, smem, g, tl[2 * tile + 1], nt);
        else
            pipe_tile<GATEUP, 32, 128>(a, smem, g, tl[2 * tile + 1], nt);
    }
}

template <bool GATEUP>
static void launch_small(const ExpertArgs& a, int num_cu, hipStream_t st) {
    const int NT = PipeCfg<128>::col_tiles(GATEUP, a.I > a.Is ? a.I : a.Is, a.H);
    long long grid = (long long)num_cu * 2;
    const long long ub = 3LL * a.mfma_cap * NT;
    if (ub < grid) grid = ub;
    grid = grid < 8 ? 8 : grid & ~7LL;  // the XCD walk deals blocks in groups of 8
    expert_mfma_small_kernel<GATEUP><<<(int)grid, 256, 0, st>>>(a);
}

void launch_mfma_pipe(const ExpertArgs& a, bool gateup, int num_cu, hipStream_t st) {
    if (gateup) {
        launch_pipe_bm<true, 256>(a, num_cu, st);
        launch_small<true>(a, num_cu, st);
    } else {
        launch_pipe_bm<false, 256>(a, num_cu, st);
        launch_small<false>(a, num_cu, st);
    }
}


// ---- 4-bit experts ---------------------------------------------------------
//
// Blocks of 4 waves for BM = 128, 64, 32 (a 256-row tile runs as two 128-row
// halves); wave w owns all BM rows and 32 columns (16 gate and the matching 16
// up columns, or 32 down columns), so no two waves expand the same weights.
// Per K step of 64 a stage holds the A rows (bf16, as above) and the weight
// codes (128 rows x 32 bytes), loaded straight into LDS; each row's per-group
// words (W4A16: scale and zero of the step's two 32-input groups; MLX affine:
// scale and bias of its 64-input group; NVFP4: the E4M3 scales of its four
// 16-input blocks) come in blocks of steps beside them.  A wave expands its
// own B operand in registers just before the MFMAs that use it.  W4A16:
// (1024 + q) as an fp16 pair per two codes (one AND and one OR), then
// v_fma_mix ((1024 + q) s - (1024 + z) s, exact in fp32: both products fit in
// 24 bits) and v_cvt_pk_bf16_f32 (round to nearest even) -- the bf16 weight
// RNE((q - z) s).  MLX affine and NVFP4: dequant8_affine, dequant8_nv below.

template <int BM>
struct W4Cfg {
    static constexpr int NW = 4;
    static constexpr int WN = 4;                         // waves along N (each 32 columns)
    static constexpr int MT = BM / 16;                   // 16-row subtiles per wave
    static constexpr int NT = 2;                         // 16-column subtiles per wave
    static constexpr int S = BM == 128 ? 3 : (BM == 64 ? 4 : 6);  // stages
    static constexpr int LA = BM / 32;                   // A loads per wave per stage
    static constexpr int L = LA + 2;                     // + codes + one scale/zero piece
    static constexpr int ATile = BM * kBK * 2;
    static constexpr int QOff = ATile;                   // 128 rows x 32 bytes of codes
    static constexpr int Stage = QOff + 4096;
    // The per-group words come in blocks of G steps, sized for the largest
    // format (W4A16: [scales | zeros] x 128 rows x G steps x 4 bytes, the
    // step's two groups), three blocks in LDS.
    static constexpr int G = BM == 128 ? 4 : 8;
    static constexpr int SZBlock = 1024 * G;
    static constexpr int SZOff = S * Stage;
    static constexpr int Lds = SZOff + 3 * SZBlock;
    static_assert(G > S - 2, "a block's buffer is refilled only after its last read");
    static constexpr int PerCU = Lds <= 80 * 1024 ? 2 : 1;
    static constexpr int Threads = 64 * NW;
};

typedef _Float16 f16x2_p __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_p __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    const bf16x2_p v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// (x & m) | k in one instruction (the compiler emits an AND and an OR: a
// VOP3 takes no literal, and only one scalar operand, so k sits in a VGPR).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t k) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(k));
    return r;
}

// Eight codes (one word, k = 0..7 in nibbles 0..7) -> eight bf16 weights.
__device__ __forceinline__ bf16x8_p dequant8(uint32_t c, float s, float n) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // fp16 pair (1024 + q_j, 1024 + q_{j+4})
        const f16x2_p h = __builtin_bit_cast(f16x2_p, and_or(c >> (4 * j), 0x000f000fu, 0x64006400u));
        v[j] = fmaf((float)h.x, s, n);
        v[j + 4] = fmaf((float)h.y, s, n);
    }
    const u32x4_p o = {pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]), pack2_bf16(v[4], v[5]),
                       pack2_bf16(v[6], v[7])};
    return __builtin_bit_cast(bf16x8_p, o);
}

// The per-group arrays of the 4-bit formats as the scale/zero blocks stage
// them.  Every lane of a piece load takes 4 bytes of one row: W4A16 one step
// (its two 32-input groups' bf16 scales, or zeros), MLX affine two steps (a
// bf16 scale, or bias, per 64-input group = per step), NVFP4 one step (its
// four 16-input groups' E4M3 scales).  A piece takes AL lanes (64, or 32 when
// the format's arrays are half as many bytes per block), so a block of G
// steps is always 4 G pieces, one per wave and step.
template <int FMT>
struct W4Fmt {
    static constexpr int NA = FMT == 3 ? 1 : 2;             // arrays (scales [, zeros / biases])
    static constexpr int BPS = FMT == 2 ? 2 : 4;            // bytes per row and step, per array
    static constexpr int SPL = 4 / BPS;                     // steps per 4-byte lane load
    static constexpr int AL = FMT == 1 ? 64 : 32;           // lanes per piece
    static constexpr int PB = 4 * AL;                       // bytes per piece
};

// MLX affine: eight codes (one word, k = 0..7 in nibbles 0..7) -> eight bf16
// weights RNE(RNE_f32(s * q + b)).  The fp16 bit pattern q is the value
// q * 2^-24 (a subnormal), so v_fma_mix with s * 2^24 (exact: a power of two)
// gives s * q + b with one fp32 rounding.
__device__ __forceinline__ bf16x8_p dequant8_affine(uint32_t c, float s24, float b) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const f16x2_p h = __builtin_bit_cast(f16x2_p, (c >> (4 * j)) & 0x000f000fu);
        v[j] = fmaf((float)h.x, s24, b);
        v[j + 4] = fmaf((float)h.y, s24, b);
    }
    const u32x4_p o = {pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]), pack2_bf16(v[4], v[5]),
                       pack2_bf16(v[6], v[7])};
    return __builtin_bit_cast(bf16x8_p, o);
}

// NVFP4: eight E2M1 codes (one word, byte j holding k = 2j and 2j + 1) -> the
// exact products e2m1(q) * e4m3(s) as bf16 (two significant bits times four
// fit in bf16's eight); the matrix scale is applied to the finished sums.
typedef float f32x2_p __attribute__((ext_vector_type(2)));
template <int B>
__device__ __forceinline__ uint32_t fp4x2_scaled_bf16(uint32_t c, float s) {
    const f32x2_p v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, B);
    return pack2_bf16(v.x * s, v.y * s);
}
__device__ __forceinline__ bf16x8_p dequant8_nv(uint32_t c, float s) {
    const u32x4_p o = {fp4x2_scaled_bf16<0>(c, s), fp4x2_scaled_bf16<1>(c, s), fp4x2_scaled_bf16<2>(c, s),
                       fp4x2_scaled_bf16<3>(c, s)};
    return __builtin_bit_cast(bf16x8_p, o);
}

// MTL: live 16-row subtiles of the tile (the group's rows past them take no
// MFMA and no A fragment reads).
template <int FMT, bool GATEUP, int BM, int MTL>
__device__ void pipe_tile_w4(const ExpertArgs& a, lds_u8* smem, const Group& g, int m0, int nt) {
    using C = W4Cfg<BM>;
    using F = W4Fmt<FMT>;
    static_assert(MTL >= 1 && MTL <= C::MT, "live subtiles");
    typedef __attribute__((address_space(3))) const uint32_t lds_u32;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int Ig = a.I;
    const int H = a.H;
    const int K = GATEUP ? H : Ig;
    const int rows = min(BM, g.n - m0);
    const int KT = K / kBK;

    const uint16_t* asrc[C::LA];
#pragma unroll
    for (int j = 0; j < C::LA; ++j) {
        const int r = 8 * (wave + C::NW * j) + (lane >> 3);
        const int c = (lane & 7) ^ (r & 7);
        const int rr = r < rows ? r : 0;
        const uint16_t* arow;
        if (GATEUP)
            arow = a.x + (size_t)(a.perm[g.row0 + m0 + rr] / a.topk) * H;
        else
            arow = a.h_r + (size_t)(g.row0 + m0 + rr) * a.I;
        asrc[j] = arow + 8 * c;
    }
    // Wave w loads the codes of rows 32 w .. 32 w + 31: lane l takes row
    // 32 w + l % 32, half l / 32 (16 bytes), so the wave's 1 KiB holds the
    // first halves of its 32 rows, then the second halves (16 rows read at one
    // offset then meet 8 bank groups, not 4).
    auto wrow = [&](int r) -> size_t {
        const int row = GATEUP ? (r < 64 ? nt * 64 + r : Ig + nt * 64 + (r - 64)) : nt * kBN + r;
        return (size_t)g.expert * (GATEUP ? 2 * (size_t)Ig : (size_t)H) + row;
    };
    const unsigned char* qsrc =
        (GATEUP ? a.qgu : a.qd) + wrow(32 * wave + (lane & 31)) * (K / 2) + 16 * (lane >> 5);
    // Scale/zero block b (steps G b .. G b + G - 1) is 4 G pieces of PB
    // bytes: piece i covers array i / (4G / NA) (scales, then zeros or
    // biases), rows (i mod (4G / NA)) R .. + R - 1, lane l < AL taking the 4
    // bytes of row + l % R at steps G b + (l / R) SPL .. + SPL - 1, stored in
    // lane order (step-major within the piece).  Per row the G steps are
    // contiguous in memory, so a piece touches R cache lines instead of 64.
    // Block 0 is loaded before the first stage, block b + 1 a piece per stage
    // (one per wave) during the stages of block b, into buffer (b + 1) mod 3.
    const unsigned char* sbase = reinterpret_cast<const unsigned char*>(GATEUP ? a.sgu : a.sd);
    const unsigned char* zbase = reinterpret_cast<const unsigned char*>(GATEUP ? a.zgu : a.zd);
    constexpr int R = F::AL * F::SPL / C::G;  // rows per piece
    constexpr int PPA = 128 / R;              // pieces per array
    const int RSB = KT * F::BPS;              // bytes of a row of one array
    auto issue_sz = [&](int b, int i) {
        const int arr = i / PPA, rg = i % PPA;
        const int r = rg * R + lane % R;
        // the 4-byte chunk of the row holding steps G b + (l / R) SPL ..; chunks
        // past the row's end reload its last one (unused)
        const int chunk = min(C::G * b / F::SPL + lane / R, RSB / 4 - 1);
        const unsigned char* src = (arr ? zbase : sbase) + wrow(r) * RSB + 4 * chunk;
        lds_u8* dst = smem + C::SZOff + (b % 3) * C::SZBlock + arr * (PPA * F::PB) + rg * F::PB;
        if (F::AL == 64 || lane < F::AL) __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
    };

    auto issue = [&](int kt) {
        lds_u8* st = smem + (kt % C::S) * C::Stage;
        const int k0 = kt * kBK;
#pragma unroll
        for (int j = 0; j < C::LA; ++j)
            __builtin_amdgcn_global_load_lds(asrc[j] + k0, st + (wave + C::NW * j) * 1024, 16, 0, 0);
        // (default policy: a 128-byte line of a row's codes serves four steps)
        __builtin_amdgcn_global_load_lds(qsrc + (size_t)kt * 32, st + C::QOff + wave * 1024, 16, 0, 0);
        issue_sz(kt / C::G + 1, 4 * (kt % C::G) + wave);
    };

    f32x4_p acc[MTL][C::NT];
#pragma unroll
    for (int i = 0; i < MTL; ++i)
#pragma unroll
        for (int j = 0; j < C::NT; ++j) acc[i][j] = f32x4_p{0.f, 0.f, 0.f, 0.f};
    int aoff[MTL], ax[MTL], brow[C::NT];
#pragma unroll
    for (int i = 0; i < MTL; ++i) {
        const int r = 16 * i + (lane & 15);
        aoff[i] = r * 128;
        ax[i] = r & 7;
    }
#pragma unroll
    for (int j = 0; j < C::NT; ++j)
        brow[j] = (GATEUP ? (j == 0 ? 0 : 64) + 16 * wave : 32 * wave + 16 * j) + (lane & 15);

    __builtin_amdgcn_s_barrier();  // every wave is done with the previous tile's stages
#pragma unroll
    for (int p = 0; p < C::G; ++p) issue_sz(0, 4 * p + wave);  // block 0, before stage 0
#pragma unroll
    for (int s = 0; s < C::S - 1; ++s)
        if (s < KT) issue(s);

    for (int kt = 0; kt < KT; ++kt) {
        // Stage kt landed (and, loaded before it, the scale/zero block of
        // step kt); stages issued after it may still be in flight.
        const int after = min(C::S - 2, KT - 1 - kt);
        if (after >= 4)
            wait_vmcnt<4 * C::L>();
        else if (after == 3)
            wait_vmcnt<3 * C::L>();
        else if (after == 2)
            wait_vmcnt<2 * C::L>();
        else if (after == 1)
            wait_vmcnt<C::L>();
        else
            wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();  // stage kt visible to all waves; stage kt-1 free
        if (kt + C::S - 1 < KT) issue(kt + C::S - 1);
        const lds_u8* st = smem + (kt % C::S) * C::Stage;
        // this step's 4-byte word of each array: chunk (kt mod G) / SPL of the
        // block, byte (kt mod SPL) BPS within it
        const lds_u8* sz = smem + C::SZOff + ((kt / C::G) % 3) * C::SZBlock + ((kt % C::G) / F::SPL) * (4 * R);
        // Every LDS read of the step first (one wait), then the expansion,
        // then the MFMAs.
        uint32_t sw[C::NT], zw[C::NT], codes[2][C::NT];
        bf16x8_p af[2][MTL];
#pragma unroll
        for (int j = 0; j < C::NT; ++j) {
            const int off = (brow[j] / R) * F::PB + (brow[j] % R) * 4;  // piece, row in piece
            sw[j] = *(lds_u32*)(sz + off);
            zw[j] = F::NA == 2 ? *(lds_u32*)(sz + PPA * F::PB + off) : 0u;
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int q = ks * 4 + (lane >> 4);  // logical 16-byte chunk = 8 codes of k
#pragma unroll
            for (int j = 0; j < C::NT; ++j)
                codes[ks][j] = *(lds_u32*)(st + C::QOff + (brow[j] >> 5) * 1024 + (q >> 2) * 512 +
                                           (brow[j] & 31) * 16 + 4 * (q & 3));
#pragma unroll
            for (int i = 0; i < MTL; ++i) af[ks][i] = *(lds_bf16x8*)(st + aoff[i] + ((q ^ ax[i]) << 4));
        }
        bf16x8_p bfr[2][C::NT];
#pragma unroll
        for (int j = 0; j < C::NT; ++j) {
            if constexpr (FMT == 1) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    // scale and zero of this lane's column for group ks of the step
                    const float sc = __uint_as_float(ks ? (sw[j] & 0xffff0000u) : (sw[j] << 16));
                    const float zz = __uint_as_float(ks ? (zw[j] & 0xffff0000u) : (zw[j] << 16));
                    bfr[ks][j] = dequant8(codes[ks][j], sc, -((1024.0f + zz) * sc));
                }
            } else if constexpr (FMT == 2) {
                // the step's one 64-input group: half kt mod 2 of the words
                const uint32_t sh = kt & 1 ? sw[j] & 0xffff0000u : sw[j] << 16;
                const uint32_t bh = kt & 1 ? zw[j] & 0xffff0000u : zw[j] << 16;
                const float s24 = __uint_as_float(sh) * 16777216.0f;
                const float bb = __uint_as_float(bh);
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) bfr[ks][j] = dequant8_affine(codes[ks][j], s24, bb);
            } else {
                // the lane's eight inputs 32 ks + 8 (lane / 16) .. lie in the
                // step's 16-input group 2 ks + lane / 32
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const float sblk = __builtin_amdgcn_cvt_f32_fp8(sw[j] >> (8 * (2 * ks + (lane >> 5))), 0);
                    bfr[ks][j] = dequant8_nv(codes[ks][j], sblk);
                }
            }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int i = 0; i < MTL; ++i)
#pragma unroll
                for (int j = 0; j < C::NT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks][i], bfr[ks][j], acc[i][j], 0, 0, 0);
    }

    // NVFP4: the matrix scales multiply the finished sums
    float mg = 1.0f, mu = 1.0f;
    if (FMT == 3) {
        mg = GATEUP ? a.ggu[2 * (size_t)g.expert] : a.gd[g.expert];
        mu = GATEUP ? a.ggu[2 * (size_t)g.expert + 1] : mg;
    }
    if (GATEUP) {
        uint16_t* hout = a.h_r + (size_t)(g.row0 + m0) * a.I;
        const int c = nt * 64 + 16 * wave + (lane & 15);
#pragma unroll
        for (int i = 0; i < MTL; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = 16 * i + 4 * (lane >> 4) + v;
                const float gv = FMT == 3 ? acc[i][0][v] * mg : acc[i][0][v];
                const float uv = FMT == 3 ? acc[i][1][v] * mu : acc[i][1][v];
                if (r < rows) hout[(size_t)r * Ig + c] = f32_to_bf16_bits(silu_mul(gv, uv));
            }
    } else {
        if (FMT == 3) {
#pragma unroll
            for (int i = 0; i < MTL; ++i)
#pragma unroll
                for (int j = 0; j < C::NT; ++j) acc[i][j] *= mg;
        }
        float* yout = a.y_r + (size_t)(g.row0 + m0) * H;
#pragma unroll
        for (int i = 0; i < MTL; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = 16 * i + 4 * (lane >> 4) + v;
                if (r >= rows) continue;
#pragma unroll
                for (int j = 0; j < C::NT; ++j)
                    yout[(size_t)r * H + nt * kBN + 32 * wave + 16 * j + (lane & 15)] = acc[i][j][v];
            }
    }
}

// Routed 4-bit groups only (the shared expert is bf16 and runs in
// expert_mfma_pipe_kernel or expert_mfma_small_kernel).  BM = 128 also takes
// the 256-row list, each tile as two 128-row halves.
template <int FMT, bool GATEUP, int BM>
__global__ __launch_bounds__(W4Cfg<BM>::Threads, W4Cfg<BM>::PerCU) void expert_mfma_w4_kernel(ExpertArgs a) {
    using C = W4Cfg<BM>;
    __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[C::Lds];
    lds_u8* smem = (lds_u8*)smem_raw;
    constexpr int list = BM == 128 ? 0 : (BM == 64 ? 1 : 2);
    const int n0 = a.plan_counts[1 + list];
    const int n3 = BM == 128 ? 2 * a.plan_counts[4] : 0;
    const int NT = GATEUP ? a.I / 64 : a.H / kBN;
    XcdWalk w(n0 + n3, NT);
    int tile, nt;
    while (w.next(&tile, &nt)) {
        int l = list, half = 0;
        if (tile >= n0) {
            tile -= n0;
            l = 3;
            half = tile & 1;
            tile >>= 1;
        }
        const int32_t* tl = a.mfma_list + 2 * (size_t)l * a.mfma_cap;
        const Group g = a.groups[tl[2 * tile]];
        if (g.expert < 0) continue;  // the shared expert is bf16
        const int m0 = tl[2 * tile + 1] + 128 * half;
        if (m0 >= g.n) continue;
        // 16-row subtiles holding rows of the group (block-uniform)
        const int live = (min(BM, g.n - m0) + 15) / 16;
        if constexpr (BM == 128) {
            if (live > 7)
                pipe_tile_w4<FMT, GATEUP, BM, 8>(a, smem, g, m0, nt);
            else if (live > 6)
                pipe_tile_w4<FMT, GATEUP, BM, 7>(a, smem, g, m0, nt);
            else if (live > 5)
                pipe_tile_w4<FMT, GATEUP, BM, 6>(a, smem, g, m0, nt);
            else if (live > 4)
                pipe_tile_w4<FMT, GATEUP, BM, 5>(a, smem, g, m0, nt);
            else if (live > 2)
                pipe_tile_w4<FMT, GATEUP, BM, 4>(a, smem, g, m0, nt);
            else
                pipe_tile_w4<FMT, GATEUP, BM, 2>(a, smem, g, m0, nt);
        } else if constexpr (BM == 64) {
            if (live > 3)
                pipe_tile_w4<FMT, GATEUP, BM, 4>(a, smem, g, m0, nt);
            else
                pipe_tile_w4<FMT, GATEUP, BM, 3>(a, smem, g, m0, nt);
        } else {
            pipe_tile_w4<FMT, GATEUP, BM, 2>(a, smem, g, m0, nt);
        }
    }
}

template <int FMT, bool GATEUP, int BM>
static void launch_w4_bm(const ExpertArgs& a, int num_cu, hipStream_t st) {
    using C = W4Cfg<BM>;
    const int NT = GATEUP ? a.I / 64 : a.H / kBN;
    long long grid = (long long)num_cu * C::PerCU;
    const long long ub = (long long)(BM == 128 ? 3 : 1) * a.mfma_cap * NT;
    if (ub < grid) grid = ub;
    grid = grid < 8 ? 8 : grid & ~7LL;  // the XCD walk deals blocks in groups of 8
    expert_mfma_w4_kernel<FMT, GATEUP, BM><<<(int)grid, C::Threads, 0, st>>>(a);
}

// ---- 4-bit experts, wide column tiles ---------------------------------------
//
// For every group of more than 8 rows when the widths are whole wide tiles
// (the 128-weight-row tiles above are bound by their loads).  One block of 8
// waves per CU (two per SIMD).  An item is up to 128 rows (groups of more
// than 64 rows; a 256-row tile as two items) or up to 64 rows (groups of
// 9..64) of a group by 256 weight rows (gate/up: 128 gate and the matching
// 128 up columns; down: 256 output columns); wave w owns 32 of the weight
// rows as two 16-column subtiles and runs as many 16-row subtiles as the
// item's rows fill.  K
// advances 128 per step.  Within a step, lane l (column l % 16 of a subtile,
// lane group l / 16) takes the 32 inputs 32 (l / 16) .. + 31 of the step, one
// 32-input group; its chunk c (c = 0..3) is the MFMA operand pair of inputs
// 32 (l / 16) + 8 c .. + 7 on both sides (the MFMA's inputs relabelled
// consistently in A and B, so the sum over the step is unchanged).  So a
// lane's codes for a step are 16 contiguous bytes of its weight row, loaded
// straight into registers four steps ahead (four buffers).  The A rows (bf16)
// go through an LDS ring of two steps, laid out for conflict-free operand
// reads (below).
// The per-group words come in blocks of whole 128-byte lines of each weight
// row per array (16 steps; MLX affine 32), through a ring of two blocks in
// LDS, so each line is fetched once.  Needs K % 512 == 0 and whole column
// tiles (I % 128 == 0 for gate/up, H % 256 == 0 for down).
constexpr int kWK = 128;                                   // K per step
constexpr int kWLds = 160 * 1024;                          // the larger of the two layouts below
constexpr int kWExpand = 20;                               // VALU instructions of one expansion (about)

// Items of up to 64 rows (MTL <= 4): A stages of 64 rows (16 KiB) and the
// per-group words in whole 128-byte lines (two blocks of 32 KiB per array):
// 160 KiB with two arrays.  Items of up to 128 rows: A stages of 32 KiB and
// half lines of 64 bytes (two blocks of 16 KiB per array): 128 KiB.
template <int FMT, int MTL>
struct WCfg {
    static constexpr int NA = FMT == 3 ? 1 : 2;      // arrays (scales [, zeros / biases])
    static constexpr int BPS = FMT == 2 ? 4 : 8;     // bytes per weight row, step and array
    static constexpr int LineB = MTL > 4 ? 64 : 128; // bytes of a row's words per block and array
    static constexpr int CPR = LineB / 16;           // 16-byte chunks of them
    static constexpr int SPB = LineB / BPS;          // steps per block
    static constexpr int NPS = NA * BPS / 8;         // piece instructions per wave every fourth step
    static constexpr int Arr = 256 * LineB;          // bytes of one array of a block
    static constexpr int PPA = Arr / 1024;           // piece instructions per array
    static constexpr int RPP = 1024 / LineB;         // rows per piece instruction
    static constexpr int AStage = MTL > 4 ? 32768 : 16384;
    static_assert(SPB % 4 == 0, "pieces are issued every fourth step");
    static_assert(2 * AStage + 2 * NA * Arr <= kWLds, "LDS");
};

template <int FMT, bool GATEUP, int MTL>
__device__ void wide_tile_w4(const ExpertArgs& a, lds_u8* smem, const Group& g, int m0, int nt) {
    using F = WCfg<FMT, MTL>;
    typedef __attribute__((address_space(3))) const uint16_t lds_cu16;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, lg = lane >> 4;
    const int Ig = a.I, H = a.H;
    const int K = GATEUP ? H : Ig;
    const int KT = K / kWK;
    const int NB = (KT + F::SPB - 1) / F::SPB;                   // blocks of per-group words
    const int rows = min(16 * MTL, g.n - m0);
    const size_t erows = GATEUP ? 2 * (size_t)Ig : (size_t)H;  // weight rows per expert
    const int RB = KT * F::BPS;                                  // bytes of a weight row of one array
    // the item's 256 weight rows: local row lr -> weight row of the expert
    // (gate/up: lr < 128 gate column nt 128 + lr, else the up row of column
    // nt 128 + lr - 128; down: output column nt 256 + lr); the widths are
    // whole tiles
    auto wrow = [&](int lr) -> int {
        if (GATEUP) return lr < 128 ? nt * 128 + lr : Ig + nt * 128 + (lr - 128);
        return nt * 256 + lr;
    };
    // subtile j of this wave: local rows lr0 + dlr(j) + 0..15
    const int lr0 = GATEUP ? 16 * wave : 32 * wave;
    auto dlr = [&](int j) -> int { return GATEUP ? 128 * j : 16 * j; };

    // A rows in a stage: two regions of 16 MTL lines of 128 bytes, region R
    // holding, for row r, the chunks 4 lg + 2 R + h (lg = 0..3, h = 0..1:
    // the 16-byte chunks that chunk steps c = 2 R + h read) at positions
    // (4 h + lg) ^ (r % 8), so that the 64 lanes of an operand read (16 rows,
    // four lane groups) meet no bank twice.  Instruction ii (= wave + 8 j,
    // below 4 MTL) fills region ii / (2 MTL), lines 8 (ii % (2 MTL)) .. + 7:
    // lane L writes position L % 8 of line 8 (ii % (2 MTL)) + L / 8.  With an
    // odd MTL the first four waves issue one instruction more than the
    // others; the waits below count only what was issued after a stage.
    constexpr int LA = (4 * MTL + 7) / 8;  // A instructions per wave and step (at most)
    constexpr int AReg = 16 * MTL * 128;  // bytes of a region
    const uint16_t* asrc[LA];
#pragma unroll
    for (int j = 0; j < LA; ++j) {
        const int ii = min(wave + 8 * j, 4 * MTL - 1);  // (an unused instruction's source stays in the tile)
        const int R = ii / (2 * MTL);
        const int r = 8 * (ii % (2 * MTL)) + (lane >> 3);
        const int hl = (lane & 7) ^ (r & 7);  // 4 h + lg
        const int q = 4 * (hl & 3) + 2 * R + (hl >> 2);
        const int rr = r < rows ? r : 0;
        const uint16_t* arow = GATEUP ? a.x + (size_t)(a.perm[g.row0 + m0 + rr] / a.topk) * H
                                      : a.h_r + (size_t)(g.row0 + m0 + rr) * Ig;
        asrc[j] = arow + 8 * q;
    }
    auto issue_a = [&](int kt, int stage) {
        lds_u8* st = smem + stage * F::AStage;
#pragma unroll
        for (int j = 0; j < LA; ++j)
            if ((4 * MTL) % 8 == 0 || wave + 8 * j < 4 * MTL)  // wave-uniform
                __builtin_amdgcn_global_load_lds(asrc[j] + kt * kWK, st + (wave + 8 * j) * 1024, 16, 0, 0);
    };
    // per-group words: block b is the LineB-byte piece b of each of the 256
    // weight rows per array (a piece past the row's end reloads the row's
    // last 16 bytes, unused).  In LDS, [array][row][LineB bytes] with the
    // row's 16-byte chunk k at position k ^ (row % CPR).  Instruction i (=
    // wave + 8 p) covers array i / PPA, rows RPP (i % PPA) .. + RPP - 1; lane
    // L writes position L % CPR of row RPP (i % PPA) + L / CPR.  A wave's
    // instructions of block b + 1 are issued NPS at a time at every fourth
    // step of block b.
    const unsigned char* sbase = reinterpret_cast<const unsigned char*>(GATEUP ? a.sgu : a.sd);
    const unsigned char* zbase = reinterpret_cast<const unsigned char*>(GATEUP ? a.zgu : a.zd);
    lds_u8* const szb = smem + 2 * F::AStage;
    auto issue_piece = [&](int b, int p) {
        const int i = wave + 8 * p;
        const int lr = F::RPP * (i % F::PPA) + lane / F::CPR;
        const int k = (lane % F::CPR) ^ (lr % F::CPR);
        const int off = min(F::LineB * b + 16 * k, RB - 16);
        const unsigned char* src =
            ((i / F::PPA) ? zbase : sbase) + ((size_t)g.expert * erows + wrow(lr)) * RB + off;
        __builtin_amdgcn_global_load_lds(src, szb + (b & 1) * (F::NA * F::Arr) + i * 1024, 16, 0, 0);
    };

    // codes: lane's 16 bytes of each subtile's weight row for step kt, four
    // steps ahead in four register buffers.  Buffer loads from the wave's
    // first weight row: the lane offset in one register, the subtile's and
    // the step's offset wave-uniform (every offset is below 2^31; the
    // descriptor's last word is the gfx9 raw 32-bit data format).
    const unsigned char* qw =
        (GATEUP ? a.qgu : a.qd) + ((size_t)g.expert * erows + wrow(lr0)) * (size_t)(K / 2);
    const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc((void*)qw, (short)0, 0x7fffffff, 0x00020000);
    const int qlane = n * (K / 2) + 16 * lg;
    auto load_codes = [&](int kt, uint4* cb) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int dj = (GATEUP ? (j ? Ig : 0) : 16 * j) * (K / 2);
            const u32x4_p v = __builtin_bit_cast(
                u32x4_p, __builtin_amdgcn_raw_buffer_load_b128(qrs, qlane, dj + 64 * kt, 0));
            cb[j] = make_uint4(v.x, v.y, v.z, v.w);
        }
    };

    f32x4_p acc[MTL][2];
#pragma unroll
    for (int i = 0; i < MTL; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_p{0.f, 0.f, 0.f, 0.f};

    // Step kt issues, in this order: A stage kt + 1 and NPS pieces (kt % 4 ==
    // 0) at its top, the codes of step kt + 4 into the buffer it has just
    // used at its end (the last steps' loads past the end reload the last
    // step: the same bytes into the same places), so the vector-memory counts
    // depend only on kt % 4; the top of step kt waits until only what step
    // kt - 1 issued after A stage kt may be in flight.  The A stage of step kt
    // is kt % 2, a constant of each unrolled step.
    __builtin_amdgcn_s_barrier();  // every wave is done with the previous item's LDS
    uint4 cb0[2], cb1[2], cb2[2], cb3[2];
#pragma unroll
    for (int p = 0; p < F::NA * F::LineB / 32; ++p) issue_piece(0, p);
    issue_a(0, 0);
    load_codes(0, cb0);
    load_codes(min(1, KT - 1), cb1);
    load_codes(min(2, KT - 1), cb2);
    load_codes(min(3, KT - 1), cb3);
    // the item starts with nothing in flight (also the compiler's count of
    // the loop-carried code buffers then needs no wait of its own)
    wait_vmcnt<0>();

    auto step = [&](int kt, int p4, uint4* cur) {
        if (p4 == 1)
            wait_vmcnt<F::NPS + 2>();
        else
            wait_vmcnt<2>();
        __builtin_amdgcn_s_barrier();  // stage kt and block kt / SPB visible; stage kt - 1 free
        asm volatile("" ::: "memory");  // no LDS read moves above the barrier
        // (the wait counts rely on this issue order: no instruction moves
        // across the scheduling barriers)
        __builtin_amdgcn_sched_barrier(0);
        issue_a(min(kt + 1, KT - 1), (p4 + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
        if (p4 == 0) {
#pragma unroll
            for (int q = 0; q < F::NPS; ++q) issue_piece(kt / F::SPB + 1, F::NPS * ((kt % F::SPB) / 4) + q);
        }
        __builtin_amdgcn_sched_barrier(0);

        const lds_u8* st = smem + (p4 & 1) * F::AStage;
        const lds_u8* sz = szb + ((kt / F::SPB) & 1) * (F::NA * F::Arr);
        const int t = kt % F::SPB;
        // this lane's per-group words of each subtile: byte bo of its row's
        // piece, in chunk bo / 16 at position (bo / 16) ^ (row % CPR)
        const int bo = FMT == 2 ? 4 * t + 2 * (lg >> 1) : 8 * t + 2 * lg;
        uint32_t sw[2], zw[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int lr = lr0 + n + dlr(j);
            const int off = lr * F::LineB + (((bo >> 4) ^ (lr % F::CPR)) << 4) + (bo & 15);
            sw[j] = *(lds_cu16*)(sz + off);
            zw[j] = F::NA == 2 ? *(lds_cu16*)(sz + F::Arr + off) : 0u;
        }
        float s0[2], s1[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if constexpr (FMT == 1) {
                const float sc = __uint_as_float(sw[j] << 16), zz = __uint_as_float(zw[j] << 16);
                s0[j] = sc;
                s1[j] = -((1024.0f + zz) * sc);
            } else if constexpr (FMT == 2) {
                s0[j] = __uint_as_float(sw[j] << 16) * 16777216.0f;
                s1[j] = __uint_as_float(zw[j] << 16);
            } else {
                s0[j] = __builtin_amdgcn_cvt_f32_fp8(sw[j], 0);
                s1[j] = __builtin_amdgcn_cvt_f32_fp8(sw[j], 1);
            }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            // One chunk at a time.  The expansion of subtile 1 is interleaved
            // with the MFMAs of subtile 0 (a few VALU instructions issue while
            // each MFMA runs), since the two waves of a SIMD pass the step
            // barrier together and would otherwise expand, and then multiply,
            // at the same time.
            __builtin_amdgcn_sched_barrier(0);
            auto expand = [&](int j) -> bf16x8_p {
                const uint32_t w = c == 0 ? cur[j].x : c == 1 ? cur[j].y : c == 2 ? cur[j].z : cur[j].w;
                if constexpr (FMT == 1)
                    return dequant8(w, s0[j], s1[j]);
                else if constexpr (FMT == 2)
                    return dequant8_affine(w, s0[j], s1[j]);
                else
                    return dequant8_nv(w, c < 2 ? s0[j] : s1[j]);
            };
            bf16x8_p af[MTL];
#pragma unroll
            for (int i = 0; i < MTL; ++i)
                af[i] = *(lds_bf16x8*)(st + (c >> 1) * AReg + (16 * i + n) * 128 + (((4 * (c & 1) + lg) ^ (n & 7)) << 4));
            const bf16x8_p b0 = expand(0);
            const bf16x8_p b1 = expand(1);
#pragma unroll
            for (int i = 0; i < MTL; ++i)
                acc[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], b0, acc[i][0], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < MTL; ++i)
                acc[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], b1, acc[i][1], 0, 0, 0);
            // order: the A reads, the first expansion, the first subtile's
            // MFMAs each followed by a share of the second expansion, then
            // the second subtile's MFMAs
            __builtin_amdgcn_sched_group_barrier(0x100, MTL, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, kWExpand, 0);
#pragma unroll
            for (int i = 0; i < MTL; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, (kWExpand + MTL - 1) / MTL, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, MTL, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        load_codes(min(kt + 4, KT - 1), cur);
    };
    // KT is a multiple of 4
    for (int kt = 0; kt < KT; kt += 4) {
        step(kt, 0, cb0);
        step(kt + 1, 1, cb1);
        step(kt + 2, 2, cb2);
        step(kt + 3, 3, cb3);
    }

    // NVFP4: the matrix scales multiply the finished sums
    float mg = 1.0f, mu = 1.0f;
    if (FMT == 3) {
        mg = GATEUP ? a.ggu[2 * (size_t)g.expert] : a.gd[g.expert];
        mu = GATEUP ? a.ggu[2 * (size_t)g.expert + 1] : mg;
    }
    if (GATEUP) {
        uint16_t* hout = a.h_r + (size_t)(g.row0 + m0) * Ig;
        const int c = nt * 128 + 16 * wave + n;
#pragma unroll
        for (int i = 0; i < MTL; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = 16 * i + 4 * lg + v;
                const float gv = FMT == 3 ? acc[i][0][v] * mg : acc[i][0][v];
                const float uv = FMT == 3 ? acc[i][1][v] * mu : acc[i][1][v];
                if (r < rows) hout[(size_t)r * Ig + c] = f32_to_bf16_bits(silu_mul(gv, uv));
            }
    } else {
        float* yout = a.y_r + (size_t)(g.row0 + m0) * H;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int c = nt * 256 + 32 * wave + 16 * j + n;
#pragma unroll
            for (int i = 0; i < MTL; ++i)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int r = 16 * i + 4 * lg + v;
                    if (r < rows) yout[(size_t)r * H + c] = FMT == 3 ? acc[i][j][v] * mg : acc[i][j][v];
                }
        }
    }
}

// The tile lists of the routed 4-bit groups in one persistent launch: the
// groups of more than 64 rows first (128-row items, a 256-row tile as two
// 128-row items), then the groups of 9..64 rows, walked per XCD as the other
// launches are.  (One block per CU either way: the LDS of an item fills it.)
template <int FMT, bool GATEUP>
__global__ __launch_bounds__(512, 2) void expert_mfma_w4w_kernel(ExpertArgs a) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[kWLds];
    lds_u8* smem = (lds_u8*)smem_raw;
    const int n128 = a.plan_counts[1], n64 = a.plan_counts[2], n32 = a.plan_counts[3];
    const int n256 = a.plan_counts[4];
    const int nbig = n128 + 2 * n256;
    const int NT = GATEUP ? a.I / 128 : a.H / 256;
    XcdWalk w(nbig + n64 + n32, NT);
    int tile, nt;
    while (w.next(&tile, &nt)) {
        int l, half = 0;
        const bool big = tile < nbig;
        if (big) {
            if (tile < n128) {
                l = 0;
            } else {
                tile -= n128;
                l = 3;
                half = tile & 1;
                tile >>= 1;
            }
        } else {
            tile -= nbig;
            l = 1;
            if (tile >= n64) {
                tile -= n64;
                l = 2;
            }
        }
        const int32_t* tl = a.mfma_list + 2 * (size_t)l * a.mfma_cap;
        const Group g = a.groups[tl[2 * tile]];
        if (g.expert < 0) continue;  // the shared expert is bf16
        const int m0 = tl[2 * tile + 1] + 128 * half;
        if (m0 >= g.n) continue;
        const int rows = min(big ? 128 : 64, g.n - m0);
        // as many 16-row subtiles as the rows fill (at least 5 for a big
        // item: the second half of a 129..256-row group may be short)
        if (big) {
            if (rows > 112)
                wide_tile_w4<FMT, GATEUP, 8>(a, smem, g, m0, nt);
            else if (rows > 96)
                wide_tile_w4<FMT, GATEUP, 7>(a, smem, g, m0, nt);
            else if (rows > 80)
                wide_tile_w4<FMT, GATEUP, 6>(a, smem, g, m0, nt);
            else
                wide_tile_w4<FMT, GATEUP, 5>(a, smem, g, m0, nt);
        } else {
            if (rows > 48)
                wide_tile_w4<FMT, GATEUP, 4>(a, smem, g, m0, nt);
            else if (rows > 32)
                wide_tile_w4<FMT, GATEUP, 3>(a, smem, g, m0, nt);
            else
                wide_tile_w4<FMT, GATEUP, 2>(a, smem, g, m0, nt);
        }
    }
}

static bool wide_ok(const ExpertArgs& a, bool gateup) {
    const int K = gateup ? a.H : a.I;
    return K % 512 == 0 && (gateup ? a.I % 128 == 0 : a.H % 256 == 0);
}

template <int FMT, bool GATEUP>
static void launch_w4w(const ExpertArgs& a, int num_cu, hipStream_t st) {
    const int NT = GATEUP ? a.I / 128 : a.H / 256;
    long long grid = num_cu;
    const long long ub = 3LL * a.mfma_cap * NT;
    if (ub < grid) grid = ub;
    grid = grid < 8 ? 8 : grid & ~7LL;  // the XCD walk deals blocks in groups of 8
    expert_mfma_w4w_kernel<FMT, GATEUP><<<(int)grid, 512, 0, st>>>(a);
}

template <int FMT>
static void launch_w4_fmt(const ExpertArgs& a, bool gateup, int num_cu, hipStream_t st) {
    if (wide_ok(a, gateup)) {
        gateup ? launch_w4w<FMT, true>(a, num_cu, st) : launch_w4w<FMT, false>(a, num_cu, st);
        return;
    }
    if (gateup) {
        launch_w4_bm<FMT, true, 128>(a, num_cu, st);
        launch_w4_bm<FMT, true, 64>(a, num_cu, st);
        launch_w4_bm<FMT, true, 32>(a, num_cu, st);
    } else {
        launch_w4_bm<FMT, false, 128>(a, num_cu, st);
        launch_w4_bm<FMT, false, 64>(a, num_cu, st);
        launch_w4_bm<FMT, false, 32>(a, num_cu, st);
    }
}

void launch_mfma_w4(const ExpertArgs& a, bool gateup, int num_cu, hipStream_t st) {
    if (a.fmt == 2)
        launch_w4_fmt<2>(a, gateup, num_cu, st);
    else if (a.fmt == 3)
        launch_w4_fmt<3>(a, gateup, num_cu, st);
    else
        launch_w4_fmt<1>(a, gateup, num_cu, st);
    // the bf16 shared expert: one group of T rows, so one tile list (9 <= T
    // since no MFMA launch runs at T <= 8); the small-list launch walks the
    // three lists and skips the 4-bit groups
    if (a.Is > 0) {
        if (a.T > 128)
            gateup ? launch_pipe_bm<true, 256>(a, num_cu, st) : launch_pipe_bm<false, 256>(a, num_cu, st);
        else
            gateup ? launch_small<true>(a, num_cu, st) : launch_small<false>(a, num_cu, st);
    }
}

}  // namespace moe
