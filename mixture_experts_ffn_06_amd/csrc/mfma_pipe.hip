// mfma_pipe.hip -- grouped bf16 expert GEMMs on the matrix cores with a
// multi-stage global->LDS pipeline (groups of more than 8 rows; prefill).
//
// [P1] "GLM-5.2 multi-GPU: expert-parallel sharding + the resident-fit
// benchmark": per-expert expertSwiGLU; its lever table: one batched call over
// all picked experts.  [P5] "GLM-5.3-Flash and full GLM-5.3 on the native CUDA
// engine (tracker) #593": fused gate/up rows 2w wide; grouped experts on
// prompt rows.
//
// A block owns a BM x 128 output tile of one group (BM = 256 with 8 waves, or
// 128, 64, 32 with 4 waves; chosen per tile from the rows it covers, so a
// small group does not pay for 256 rows of matrix work and a large one reads
// each weight tile once per 256 rows) and walks K in steps of 64.  Tiles of A
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

namespace moe {

typedef __bf16 bf16x8_p __attribute__((ext_vector_type(8)));
typedef float f32x4_p __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) const bf16x8_p lds_bf16x8;

constexpr int kBTileBytes = kBN * kBK * 2;  // 16 KiB of weight rows per stage

template <int BM>
struct PipeCfg {
    static constexpr int NW = BM == 256 ? 8 : 4;                  // waves per block
    static constexpr int WM = BM == 256 ? 4 : (BM == 128 ? 2 : 1);  // waves along M
    static constexpr int WN = NW / WM;                            // waves along N
    static constexpr int MT = BM / WM / 16;                       // 16-row subtiles per wave
    static constexpr int NT = kBN / WN / 16;                      // 16-column subtiles per wave
    static constexpr int S = BM == 256 ? 3 : (BM == 128 ? 2 : (BM == 64 ? 3 : 4));  // stages
    static constexpr int LA = BM / 8 / NW;                        // A loads per wave per stage
    static constexpr int LB = kBN / 8 / NW;                       // B loads per wave per stage
    static constexpr int L = LA + LB;                             // all loads per wave per stage
    static constexpr int ATile = BM * kBK * 2;
    static constexpr int Stage = ATile + kBTileBytes;
    static constexpr int Lds = S * Stage;
    static constexpr int PerCU = Lds <= 80 * 1024 ? 2 : 1;
    static constexpr int Threads = 64 * NW;
};

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xf) | (0x7 << 4) | (0xf << 8) | ((N >> 4) << 14));
}

template <bool GATEUP, int BM>
__device__ void pipe_tile(const ExpertArgs& a, lds_u8* smem, const Group& g, int m0, int nt) {
    using C = PipeCfg<BM>;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int wm = wave / C::WN, wn = wave % C::WN;
    const bool shared = g.expert < 0;
    const int Ig = shared ? a.Is : a.I;
    const int H = a.H;
    const int K = GATEUP ? H : Ig;
    const int rows = min(BM, g.n - m0);
    const int KT = K / kBK;

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
        if (GATEUP)
            brow = r < 64 ? nt * 64 + r : Ig + nt * 64 + (r - 64);
        else
            brow = nt * kBN + r;
        bsrc[j] = wbase + (size_t)brow * K + 8 * c;
    }

    auto issue = [&](int kt) {
        lds_u8* st = smem + (kt % C::S) * C::Stage;
        const int k0 = kt * kBK;
#pragma unroll
        for (int j = 0; j < C::LA; ++j)
            __builtin_amdgcn_global_load_lds(asrc[j] + k0, st + (wave + C::NW * j) * 1024, 16, 0, 0);
#pragma unroll
        for (int j = 0; j < C::LB; ++j)
            __builtin_amdgcn_global_load_lds(bsrc[j] + k0, st + C::ATile + (wave + C::NW * j) * 1024,
                                             16, 0, 0);
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
            rb = (j < half ? 0 : 64) + wn * (64 / C::WN) + 16 * (j % half);
        } else {
            rb = wn * (kBN / C::WN) + 16 * j;
        }
        rb += lane & 15;
        boff[j] = C::ATile + rb * 128;
        bx[j] = rb & 7;
    }

    // Plain s_barrier, not __syncthreads(): the latter's release fence would
    // wait for every load in flight and undo the pipeline.  LDS reads are
    // complete before the barrier because the MFMAs consumed them.
    __builtin_amdgcn_s_barrier();  // every wave is done with the previous tile's stages
#pragma unroll
    for (int s = 0; s < C::S - 1; ++s)
        if (s < KT) issue(s);

    for (int kt = 0; kt < KT; ++kt) {
        // Stage kt is complete once at most (stages issued after it) x L of
        // this wave's loads are still in flight.
        const int after = min(C::S - 2, KT - 1 - kt);
        if (after >= 2)
            wait_vmcnt<2 * C::L>();
        else if (after == 1)
            wait_vmcnt<C::L>();
        else
            wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();  // stage kt visible to all waves; stage kt-1 free
        if (kt + C::S - 1 < KT) issue(kt + C::S - 1);
        const lds_u8* st = smem + (kt % C::S) * C::Stage;
#pragma unroll
        for (int ks = 0; ks < kBK / 32; ++ks) {
            const int q = ks * 4 + (lane >> 4);  // logical 16-byte chunk of the operand
            bf16x8_p af[C::MT], bfr[C::NT];
#pragma unroll
            for (int i = 0; i < C::MT; ++i) af[i] = *(lds_bf16x8*)(st + aoff[i] + ((q ^ ax[i]) << 4));
#pragma unroll
            for (int j = 0; j < C::NT; ++j) bfr[j] = *(lds_bf16x8*)(st + boff[j] + ((q ^ bx[j]) << 4));
#pragma unroll
            for (int i = 0; i < C::MT; ++i)
#pragma unroll
                for (int j = 0; j < C::NT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    }

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
                    const int c = nt * 64 + wn * (64 / C::WN) + 16 * j + (lane & 15);
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
                    const int c = nt * kBN + wn * (kBN / C::WN) + 16 * j + (lane & 15);
                    yout[(size_t)r * H + c] = acc[i][j][v];
                }
            }
    }
}

template <bool GATEUP, int BM>
__global__ __launch_bounds__(PipeCfg<BM>::Threads) void expert_mfma_pipe_kernel(ExpertArgs a) {
    using C = PipeCfg<BM>;
    __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[C::Lds];
    lds_u8* smem = (lds_u8*)smem_raw;
    constexpr int list = BM == 256 ? 3 : (BM == 128 ? 0 : (BM == 64 ? 1 : 2));
    const int ntiles = a.plan_counts[1 + list];
    const int32_t* tl = a.mfma_list + 2 * (size_t)list * a.mfma_cap;
    // Every tile gets the same number of column tiles (the larger of the
    // routed and shared widths); items past a group's width are skipped.
    const int NTr = GATEUP ? a.I / 64 : a.H / kBN;
    const int NTs = GATEUP ? a.Is / 64 : a.H / kBN;
    const int NT = NTr > NTs ? NTr : NTs;
    const int total = ntiles * NT;
    for (int item = blockIdx.x; item < total; item += gridDim.x) {
        const int tile = item / NT, nt = item - tile * NT;
        const Group g = a.groups[tl[2 * tile]];
        if (nt >= (g.expert < 0 ? NTs : NTr)) continue;
        pipe_tile<GATEUP, BM>(a, smem, g, tl[2 * tile + 1], nt);
    }
}

template <bool GATEUP, int BM>
static void launch_pipe_bm(const ExpertArgs& a, int num_cu, hipStream_t st) {
    using C = PipeCfg<BM>;
    const int NT = GATEUP ? (a.I > a.Is ? a.I : a.Is) / 64 : a.H / kBN;
    long long grid = (long long)num_cu * C::PerCU;
    const long long ub = (long long)a.mfma_cap * NT;
    if (ub < grid) grid = ub;
    if (grid < 1) grid = 1;
    expert_mfma_pipe_kernel<GATEUP, BM><<<(int)grid, C::Threads, 0, st>>>(a);
}

void launch_mfma_pipe(const ExpertArgs& a, bool gateup, int num_cu, hipStream_t st) {
    if (gateup) {
        launch_pipe_bm<true, 256>(a, num_cu, st);
        launch_pipe_bm<true, 128>(a, num_cu, st);
        launch_pipe_bm<true, 64>(a, num_cu, st);
        launch_pipe_bm<true, 32>(a, num_cu, st);
    } else {
        launch_pipe_bm<false, 256>(a, num_cu, st);
        launch_pipe_bm<false, 128>(a, num_cu, st);
        launch_pipe_bm<false, 64>(a, num_cu, st);
        launch_pipe_bm<false, 32>(a, num_cu, st);
    }
}

}  // namespace moe
