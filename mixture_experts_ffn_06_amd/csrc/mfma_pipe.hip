// mfma_pipe.hip -- grouped bf16 expert GEMMs on the matrix cores with a
// four-stage global->LDS pipeline (groups of more than 8 rows; prefill).
//
// [P1] "GLM-5.2 multi-GPU: expert-parallel sharding + the resident-fit
// benchmark": per-expert expertSwiGLU; its lever table: one batched call over
// all picked experts.  [P5] "GLM-5.3-Flash and full GLM-5.3 on the native CUDA
// engine (tracker) #593": fused gate/up rows 2w wide; grouped experts on
// prompt rows.
//
// A block of 4 waves owns a 128 x 128 output tile of one group and walks K in
// steps of 64.  Tiles of A (the group's rows) and B (weight rows) go straight
// from global memory into LDS with global_load_lds_dwordx4 (16 bytes per lane,
// a wave filling 1 KiB = 8 rows of 128 bytes), four K steps in flight.  In
// LDS a row's eight 16-byte chunks are XOR-swizzled by the row index so the
// MFMA operand reads of 16 consecutive rows hit different banks.  Each wave
// computes a 64 x 64 piece with 16x16x32 bf16 MFMAs; gate/up tiles hold 64 gate
// and the matching 64 up columns so the SwiGLU epilogue stays in registers.
#include "common.h"

namespace moe {

typedef __bf16 bf16x8_p __attribute__((ext_vector_type(8)));
typedef float f32x4_p __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) const bf16x8_p lds_bf16x8;

constexpr int kStages = 4;
constexpr int kTileBytes = kBM * kBK * 2;          // 16 KiB for A, the same for B
constexpr int kStageBytes = 2 * kTileBytes;        // A then B
constexpr int kPipeLds = kStages * kStageBytes;    // 128 KiB
constexpr int kPipeThreads = 256;
constexpr int kLoadsPerStage = 8;                  // per wave: 4 for A, 4 for B

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xf) | (0x7 << 4) | (0xf << 8) | ((N >> 4) << 14));
}

template <bool GATEUP>
__device__ void pipe_tile(const ExpertArgs& a, lds_u8* smem, const Group& g, int m0, int nt) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int wm = wave >> 1, wn = wave & 1;
    const bool shared = g.expert < 0;
    const int Ig = shared ? a.Is : a.I;
    const int H = a.H;
    const int K = GATEUP ? H : Ig;
    const int rows = min(kBM, g.n - m0);
    const int KT = K / kBK;

    // This lane's load sources.  Load instruction j of this wave fills tile
    // rows 8 (wave + 4 j) .. +7; lane l writes physical chunk l % 8 of row
    // 8 (wave + 4 j) + l / 8, which holds logical chunk (l % 8) ^ (row % 8).
    const uint16_t* asrc[4];
    const uint16_t* bsrc[4];
    const uint16_t* wbase = GATEUP ? (shared ? a.swgu : a.wgu + (size_t)g.expert * 2 * Ig * H)
                                   : (shared ? a.swd : a.wd + (size_t)g.expert * H * Ig);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 8 * (wave + 4 * j) + (lane >> 3);
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
        int brow;
        if (GATEUP)
            brow = r < 64 ? nt * 64 + r : Ig + nt * 64 + (r - 64);
        else
            brow = nt * kBN + r;
        bsrc[j] = wbase + (size_t)brow * K + 8 * c;
    }

    auto issue = [&](int kt) {
        lds_u8* st = smem + (kt % kStages) * kStageBytes;
        const int k0 = kt * kBK;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_global_load_lds(asrc[j] + k0, st + (wave + 4 * j) * 1024, 16, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_global_load_lds(bsrc[j] + k0, st + kTileBytes + (wave + 4 * j) * 1024, 16,
                                             0, 0);
    };

    f32x4_p acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_p{0.f, 0.f, 0.f, 0.f};

    // B tile rows of this wave's four 16-column subtiles.
    int bcol[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (GATEUP)
            bcol[j] = (j < 2) ? wn * 32 + 16 * j : 64 + wn * 32 + 16 * (j - 2);
        else
            bcol[j] = wn * 64 + 16 * j;
    }
    // Byte offsets (within a stage) of this lane's operand rows; the chunk is
    // XORed with the row's low bits when read.
    int aoff[4], boff[4], ax[4], bx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = wm * 64 + 16 * i + (lane & 15);
        aoff[i] = r * 128;
        ax[i] = r & 7;
        const int rb = bcol[i] + (lane & 15);
        boff[i] = kTileBytes + rb * 128;
        bx[i] = rb & 7;
    }

    // Plain s_barrier, not __syncthreads(): the latter's release fence would
    // wait for every load in flight and undo the pipeline.  LDS reads are
    // complete before the barrier because the MFMAs consumed them.
    __builtin_amdgcn_s_barrier();  // every wave is done with the previous tile's stages
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
        if (s < KT) issue(s);

    for (int kt = 0; kt < KT; ++kt) {
        // Stage kt is complete once at most (stages issued after it) x 8 of
        // this wave's loads are still in flight.
        const int after = min(kStages - 2, KT - 1 - kt);
        if (after >= 2)
            wait_vmcnt<2 * kLoadsPerStage>();
        else if (after == 1)
            wait_vmcnt<kLoadsPerStage>();
        else
            wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();  // stage kt visible to all waves; stage kt-1 free
        if (kt + kStages - 1 < KT) issue(kt + kStages - 1);
        const lds_u8* st = smem + (kt % kStages) * kStageBytes;
#pragma unroll
        for (int ks = 0; ks < kBK / 32; ++ks) {
            const int q = ks * 4 + (lane >> 4);  // logical 16-byte chunk of the operand
            bf16x8_p af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *(lds_bf16x8*)(st + aoff[i] + ((q ^ ax[i]) << 4));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bfr[j] = *(lds_bf16x8*)(st + boff[j] + ((q ^ bx[j]) << 4));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    }

    // Epilogue.  Lane holds D[4 (lane >> 4) + v][lane & 15] of each 16x16 subtile.
    if (GATEUP) {
        uint16_t* hout = shared ? a.h_s + (size_t)m0 * a.Is : a.h_r + (size_t)(g.row0 + m0) * a.I;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = wm * 64 + 16 * i + 4 * (lane >> 4) + v;
                if (r >= rows) continue;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int c = nt * 64 + wn * 32 + 16 * j + (lane & 15);
                    hout[(size_t)r * Ig + c] = f32_to_bf16_bits(silu_mul(acc[i][j][v], acc[i][j + 2][v]));
                }
            }
    } else {
        float* yout = shared ? a.y_s + (size_t)m0 * H : a.y_r + (size_t)(g.row0 + m0) * H;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = wm * 64 + 16 * i + 4 * (lane >> 4) + v;
                if (r >= rows) continue;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = nt * kBN + wn * 64 + 16 * j + (lane & 15);
                    yout[(size_t)r * H + c] = acc[i][j][v];
                }
            }
    }
}

template <bool GATEUP>
__global__ __launch_bounds__(kPipeThreads) void expert_mfma_pipe_kernel(ExpertArgs a, int sh_tiles) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[kPipeLds];
    lds_u8* smem = (lds_u8*)smem_raw;
    const int ntiles = a.plan_counts[1];
    if (ntiles == 0) return;
    const int last_group = a.mfma_list[2 * (ntiles - 1)];
    const int shn = a.groups[last_group].expert < 0 ? sh_tiles : 0;
    const int rt = ntiles - shn;
    const int NTr = GATEUP ? a.I / 64 : a.H / kBN;
    const int NTs = GATEUP ? a.Is / 64 : a.H / kBN;
    const int total = rt * NTr + shn * NTs;
    for (int item = blockIdx.x; item < total; item += gridDim.x) {
        int tile, nt;
        if (item < rt * NTr) {
            tile = item / NTr;
            nt = item - tile * NTr;
        } else {
            const int it2 = item - rt * NTr;
            tile = rt + it2 / NTs;
            nt = it2 - (it2 / NTs) * NTs;
        }
        const Group g = a.groups[a.mfma_list[2 * tile]];
        const int m0 = a.mfma_list[2 * tile + 1];
        pipe_tile<GATEUP>(a, smem, g, m0, nt);
    }
}

void launch_mfma_pipe(const ExpertArgs& a, bool gateup, int max_tiles, int num_cu, hipStream_t st) {
    const int sh_tiles = (a.T + kBM - 1) / kBM;
    const int nt = gateup ? (a.I > a.Is ? a.I : a.Is) / 64 : a.H / kBN;
    long long grid = num_cu;  // one 128 KiB block per CU
    if ((long long)max_tiles * nt < grid) grid = (long long)max_tiles * nt;
    if (grid < 1) grid = 1;
    if (gateup)
        expert_mfma_pipe_kernel<true><<<(int)grid, kPipeThreads, 0, st>>>(a, sh_tiles);
    else
        expert_mfma_pipe_kernel<false><<<(int)grid, kPipeThreads, 0, st>>>(a, sh_tiles);
}

}  // namespace moe
