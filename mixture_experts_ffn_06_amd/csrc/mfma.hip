// mfma.hip -- grouped expert GEMMs on the bf16 matrix cores for groups of more
// than 8 rows (prefill): gate/up with the SwiGLU epilogue fused, then down.
//
// [P1] "GLM-5.2 multi-GPU: expert-parallel sharding + the resident-fit
// benchmark": per-expert expertSwiGLU; its lever table: one batched call over
// all picked experts instead of a loop.  [P5] "GLM-5.3-Flash and full GLM-5.3
// on the native CUDA engine (tracker) #593": fused gate/up rows 2w wide; W4A16
// experts; grouped experts on prompt rows.
//
// One block (4 waves) computes a 128 x 128 output tile of one group with a
// 64-deep K step, double-buffered through LDS.  Gate/up tiles hold 64 gate and
// the matching 64 up columns, so each lane ends with gate and up values of the
// same (row, column) and applies silu(gate) * up in registers.  Wave tile
// 64 x 64 of 16x16x32 bf16 MFMAs.  4-bit weights are expanded to bf16 (round
// to nearest even of (code - zero) * scale, exact in fp32) between the global
// load and the LDS store.  Blocks are persistent over (tile, column tile) work
// items; with column-tile counts that are multiples of 8, a weight column tile
// always lands on the same XCD, so its re-reads by other row tiles of the same
// expert hit that XCD's L2.
#include "common.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kLdsStride = kBK + 8;  // bf16 elements per LDS row (padding against bank conflicts)
constexpr int kMfmaThreads = 256;

struct TileSmem {
    uint16_t a[2][kBM * kLdsStride];
    uint16_t b[2][kBN * kLdsStride];
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// 32 codes (16 bytes, low nibble first) of one group -> 32 bf16 values.
__device__ __forceinline__ void dequant32(const uint4& q, float sc, float zz, uint4 out[4]) {
    const uint32_t qd[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = ((float)((qd[d] >> (4 * i)) & 0xfu) - zz) * sc;
        out[d].x = pack_bf16x2(v[0], v[1]);
        out[d].y = pack_bf16x2(v[2], v[3]);
        out[d].z = pack_bf16x2(v[4], v[5]);
        out[d].w = pack_bf16x2(v[6], v[7]);
    }
}

template <int W4, bool GATEUP>
__device__ void mfma_tile(const ExpertArgs& a, TileSmem& sm, const Group& g, int m0, int nt) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const bool shared = g.expert < 0;
    const int Ig = shared ? a.Is : a.I;
    const int H = a.H;
    const int K = GATEUP ? H : Ig;
    const int rows = min(kBM, g.n - m0);

    // A rows this thread loads: (tid >> 3) + 32 i, 16 bytes at k (tid & 7) * 8.
    const uint16_t* asrc[4];
    bool avalid[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (tid >> 3) + 32 * i;
        avalid[i] = r < rows;
        const int rr = avalid[i] ? r : 0;
        if (GATEUP) {
            const int tok = shared ? m0 + rr : a.perm[g.row0 + m0 + rr] / a.topk;
            asrc[i] = a.x + (size_t)tok * H;
        } else {
            asrc[i] = shared ? a.h_s + (size_t)(m0 + rr) * a.Is
                             : a.h_r + (size_t)(g.row0 + m0 + rr) * a.I;
        }
    }
    // B (weight) rows.  bf16: rows (tid >> 3) + 32 i; 4-bit: row tid >> 1, half tid & 1.
    const uint16_t* bsrc[4];
    size_t qrow = 0;
    if (!W4 || shared) {
        const uint16_t* wbase = GATEUP ? (shared ? a.swgu : a.wgu + (size_t)g.expert * 2 * Ig * H)
                                       : (shared ? a.swd : a.wd + (size_t)g.expert * H * Ig);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = (tid >> 3) + 32 * i;
            int row;
            if (GATEUP)
                row = j < 64 ? nt * 64 + j : Ig + nt * 64 + (j - 64);
            else
                row = nt * kBN + j;
            bsrc[i] = wbase + (size_t)row * K;
        }
    } else {
        const int j = tid >> 1;
        int row;
        if (GATEUP)
            row = j < 64 ? nt * 64 + j : Ig + nt * 64 + (j - 64);
        else
            row = nt * kBN + j;
        qrow = (size_t)g.expert * (GATEUP ? 2 * (size_t)Ig : (size_t)H) + row;
    }
    const uint8_t* qbase = GATEUP ? a.qgu : a.qd;
    const uint16_t* sbase = GATEUP ? a.sgu : a.sd;
    const uint16_t* zbase = GATEUP ? a.zgu : a.zd;

    uint4 ra[4], rb[4];
    auto gload = [&](int k0) {
        const int kc = (tid & 7) * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            ra[i] = avalid[i] ? *reinterpret_cast<const uint4*>(asrc[i] + k0 + kc) : make_uint4(0, 0, 0, 0);
        if (!W4 || shared) {
#pragma unroll
            for (int i = 0; i < 4; ++i) rb[i] = *reinterpret_cast<const uint4*>(bsrc[i] + k0 + kc);
        } else {
            const int half = tid & 1;
            const int kk = k0 + 32 * half;
            const uint4 q = *reinterpret_cast<const uint4*>(qbase + qrow * (K / 2) + kk / 2);
            const float sc = bf16_bits_to_f32(sbase[qrow * (K / 32) + kk / 32]);
            const float zz = bf16_bits_to_f32(zbase[qrow * (K / 32) + kk / 32]);
            dequant32(q, sc, zz, rb);
        }
    };
    auto sstore = [&](int buf) {
        const int kc = (tid & 7) * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = (tid >> 3) + 32 * i;
            *reinterpret_cast<uint4*>(&sm.a[buf][r * kLdsStride + kc]) = ra[i];
        }
        if (!W4 || shared) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = (tid >> 3) + 32 * i;
                *reinterpret_cast<uint4*>(&sm.b[buf][r * kLdsStride + kc]) = rb[i];
            }
        } else {
            const int r = tid >> 1, half = tid & 1;
#pragma unroll
            for (int d = 0; d < 4; ++d)
                *reinterpret_cast<uint4*>(&sm.b[buf][r * kLdsStride + 32 * half + 8 * d]) = rb[d];
        }
    };

    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // B row offsets of this wave's four 16-column subtiles.
    int bcol[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (GATEUP)
            bcol[j] = (j < 2) ? wn * 32 + 16 * j : 64 + wn * 32 + 16 * (j - 2);
        else
            bcol[j] = wn * 64 + 16 * j;
    }

    const int KT = K / kBK;
    __syncthreads();  // the previous tile's readers are done with the buffers
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) gload((kt + 1) * kBK);
#pragma unroll
        for (int ks = 0; ks < kBK / 32; ++ks) {
            const int kofs = ks * 32 + (lane >> 4) * 8;
            bf16x8_t af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wm * 64 + 16 * i + (lane & 15);
                af[i] = *reinterpret_cast<const bf16x8_t*>(&sm.a[buf][r * kLdsStride + kofs]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = bcol[j] + (lane & 15);
                bfr[j] = *reinterpret_cast<const bf16x8_t*>(&sm.b[buf][r * kLdsStride + kofs]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < KT) sstore(buf ^ 1);
        __syncthreads();
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

// Walks the tile lists of the dispatch with 128-row tiles: a 256-row tile is
// two of them; a shorter tile's missing rows are zero and never stored.
template <int W4, bool GATEUP>
__global__ __launch_bounds__(kMfmaThreads) void expert_mfma_kernel(ExpertArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    TileSmem& sm = *reinterpret_cast<TileSmem*>(smem_raw);
    const int n0 = a.plan_counts[1], n1 = a.plan_counts[2], n2 = a.plan_counts[3];
    const int n3 = 2 * a.plan_counts[4];  // 256-row tiles as pairs of 128-row tiles
    const int ntiles = n0 + n1 + n2 + n3;
    const int NTr = GATEUP ? a.I / 64 : a.H / kBN;
    const int NTs = GATEUP ? a.Is / 64 : a.H / kBN;
    const int NT = NTr > NTs ? NTr : NTs;
    const int total = ntiles * NT;
    for (int item = blockIdx.x; item < total; item += gridDim.x) {
        int tile = item / NT;
        const int nt = item - tile * NT;
        int list = 0, half = 0;
        if (tile >= n0) {
            tile -= n0;
            list = 1;
            if (tile >= n1) {
                tile -= n1;
                list = 2;
                if (tile >= n2) {
                    tile -= n2;
                    list = 3;
                    half = tile & 1;
                    tile >>= 1;
                }
            }
        }
        const int32_t* tl = a.mfma_list + 2 * (size_t)list * a.mfma_cap;
        const Group g = a.groups[tl[2 * tile]];
        if (nt >= (g.expert < 0 ? NTs : NTr)) continue;
        const int m0 = tl[2 * tile + 1] + 128 * half;
        if (m0 >= g.n) continue;
        if (W4 && g.expert >= 0)
            mfma_tile<1, GATEUP>(a, sm, g, m0, nt);
        else
            mfma_tile<0, GATEUP>(a, sm, g, m0, nt);
    }
}

static int mfma_grid(int num_cu, long long ub) {
    long long g = (long long)num_cu * 2;
    if (ub < g) g = ub;
    return (int)(g < 1 ? 1 : g);
}

void launch_gateup_mfma(const ExpertArgs& a, int max_tiles, int num_cu, hipStream_t st) {
    const int nt = (a.I > a.Is ? a.I : a.Is) / 64;
    const int grid = mfma_grid(num_cu, 5LL * max_tiles * nt);
    const size_t lds = sizeof(TileSmem);
    if (a.fmt) {
        allow_lds(expert_mfma_kernel<1, true>, lds);
        expert_mfma_kernel<1, true><<<grid, kMfmaThreads, lds, st>>>(a);
    } else {
        allow_lds(expert_mfma_kernel<0, true>, lds);
        expert_mfma_kernel<0, true><<<grid, kMfmaThreads, lds, st>>>(a);
    }
}

void launch_down_mfma(const ExpertArgs& a, int max_tiles, int num_cu, hipStream_t st) {
    const int nt = a.H / kBN;
    const int grid = mfma_grid(num_cu, 5LL * max_tiles * nt);
    const size_t lds = sizeof(TileSmem);
    if (a.fmt) {
        allow_lds(expert_mfma_kernel<1, false>, lds);
        expert_mfma_kernel<1, false><<<grid, kMfmaThreads, lds, st>>>(a);
    } else {
        allow_lds(expert_mfma_kernel<0, false>, lds);
        expert_mfma_kernel<0, false><<<grid, kMfmaThreads, lds, st>>>(a);
    }
}

}  // namespace moe
