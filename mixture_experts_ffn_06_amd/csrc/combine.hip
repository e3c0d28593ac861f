// combine.hip -- the weighted sum of each row's in-band expert outputs (in pick
// order, or along the canonical tree over expert ids), then the shared expert,
// in fp32 with no atomics; and the sum of band partials (moe_ffn_reduce).
//
// [P1] "GLM-5.2 multi-GPU: expert-parallel sharding + the resident-fit
// benchmark", "What landed": per-rank [H] residual partials, each rank adding
// only the picks it owns; gates table: bit-exact when all picks sit on one
// rank.  [P2] "GLM-5.3-Flash on CUDA: attention on one GPU, routed experts on
// the Sparks (proposal) #214", "Per MoE layer": partials summed in a fixed
// (rank) order.  [P4] "GLM-5.3-Flash on CUDA over three ranks (--tp 3) ...
// #310": fp32 partial rows.
#include "common.h"

// every product and sum below is rounded where it is written (the tree's
// leaves are rounded products): no contraction into fused multiply-adds
#pragma clang fp contract(off)

namespace moe {

// acc + four bf16 residual values (fp32 adds; the bf16 -> fp32 widening is exact)
__device__ __forceinline__ float4 add_res(float4 acc, const uint16_t* r) {
    const uint2 b = *reinterpret_cast<const uint2*>(r);
    return make_float4(acc.x + bf16_lo(b.x), acc.y + bf16_hi(b.x), acc.z + bf16_lo(b.y),
                       acc.w + bf16_hi(b.y));
}

// The expert outputs, the shared output and the partials are each read once
// here: their loads carry the non-temporal hint (the `nt` cache-policy bit),
// so they do not hold cache lines in preference to data that is reused
// (prefill pick-order combine 206 -> 167 us).
typedef float f32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 cload(const float* p) {
    const f32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_nt*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_r,
                                                     const float* __restrict__ y_s,
                                                     const uint16_t* __restrict__ res,
                                                     const int32_t* __restrict__ pos,
                                                     const float* __restrict__ w, int H, int k,
                                                     int ctiles, float* __restrict__ out) {
    const int t = blockIdx.x / ctiles;
    const int c = ((blockIdx.x - t * ctiles) * 256 + threadIdx.x) * 4;
    if (c >= H) return;
    // every pick's slot and weight first, then all of its rows' loads, then
    // the sum in pick order (the loads overlap instead of queueing)
    int p[16];
    float wj[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        p[j] = j < k ? pos[(size_t)t * k + j] : -1;
        wj[j] = p[j] >= 0 ? w[(size_t)t * k + j] : 0.0f;
    }
    float4 v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
        if (p[j] >= 0) v[j] = cload(y_r + (size_t)p[j] * H + c);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        if (p[j] < 0) continue;
        acc.x = __builtin_fmaf(wj[j], v[j].x, acc.x);
        acc.y = __builtin_fmaf(wj[j], v[j].y, acc.y);
        acc.z = __builtin_fmaf(wj[j], v[j].z, acc.z);
        acc.w = __builtin_fmaf(wj[j], v[j].w, acc.w);
    }
    if (y_s) {
        const float4 v = cload(y_s + (size_t)t * H + c);
        acc.x = acc.x + v.x;
        acc.y = acc.y + v.y;
        acc.z = acc.z + v.z;
        acc.w = acc.w + v.w;
    }
    if (res) acc = add_res(acc, res + (size_t)t * H + c);
    *reinterpret_cast<float4*>(out + (size_t)t * H + c) = acc;
}

void launch_combine(const float* y_r, const float* y_s, const uint16_t* res, const int32_t* pos,
                    const float* w, int T, int H, int k, float* out, hipStream_t st) {
    const int ctiles = (H / 4 + 255) / 256;
    combine_kernel<<<T * ctiles, 256, 0, st>>>(y_r, y_s, res, pos, w, H, k, ctiles, out);
}

// ---- the canonical tree ------------------------------------------------------
//
// [P4] "GLM-5.3-Flash on CUDA over three ranks (--tp 3) ... #310", maintainer
// reply: every sum follows one fixed tree of slices however the slices fall
// over ranks.  The tree is the complete binary tree over expert ids; a row's
// leaf e is w_j * y_j for its in-band pick j of expert e, +0.0 elsewhere, and
// an inner node is left + right.  Only the picked leaves are visited: sorted
// by id, two neighbours meet at the node of level c = bit length of (e_a xor
// e_b), and an entry waiting for its right neighbour at level c is kept in
// pend[c] (waiting levels are distinct and grow towards the bottom of the
// stack, so indexing by level is a stack).  A node whose leaves all sit in
// one child equals that child + (+0.0): it turns -0.0 into +0.0 and changes
// nothing else, and applying it twice is applying it once, so an operand is
// "normalised" when at least one such node lies between it and the node
// where it is added.

constexpr int kTreeLevels = 11;  // levels 0..10: E <= 1024

__device__ __forceinline__ float4 add4(float4 a, float4 b) {
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}
__device__ __forceinline__ float4 norm4(float4 a) { return add4(a, make_float4(0.f, 0.f, 0.f, 0.f)); }

// One block per (row, column slice).  The first wave loads the row's picks (a lane each),
// ranks the in-band ones by expert id with shuffles (ids in a row are
// distinct) and stores them sorted; thread 0 then builds the row's program:
// before leaf i is taken, the levels whose waiting entries merge with the
// running value (ascending), the operands to normalise there, and the level
// where the running value then waits; entry m holds the final merges.  Every
// thread then runs the program on its columns, four at a time.
__global__ __launch_bounds__(256) void combine_tree_kernel(const float* __restrict__ y_r,
                                                          const float* __restrict__ y_s,
                                                          const uint16_t* __restrict__ res,
                                                          const int32_t* __restrict__ ids,
                                                          const int32_t* __restrict__ pos,
                                                          const float* __restrict__ w, int H, int k,
                                                          int nsplit, int node_level,
                                                          float* __restrict__ out) {
    __shared__ int s_e[16], s_p[16];
    __shared__ float s_w[16];
    __shared__ uint32_t s_mask[17], s_nl[17], s_nr[17];
    __shared__ int s_push[17];
    __shared__ int s_m, s_rootnorm;
    const int t = blockIdx.x / nsplit;
    const int slice = blockIdx.x - t * nsplit;
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int e = 0x7fffffff, p = -1;
        float wj = 0.0f;
        if (lane < k) {
            p = pos[(size_t)t * k + lane];
            if (p >= 0) {
                e = ids[(size_t)t * k + lane];
                wj = w[(size_t)t * k + lane];
            }
        }
        int rank = 0, m = 0;
        for (int i = 0; i < k; ++i) {
            const int ei = __shfl(e, i, 64);
            if (ei != 0x7fffffff) {
                ++m;
                if (ei < e) ++rank;
            }
        }
        if (lane < k && p >= 0) {
            s_e[rank] = e;
            s_p[rank] = p;
            s_w[rank] = wj;
        }
        if (lane == 0) s_m = m;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const int m = s_m;
        uint32_t occ = 0;     // levels holding a waiting entry
        int tl[kTreeLevels];  // level of the top node of each waiting entry
        int tlc = 0;          // level of the top node of the running value
        for (int i = 1; i <= m; ++i) {
            const int c = i < m ? 32 - __clz(s_e[i - 1] ^ s_e[i]) : kTreeLevels;
            const uint32_t mask = occ & ((1u << c) - 1u);
            uint32_t nl = 0, nr = 0;
            for (int lev = 1; lev < kTreeLevels; ++lev) {
                if (!(mask >> lev & 1u)) continue;
                if (tl[lev] < lev - 1) nl |= 1u << lev;
                if (tlc < lev - 1) nr |= 1u << lev;
                tlc = lev;
            }
            occ &= ~mask;
            s_mask[i] = mask;
            s_nl[i] = nl;
            s_nr[i] = nr;
            s_push[i] = c;
            if (i < m) {
                occ |= 1u << c;
                tl[c] = tlc;
                tlc = 0;
            }
        }
        s_rootnorm = (m > 0 && tlc < node_level) ? 1 : 0;
    }
    __syncthreads();
    const int m = __builtin_amdgcn_readfirstlane(s_m);
    const int rootnorm = __builtin_amdgcn_readfirstlane(s_rootnorm);
    // the slice's columns: 1024-column steps slice, slice + nsplit, ...
    for (int c = 1024 * slice + 4 * threadIdx.x; c < H; c += 1024 * nsplit) {
        float4 cur = make_float4(0.f, 0.f, 0.f, 0.f);
        float4 pend[kTreeLevels];
#pragma unroll
        for (int lev = 0; lev < kTreeLevels; ++lev) pend[lev] = cur;
        for (int i = 0; i <= m; ++i) {
            if (i > 0) {
                const uint32_t mask = __builtin_amdgcn_readfirstlane(s_mask[i]);
                const uint32_t nl = __builtin_amdgcn_readfirstlane(s_nl[i]);
                const uint32_t nr = __builtin_amdgcn_readfirstlane(s_nr[i]);
                const int push = __builtin_amdgcn_readfirstlane(s_push[i]);
#pragma unroll
                for (int lev = 1; lev < kTreeLevels; ++lev) {
                    if (mask >> lev & 1u) {
                        float4 l = pend[lev], r = cur;
                        if (nl >> lev & 1u) l = norm4(l);
                        if (nr >> lev & 1u) r = norm4(r);
                        cur = add4(l, r);
                    }
                }
                if (i < m) {
#pragma unroll
                    for (int lev = 1; lev < kTreeLevels; ++lev)
                        if (lev == push) pend[lev] = cur;
                }
            }
            if (i < m) {
                const int p = __builtin_amdgcn_readfirstlane(s_p[i]);
                const float wi = __builtin_bit_cast(
                    float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, s_w[i])));
                const float4 v = cload(y_r + (size_t)p * H + c);
                cur = make_float4(wi * v.x, wi * v.y, wi * v.z, wi * v.w);
            }
        }
        if (rootnorm) cur = norm4(cur);
        if (y_s) cur = add4(cur, cload(y_s + (size_t)t * H + c));
        if (res) cur = add_res(cur, res + (size_t)t * H + c);
        *reinterpret_cast<float4*>(out + (size_t)t * H + c) = cur;
    }
}

void launch_combine_tree(const float* y_r, const float* y_s, const uint16_t* res, const int32_t* ids,
                         const int32_t* pos, const float* w, int T, int H, int k, int node_level,
                         float* out, hipStream_t st) {
    // small batches split each row over several blocks so the grid fills the chip
    const int steps = (H + 1023) / 1024;
    int nsplit = (2048 + T - 1) / T;
    if (nsplit > steps) nsplit = steps;
    if (nsplit < 1) nsplit = 1;
    combine_tree_kernel<<<T * nsplit, 256, 0, st>>>(y_r, y_s, res, ids, pos, w, H, k, nsplit,
                                                    node_level, out);
}

// ---- sum of band partials ------------------------------------------------------
//
// Rank order: ((p_0 + p_1) + p_2) + ...  ([P2] "Per MoE layer": the partials
// are summed in rank order).  Tree order: the host turns the parts (tree nodes
// tiling a node) into pushes of a node value at level l0, which then merges
// with the waiting entries at levels l0 .. l1-1 (left + right) and waits at
// level l1; nodes past E with no part are pushed as +0.0.  Then the shared
// expert's output and the residual are added, in that order.

__global__ __launch_bounds__(256) void reduce_kernel(ReduceProgram pg, const float* __restrict__ y_s,
                                                    const uint16_t* __restrict__ res, size_t n4,
                                                    float* __restrict__ y) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
        float4 acc;
        if (pg.order == 0) {
            acc = cload(pg.part[0] + 4 * i);
            for (int p = 1; p < pg.nparts; ++p)
                acc = add4(acc, cload(pg.part[p] + 4 * i));
        } else {
            float4 pend[kTreeLevels];
            const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int lev = 0; lev < kTreeLevels; ++lev) pend[lev] = zero;
            for (int o = 0; o < pg.nops; ++o) {
                const int pi = pg.op_part[o], l0 = pg.op_l0[o], l1 = pg.op_l1[o];
                float4 v = pi >= 0 ? cload(pg.part[pi] + 4 * i) : zero;
#pragma unroll
                for (int lev = 0; lev < kTreeLevels; ++lev)
                    if (lev >= l0 && lev < l1) v = add4(pend[lev], v);
#pragma unroll
                for (int lev = 0; lev < kTreeLevels; ++lev)
                    if (lev == l1) pend[lev] = v;
            }
            acc = zero;
#pragma unroll
            for (int lev = 0; lev < kTreeLevels; ++lev)
                if (lev == pg.root_level) acc = pend[lev];
        }
        if (y_s) acc = add4(acc, cload(y_s + 4 * i));
        if (res) acc = add_res(acc, res + 4 * i);
        reinterpret_cast<float4*>(y)[i] = acc;
    }
}

void launch_reduce(const ReduceProgram& pg, const float* y_s, const uint16_t* res, size_t n,
                   float* y, int num_cu, hipStream_t st) {
    const size_t n4 = n / 4;
    size_t grid = (n4 + 255) / 256;
    const size_t cap = (size_t)num_cu * 8;
    if (grid > cap) grid = cap;
    if (grid < 1) grid = 1;
    reduce_kernel<<<(int)grid, 256, 0, st>>>(pg, y_s, res, n4, y);
}

}  // namespace moe
