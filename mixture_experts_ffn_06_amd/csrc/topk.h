// topk.h -- top-k selection of one row of router logits by one wave, with
// the softmax over the picks.  Shared by the stand-alone top-k kernel and the
// fused top-k + dispatch kernel for small batches.
//
// [P2] "GLM-5.3-Flash on CUDA: attention on one GPU, routed experts on the
// Sparks (proposal) #214", "Per MoE layer": rows travel with their top-k ids
// and weights.  Experts are ordered by (logit descending, id ascending); the
// first k in that order are the picks, in pick order; the weights are the
// softmax over the picks.
#pragma once
#include "common.h"

namespace moe {

// (value, id) keys: a larger value wins, equal values go to the lower id;
// id 0x7fffffff marks "nothing left" and always loses.
__device__ __forceinline__ bool key_better(float v2, int i2, float v1, int i1) {
    return i2 != 0x7fffffff && (i1 == 0x7fffffff || v2 > v1 || (v2 == v1 && i2 < i1));
}

template <int CTRL>
__device__ __forceinline__ void key_step(float& v, int& i) {
    const float ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
    const int oi = __builtin_amdgcn_update_dpp(0, i, CTRL, 0xf, 0xf, false);
    if (key_better(ov, oi, v, i)) {
        v = ov;
        i = oi;
    }
}

// Best key of the wave: four DPP steps give every lane its row's best, then
// the four row winners are combined.  Every lane gets the result.
__device__ __forceinline__ void wave_best(float& v, int& i) {
    key_step<0xB1>(v, i);   // quad_perm [1,0,3,2]
    key_step<0x4E>(v, i);   // quad_perm [2,3,0,1]
    key_step<0x141>(v, i);  // row_half_mirror
    key_step<0x140>(v, i);  // row_mirror
    float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
        const float rv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * r));
        const int ri = __builtin_amdgcn_readlane(i, 16 * r);
        if (key_better(rv, ri, bv, bi)) {
            bv = rv;
            bi = ri;
        }
    }
    v = bv;
    i = bi;
}

// Row t of logits [T, E] (PER = ceil(E / 64) values per lane): writes the k
// picks and weights to ids[t k ..], w[t k ..] and, when sids is not null, the
// ids to sids[t k ..] as well.  Called by all 64 lanes of a wave.
template <int PER>
__device__ __forceinline__ void topk_row(const float* __restrict__ logits, int t, int E, int k,
                                         int32_t* __restrict__ ids, float* __restrict__ w, int32_t* sids) {
#pragma clang fp contract(off)
    const int lane = threadIdx.x & 63;
    float v[PER];
    uint32_t taken = 0;
#pragma unroll
    for (int m = 0; m < PER; ++m) {
        int e = lane + 64 * m;
        v[m] = (e < E) ? logits[(size_t)t * E + e] : -INFINITY;
        if (e >= E) taken |= 1u << m;
    }
    float sel_v[16];
    int sel_id[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        sel_v[j] = 0.0f;
        sel_id[j] = 0;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        if (j >= k) break;
        float bv = -INFINITY;
        int bid = 0x7fffffff;
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            if (taken >> m & 1u) continue;
            // ids grow with m inside a lane, so a strict compare keeps the lower id on ties
            if (bid == 0x7fffffff || v[m] > bv) {
                bv = v[m];
                bid = lane + 64 * m;
            }
        }
        wave_best(bv, bid);
        if ((bid & 63) == lane) taken |= 1u << (bid >> 6);
        sel_v[j] = bv;
        sel_id[j] = bid;
    }
    const float m0 = sel_v[0];
    float a[16];
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        if (j >= k) break;
        a[j] = expf(sel_v[j] - m0);
        s = s + a[j];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        if (j >= k) break;
        if (lane == j) {
            ids[(size_t)t * k + j] = sel_id[j];
            w[(size_t)t * k + j] = a[j] / s;
            if (sids) sids[t * k + j] = sel_id[j];
        }
    }
}

}  // namespace moe
