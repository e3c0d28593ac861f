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

// The sigmoid router's fixed fp32 sigmoid ([P5] "What exists now": GLM's
// router is sigmoid + bias top-k; the selection turns on these fp32 values,
// so every step is pinned): exp_c(x) reduces x by n = rint(x log2 e) times
// ln 2 split in two parts (0.693145751953125, exact in 16 bits, and the fp32
// value nearest the rest), evaluates the Taylor terms 1/i!, i = 6..0, as fp32
// coefficients in Horner form with fused multiply-adds, and scales by 2^n;
// sigmoid_c(l) = 1 / (1 + exp_c(-l)) with IEEE fp32 operations.
__device__ __forceinline__ float exp_c(float x) {
#pragma clang fp contract(off)
    if (x > 88.8f) return INFINITY;
    if (x < -104.0f) return 0.0f;
    const float n = __builtin_rintf(x * 1.44269504088896341f);
    float r = __builtin_fmaf(-n, 0.693145751953125f, x);
    r = __builtin_fmaf(-n, 1.42860682030941723212e-6f, r);
    float p = (float)(1.0 / 720.0);
    p = __builtin_fmaf(p, r, (float)(1.0 / 120.0));
    p = __builtin_fmaf(p, r, (float)(1.0 / 24.0));
    p = __builtin_fmaf(p, r, (float)(1.0 / 6.0));
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    return __builtin_ldexpf(p, (int)n);
}

__device__ __forceinline__ float sigmoid_c(float l) {
#pragma clang fp contract(off)
    const float d = 1.0f + exp_c(-l);
    return 1.0f / d;
}

// Row t of logits [T, E] (PER = ceil(E / 64) values per lane): writes the k
// picks and weights to ids[t k ..], w[t k ..] and, when sids is not null, the
// ids to sids[t k ..] as well.  Called by all 64 lanes of a wave.
// sigmoid = 0: the logits carry the bias; picks by logit, weights the softmax
// over the picks.  sigmoid = 1: the logits are unbiased; picks by
// sigmoid_c(l) + bias (-0.0 as +0.0), weights the picks' raw scores.
template <int PER>
__device__ __forceinline__ void topk_row(const float* __restrict__ logits, const float* __restrict__ bias,
                                         int sigmoid, int t, int E, int k,
                                         int32_t* __restrict__ ids, float* __restrict__ w, int32_t* sids) {
#pragma clang fp contract(off)
    const int lane = threadIdx.x & 63;
    float v[PER], sc[PER];
    uint32_t taken = 0;
#pragma unroll
    for (int m = 0; m < PER; ++m) {
        int e = lane + 64 * m;
        v[m] = (e < E) ? logits[(size_t)t * E + e] : -INFINITY;
        sc[m] = 0.0f;
        if (sigmoid && e < E) {
            sc[m] = sigmoid_c(v[m]);
            float key = bias ? sc[m] + bias[e] : sc[m];
            v[m] = key == 0.0f ? 0.0f : key;
        }
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
        if (sigmoid) {
            // the pick's raw score, from the lane that holds it
            float mine = 0.0f;
#pragma unroll
            for (int m = 0; m < PER; ++m)
                if (m == (bid >> 6)) mine = sc[m];
            sel_v[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), bid & 63));
        }
    }
    if (sigmoid) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (j >= k) break;
            if (lane == j) {
                ids[(size_t)t * k + j] = sel_id[j];
                w[(size_t)t * k + j] = sel_v[j];
                if (sids) sids[t * k + j] = sel_id[j];
            }
        }
        return;
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
