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

// (value, id) keys: a larger value wins, equal values go to the lower id.
// Both fit one unsigned 64-bit key: the high word is the value's bits made
// monotonic (negative values inverted, the sign bit set on the others; -0.0
// is first turned into +0.0), the low word is ~id.  Values are finite or
// infinite (the router produces no NaN from finite inputs).  Key 0 is below
// every real key and marks "nothing left".
__device__ __forceinline__ uint64_t topk_key(float v, int id) {
    uint32_t b = __float_as_uint(v == 0.0f ? 0.0f : v);
    b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)b << 32) | (uint32_t)~id;
}
__device__ __forceinline__ float topk_key_value(uint64_t key) {
    const uint32_t b = (uint32_t)(key >> 32);
    return __uint_as_float((b & 0x80000000u) ? (b & 0x7fffffffu) : ~b);
}
__device__ __forceinline__ int topk_key_id(uint64_t key) { return (int)~(uint32_t)key; }

// One DPP step of the wave maximum: lanes of the rows in ROWMASK compare
// with the lane CTRL names; other lanes keep their key.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ uint64_t key_max_step(uint64_t k) {
    const uint32_t lo = (uint32_t)k, hi = (uint32_t)(k >> 32);
    const uint32_t olo = __builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWMASK, 0xf, false);
    const uint32_t ohi = __builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWMASK, 0xf, false);
    const uint64_t o = ((uint64_t)ohi << 32) | olo;
    return o > k ? o : k;
}

// Largest key of the wave: four steps give every lane its row's maximum, two
// row broadcasts carry rows 0-1 into row 3 (the maximum of a total order does
// not depend on the tree), and lane 63's key goes to every lane.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
    k = key_max_step<0xB1, 0xf>(k);   // quad_perm [1,0,3,2]
    k = key_max_step<0x4E, 0xf>(k);   // quad_perm [2,3,0,1]
    k = key_max_step<0x141, 0xf>(k);  // row_half_mirror
    k = key_max_step<0x140, 0xf>(k);  // row_mirror
    k = key_max_step<0x142, 0xa>(k);  // row_bcast:15 into rows 1 and 3
    k = key_max_step<0x143, 0xc>(k);  // row_bcast:31 into rows 2 and 3
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)k, 63);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(k >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
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
    float sc[PER];
    uint64_t key[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) {
        const int e = lane + 64 * m;
        float v = (e < E) ? logits[(size_t)t * E + e] : 0.0f;
        sc[m] = 0.0f;
        if (sigmoid && e < E) {
            sc[m] = sigmoid_c(v);
            v = bias ? sc[m] + bias[e] : sc[m];
        }
        key[m] = e < E ? topk_key(v, e) : 0ull;
    }
    // lane j keeps pick j (its value and id), so no register array is
    // indexed by the runtime pick number
    float my_v = 0.0f;
    int my_id = 0;
    for (int j = 0; j < k; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int m = 1; m < PER; ++m) best = key[m] > best ? key[m] : best;
        best = wave_max_key(best);
        const int bid = topk_key_id(best);
        // the lane that held the pick takes it out
#pragma unroll
        for (int m = 0; m < PER; ++m)
            if (lane + 64 * m == bid) key[m] = 0ull;
        float v = topk_key_value(best);
        if (sigmoid) {
            // the pick's raw score, from the lane that holds it
            float mine = 0.0f;
#pragma unroll
            for (int m = 0; m < PER; ++m)
                if (m == (bid >> 6)) mine = sc[m];
            v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), bid & 63));
        }
        if (lane == j) {
            my_v = v;
            my_id = bid;
        }
    }
    if (lane >= k) return;
    ids[(size_t)t * k + lane] = my_id;
    if (sids) sids[t * k + lane] = my_id;
    if (sigmoid) {
        w[(size_t)t * k + lane] = my_v;
        return;
    }
    // softmax over the picks: a_j = exp(l_j - l_0), summed in pick order
    const float m0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_v), 0));
    const float a = expf(my_v - m0);
    float s = 0.0f;
    for (int j = 0; j < k; ++j) s = s + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), j));
    w[(size_t)t * k + lane] = a / s;
}

}  // namespace moe
