// router.hip -- router logits (fp32 fixed-order dot) and top-k selection with
// renormalised weights, for every row and every expert.
//
// [P1] "GLM-5.2 multi-GPU: expert-parallel sharding + the resident-fit
// benchmark", "What landed": the router runs replicated and picks the same
// top-k on every rank, so the logits must come out bit-identical wherever they
// are computed.  [P5] "GLM-5.3-Flash and full GLM-5.3 on the native CUDA
// engine (tracker) #593", "What exists now": fp32 fixed-order reductions.
// The fixed order: 64 lane partials, lane l accumulating fused multiply-adds
// over k = 256 i + 4 l + c (i outer, c inner) from +0.0, then pairwise rounds
// with lane l xor 1, 2, 4, 8, 16, 32.  Every lane of a wave plays one lane of
// that order, so a wave computes a dot in exactly that order.
#include "common.h"

#pragma clang fp contract(off)

namespace moe {

// One wave computes a tile of RB rows x EB experts; four waves per block.
// One wave computes a tile of RB rows x EB experts; four waves per block.
// The loads of BATCH steps of i are issued before any of them is used.
template <int RB, int EB, int BATCH>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ wr,
                                                            const float* __restrict__ bias,
                                                            int T, int H, int E,
                                                            float* __restrict__ logits) {
    const int lane = threadIdx.x & 63;
    // wave-uniform values live in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    const int ET = (E + EB - 1) / EB;
    const int RT = (T + RB - 1) / RB;
    if (wave >= RT * ET) return;
    const int rt = wave / ET, et = wave % ET;
    const int t0 = rt * RB, e0 = et * EB;

    const uint16_t* xp[RB];
    const float* wp[EB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        int t = min(t0 + r, T - 1);
        xp[r] = x + (size_t)t * H;
    }
#pragma unroll
    for (int e = 0; e < EB; ++e) {
        int ee = min(e0 + e, E - 1);
        wp[e] = wr + (size_t)ee * H;
    }
    float acc[RB][EB];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int e = 0; e < EB; ++e) acc[r][e] = 0.0f;

    const int nI = H / 256;
    for (int i0 = 0; i0 < nI; i0 += BATCH) {
        uint2 xu[BATCH][RB];
        float4 wf[BATCH][EB];
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
            const int i = min(i0 + b, nI - 1);  // steps past the end reload the last one, unused
#pragma unroll
            for (int r = 0; r < RB; ++r)
                xu[b][r] = *reinterpret_cast<const uint2*>(xp[r] + 256 * i + 4 * lane);
#pragma unroll
            for (int e = 0; e < EB; ++e)
                wf[b][e] = *reinterpret_cast<const float4*>(wp[e] + 256 * i + 4 * lane);
        }
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
            if (i0 + b < nI) {  // wave-uniform
            float xv[RB][4], wv[EB][4];
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                xv[r][0] = bf16_lo(xu[b][r].x);
                xv[r][1] = bf16_hi(xu[b][r].x);
                xv[r][2] = bf16_lo(xu[b][r].y);
                xv[r][3] = bf16_hi(xu[b][r].y);
            }
#pragma unroll
            for (int e = 0; e < EB; ++e) {
                wv[e][0] = wf[b][e].x;
                wv[e][1] = wf[b][e].y;
                wv[e][2] = wf[b][e].z;
                wv[e][3] = wf[b][e].w;
            }
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int r = 0; r < RB; ++r)
#pragma unroll
                    for (int e = 0; e < EB; ++e) acc[r][e] = __builtin_fmaf(xv[r][c], wv[e][c], acc[r][e]);
            }
        }
    }
#pragma unroll
    for (int s = 1; s < 64; s <<= 1)
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int e = 0; e < EB; ++e) acc[r][e] = acc[r][e] + __shfl_xor(acc[r][e], s, 64);

#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int e = 0; e < EB; ++e) {
            if (((r * EB + e) & 63) != lane) continue;
            const int t = t0 + r, ee = e0 + e;
            if (t >= T || ee >= E) continue;
            float v = acc[r][e];
            if (bias) v = v + bias[ee];
            v = (v == 0.0f) ? 0.0f : v;  // -0.0 -> +0.0
            logits[(size_t)t * E + ee] = v;
        }
}

void launch_router_logits(const uint16_t* x, const float* wr, const float* bias, int T, int H,
                          int E, float* logits, hipStream_t st) {
    int waves, blocks;
    if (T <= 1) {
        waves = E;
        blocks = (waves + 3) / 4;
        router_logits_kernel<1, 1, 12><<<blocks, 256, 0, st>>>(x, wr, bias, T, H, E, logits);
    } else if (T <= 2) {
        waves = E;
        blocks = (waves + 3) / 4;
        router_logits_kernel<2, 1, 12><<<blocks, 256, 0, st>>>(x, wr, bias, T, H, E, logits);
    } else if (T <= 4) {
        waves = E;
        blocks = (waves + 3) / 4;
        router_logits_kernel<4, 1, 8><<<blocks, 256, 0, st>>>(x, wr, bias, T, H, E, logits);
    } else if (T <= 64) {
        waves = ((T + 7) / 8) * E;
        blocks = (waves + 3) / 4;
        router_logits_kernel<8, 1, 6><<<blocks, 256, 0, st>>>(x, wr, bias, T, H, E, logits);
    } else {
        waves = ((T + 7) / 8) * ((E + 7) / 8);
        blocks = (waves + 3) / 4;
        router_logits_kernel<8, 8, 2><<<blocks, 256, 0, st>>>(x, wr, bias, T, H, E, logits);
    }
}

// Top-k of one row per wave: experts ordered by (logit descending, id
// ascending); the first k in that order are the picks, in pick order.  The
// weights are the softmax over the picks ([P2] "GLM-5.3-Flash on CUDA:
// attention on one GPU, routed experts on the Sparks (proposal) #214", "Per
// MoE layer": rows travel with their top-k ids and weights).
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

// Top-k of one row per wave: experts ordered by (logit descending, id
// ascending); the first k in that order are the picks, in pick order.  The
// weights are the softmax over the picks ([P2] "GLM-5.3-Flash on CUDA:
// attention on one GPU, routed experts on the Sparks (proposal) #214", "Per
// MoE layer": rows travel with their top-k ids and weights).
template <int PER>
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ logits, int T,
                                                          int E, int k, int32_t* __restrict__ ids,
                                                          float* __restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
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
        }
    }
}

void launch_router_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                        hipStream_t st) {
    int blocks = (T + 3) / 4;
    int per = (E + 63) / 64;
    if (per <= 1)
        router_topk_kernel<1><<<blocks, 256, 0, st>>>(logits, T, E, k, ids, w);
    else if (per <= 2)
        router_topk_kernel<2><<<blocks, 256, 0, st>>>(logits, T, E, k, ids, w);
    else if (per <= 4)
        router_topk_kernel<4><<<blocks, 256, 0, st>>>(logits, T, E, k, ids, w);
    else if (per <= 8)
        router_topk_kernel<8><<<blocks, 256, 0, st>>>(logits, T, E, k, ids, w);
    else
        router_topk_kernel<16><<<blocks, 256, 0, st>>>(logits, T, E, k, ids, w);
}

}  // namespace moe
