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
#include "topk.h"

#pragma clang fp contract(off)

namespace moe {

// One wave computes a tile of RB rows x EB experts.
// The loads of BATCH steps of i are issued before any of them is used.
template <int RB, int EB, int BATCH>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ wr,
                                                            const float* __restrict__ bias,
                                                            int T, int H, int E,
                                                            float* __restrict__ logits) {
    const int lane = threadIdx.x & 63;
    // wave-uniform values live in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
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
            // wave-uniform row pointers plus an unsigned 32-bit lane offset:
            // scalar-base addressing, no 64-bit address arithmetic per load
            const uint32_t k0 = 256u * (uint32_t)i + 4u * (uint32_t)lane;
#pragma unroll
            for (int r = 0; r < RB; ++r)
                xu[b][r] = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(xp[r]) + 2u * k0);
#pragma unroll
            for (int e = 0; e < EB; ++e)
                wf[b][e] = *reinterpret_cast<const float4*>(reinterpret_cast<const char*>(wp[e]) + 4u * k0);
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
    // The xor rounds 1, 2, 4, .., 32 over the lane partials.  A few values:
    // by DPP moves and four row totals (wave_sum: after each round every lane
    // of a block of 2^j lanes holds the same value, so the DPP partner lane
    // of the pair, quad, half-row and row mirrors stands in for the xor
    // partner and the adds meet the same operands).  Many values: by
    // shuffles, which keep the many independent chains free of DPP wait
    // states.
    if constexpr (RB * EB <= 8) {
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int e = 0; e < EB; ++e) acc[r][e] = wave_sum(acc[r][e]);
    } else {
#pragma unroll
        for (int s = 1; s < 64; s <<= 1)
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int e = 0; e < EB; ++e) acc[r][e] = acc[r][e] + __shfl_xor(acc[r][e], s, 64);
    }

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

// RMSNorm of the rows before routing ([P2] "GLM-5.3-Flash on CUDA: attention
// on one GPU, routed experts on the Sparks (proposal) #214", "Per MoE layer":
// the expert side receives the normed rows; [P5] "What exists now": rmsnorm
// is a fixed-order fp32 glue kernel, and its first byte-gate run found the
// cross-lane total reaching only some lanes).  One wave per row: the sum of
// squares in the router's fixed order (lane l: fused multiply-adds over
// k = 256 i + 4 l + c, then the xor rounds, after which every lane holds the
// total), ms = ss / H, inv = 1 / sqrt(ms + eps) (correctly rounded division
// and square root), xn = bf16((x * inv) * gamma).
__device__ __forceinline__ uint2 rms_scale4(uint2 u, uint2 g, float inv) {
    const float v0 = (bf16_lo(u.x) * inv) * bf16_lo(g.x);
    const float v1 = (bf16_hi(u.x) * inv) * bf16_hi(g.x);
    const float v2 = (bf16_lo(u.y) * inv) * bf16_lo(g.y);
    const float v3 = (bf16_hi(u.y) * inv) * bf16_hi(g.y);
    uint2 o;
    o.x = (uint32_t)f32_to_bf16_bits(v0) | ((uint32_t)f32_to_bf16_bits(v1) << 16);
    o.y = (uint32_t)f32_to_bf16_bits(v2) | ((uint32_t)f32_to_bf16_bits(v3) << 16);
    return o;
}

__device__ __forceinline__ float rms_inv(float ss, int H, float eps) {
    const float ms = ss / (float)H;
    return 1.0f / __builtin_sqrtf(ms + eps);
}

// Rows of up to kRmsRegSteps * 256 values stay in registers: every load of
// the row and of the weight is issued at once (one memory round trip).
constexpr int kRmsRegSteps = 32;

__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ gamma, float eps,
                                                     int T, int H, uint16_t* __restrict__ xn) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const uint16_t* xr = x + (size_t)t * H;
    uint16_t* out = xn + (size_t)t * H;
    const int nI = H / 256;
    float p = 0.0f;
    if (nI <= kRmsRegSteps) {
        // static indices (guarded, no early exit) keep the arrays in registers
        uint2 u[kRmsRegSteps], g[kRmsRegSteps];
#pragma unroll
        for (int i = 0; i < kRmsRegSteps; ++i) {
            u[i] = make_uint2(0u, 0u);
            g[i] = make_uint2(0u, 0u);
            if (i < nI) {
                u[i] = *reinterpret_cast<const uint2*>(xr + 256 * i + 4 * lane);
                g[i] = *reinterpret_cast<const uint2*>(gamma + 256 * i + 4 * lane);
            }
        }
#pragma unroll
        for (int i = 0; i < kRmsRegSteps; ++i) {
            if (i < nI) {
                const float v0 = bf16_lo(u[i].x), v1 = bf16_hi(u[i].x), v2 = bf16_lo(u[i].y),
                            v3 = bf16_hi(u[i].y);
                p = __builtin_fmaf(v0, v0, p);
                p = __builtin_fmaf(v1, v1, p);
                p = __builtin_fmaf(v2, v2, p);
                p = __builtin_fmaf(v3, v3, p);
            }
        }
        p = wave_sum(p);  // the xor rounds, as in the router
        const float inv = rms_inv(p, H, eps);
#pragma unroll
        for (int i = 0; i < kRmsRegSteps; ++i)
            if (i < nI) *reinterpret_cast<uint2*>(out + 256 * i + 4 * lane) = rms_scale4(u[i], g[i], inv);
        return;
    }
    // longer rows: two passes, loads of 8 steps issued together
    constexpr int B = 8;
    for (int i0 = 0; i0 < nI; i0 += B) {
        uint2 u[B];
#pragma unroll
        for (int b = 0; b < B; ++b)
            u[b] = i0 + b < nI ? *reinterpret_cast<const uint2*>(xr + 256 * (i0 + b) + 4 * lane)
                               : make_uint2(0u, 0u);
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (i0 + b >= nI) break;
            const float v0 = bf16_lo(u[b].x), v1 = bf16_hi(u[b].x), v2 = bf16_lo(u[b].y),
                        v3 = bf16_hi(u[b].y);
            p = __builtin_fmaf(v0, v0, p);
            p = __builtin_fmaf(v1, v1, p);
            p = __builtin_fmaf(v2, v2, p);
            p = __builtin_fmaf(v3, v3, p);
        }
    }
    p = wave_sum(p);  // the xor rounds, as in the router
    const float inv = rms_inv(p, H, eps);
    for (int i = 0; i < nI; ++i) {
        const int c = 256 * i + 4 * lane;
        *reinterpret_cast<uint2*>(out + c) = rms_scale4(*reinterpret_cast<const uint2*>(xr + c),
                                                        *reinterpret_cast<const uint2*>(gamma + c), inv);
    }
}

void launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps, int T, int H, uint16_t* xn,
                    hipStream_t st) {
    rmsnorm_kernel<<<(T + 3) / 4, 256, 0, st>>>(x, gamma, eps, T, H, xn);
}

void launch_router_logits(const uint16_t* x, const float* wr, const float* bias, int T, int H,
                          int E, float* logits, hipStream_t st) {
    // Up to 64 rows: one wave per block, so the E (or a few times E) waves
    // spread over every CU; larger batches: four waves per block.  Up to 8
    // rows, a wave takes one or two rows and issues all 24 steps' loads of
    // H = 6144 at once (one memory round trip).
    if (T <= 1) {
        router_logits_kernel<1, 1, 24><<<E, 64, 0, st>>>(x, wr, bias, T, H, E, logits);
    } else if (T <= 8) {
        router_logits_kernel<2, 1, 24><<<((T + 1) / 2) * E, 64, 0, st>>>(x, wr, bias, T, H, E, logits);
    } else if (T <= 64) {
        router_logits_kernel<8, 1, 6><<<((T + 7) / 8) * E, 64, 0, st>>>(x, wr, bias, T, H, E, logits);
    } else {
        const int waves = ((T + 7) / 8) * ((E + 7) / 8);
        // one step's loads at a time: 131 registers and three waves per SIMD
        // either way, and the 8 x 8 tile's FMAs cover one step's latency
        // (prefill 280 -> 269 us against two steps; three steps 341 us)
        router_logits_kernel<8, 8, 1><<<(waves + 3) / 4, 256, 0, st>>>(x, wr, bias, T, H, E, logits);
    }
}

// Top-k of one row per wave (topk.h).
template <int PER>
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ logits,
                                                          const float* __restrict__ bias, int sigmoid,
                                                          int T, int E, int k, int32_t* __restrict__ ids,
                                                          float* __restrict__ w) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    topk_row<PER>(logits, bias, sigmoid, t, E, k, ids, w, nullptr);
}
void launch_router_topk(const float* logits, const float* bias, int sigmoid, int T, int E, int k,
                        int32_t* ids, float* w, hipStream_t st) {
    int blocks = (T + 3) / 4;
    int per = (E + 63) / 64;
    if (per <= 1)
        router_topk_kernel<1><<<blocks, 256, 0, st>>>(logits, bias, sigmoid, T, E, k, ids, w);
    else if (per <= 2)
        router_topk_kernel<2><<<blocks, 256, 0, st>>>(logits, bias, sigmoid, T, E, k, ids, w);
    else if (per <= 4)
        router_topk_kernel<4><<<blocks, 256, 0, st>>>(logits, bias, sigmoid, T, E, k, ids, w);
    else if (per <= 8)
        router_topk_kernel<8><<<blocks, 256, 0, st>>>(logits, bias, sigmoid, T, E, k, ids, w);
    else
        router_topk_kernel<16><<<blocks, 256, 0, st>>>(logits, bias, sigmoid, T, E, k, ids, w);
}

}  // namespace moe
