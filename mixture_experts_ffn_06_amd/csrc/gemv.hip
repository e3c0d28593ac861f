// gemv.hip -- bandwidth-bound expert projections for groups of 1..8 rows
// (decode): gate/up with the SwiGLU epilogue fused, then the down projection.
//
// [P1] "GLM-5.2 multi-GPU: expert-parallel sharding + the resident-fit
// benchmark", "Update (later 2026-06-29)": the per-expert expertSwiGLU;
// [P5] "GLM-5.3-Flash and full GLM-5.3 on the native CUDA engine (tracker)
// #593", "What exists now": fused gate/up rows are 2w wide (gate rows first
// here); "The pieces, in order": W4A16 (4-bit weights, 16-bit activations).
//
// Layout of the work: a block of 8 waves owns one work item (16 intermediate
// columns of one group for gate/up, 64 output columns for down) and keeps the
// group's rows (at most 8) in LDS.  A wave streams whole weight rows (every
// lane loads 16 contiguous bytes per step, so a step reads 1 KiB of one row),
// multiplies them with all rows of the group, and reduces across lanes once
// per weight row.  Work items are dealt to the blocks round-robin.
//
// 4-bit weights: (code - zero) * scale with (scale, zero) per 32 inputs.  One
// lane step covers exactly one 32-input group: the codes are widened to the
// bf16 values 128 + code with two bit operations per pair, dotted with the
// rows (inputs stored pairwise-permuted in LDS to match the nibble order), and
// the group contributes scale * (dot - (128 + zero) * sum(inputs)).  MLX
// affine (scale * code + bias per 64 inputs) takes the same widening: a lane
// step is half a group and contributes scale * (dot - 128 * sum) + bias * sum.
// NVFP4 (E2M1 codes, an E4M3 scale per 16 inputs, an fp32 scale per matrix):
// the hardware conversion turns two codes at a time into exact bf16 values,
// dotted with the rows in their plain order; each 16-input block adds its
// scale times its dot, and the matrix scale multiplies the finished sum.
#include "common.h"

#include <type_traits>

namespace moe {

constexpr int kGemvThreads = 512;
constexpr int kGemvWaves = kGemvThreads / 64;

// 4-bit layout of a staged row: the 32 inputs of group g (read by one lane
// of a 4-bit lane step, lane = g mod 64) are four 16-byte chunks, chunk d
// stored at position (d + lane / 2) mod 4 of the group, so the eight lanes
// of a 128-byte LDS access meet eight different bank groups.
__device__ __forceinline__ int w4_chunk(int g, int d) { return (d + ((g & 63) >> 1)) & 3; }

// Stage the rows of a group in LDS.  src_h: rows come from the intermediate
// h (down projection), else from x (gate/up).  permute: store each 8 inputs as
// (0,4),(1,5),(2,6),(3,7) pairs and the per-32 sums (4-bit path).
__device__ void stage_rows(const ExpertArgs& a, const Group& g, bool src_h, int K, int nr,
                           bool permute, uint16_t* xs, float* xsum) {
    const bool shared = g.expert < 0;
    const int c8n = K / 8;
    for (int idx = threadIdx.x; idx < nr * c8n; idx += blockDim.x) {
        const int r = idx / c8n, c8 = idx - r * c8n;
        const uint16_t* src;
        if (src_h)
            src = shared ? a.h_s + (size_t)r * a.Is : a.h_r + (size_t)(g.row0 + r) * a.I;
        else
            src = a.x + (size_t)(shared ? r : a.perm[g.row0 + r] / a.topk) * a.H;
        uint4 v = *reinterpret_cast<const uint4*>(src + 8 * c8);
        int dst = c8;
        if (permute) {
            uint4 p;
            p.x = (v.x & 0xffffu) | (v.z << 16);
            p.y = (v.x >> 16) | (v.z & 0xffff0000u);
            p.z = (v.y & 0xffffu) | (v.w << 16);
            p.w = (v.y >> 16) | (v.w & 0xffff0000u);
            v = p;
            dst = (c8 & ~3) | w4_chunk(c8 >> 2, c8 & 3);
        }
        *reinterpret_cast<uint4*>(xs + (size_t)r * K + 8 * dst) = v;
    }
    if (permute) {
        // per-32 sums, from the staged copy (a fixed order over its 32 values)
        __syncthreads();
        const int gn = K / 32;
        for (int idx = threadIdx.x; idx < nr * gn; idx += blockDim.x) {
            const int r = idx / gn, gi = idx - r * gn;
            const uint4* src = reinterpret_cast<const uint4*>(xs + (size_t)r * K + 32 * gi);
            float s = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint4 v = src[w4_chunk(gi, q)];
                s += bf16_lo(v.x) + bf16_hi(v.x);
                s += bf16_lo(v.y) + bf16_hi(v.y);
                s += bf16_lo(v.z) + bf16_hi(v.z);
                s += bf16_lo(v.w) + bf16_hi(v.w);
            }
            xsum[r * gn + gi] = s;
        }
    }
}

// ---- dot helpers ---------------------------------------------------------

// bf16 weights: 8 inputs per lane step.
template <int NR>
__device__ __forceinline__ void dot_step_bf16(const uint4& w, const uint16_t* xs, int K, int k,
                                              float* acc) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        uint4 xv = *reinterpret_cast<const uint4*>(xs + r * K + k);
        float s = acc[r];
        s = dot2_bf16(w.x, xv.x, s);
        s = dot2_bf16(w.y, xv.y, s);
        s = dot2_bf16(w.z, xv.z, s);
        s = dot2_bf16(w.w, xv.w, s);
        acc[r] = s;
    }
}

// (x & m) | k in one instruction (the compiler emits an AND and an OR: a
// VOP3 takes no literal, and only one scalar operand, so k sits in a VGPR).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t k) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(k));
    return r;
}

// 4-bit weights: 32 inputs (one group) per lane step.
template <int NR>
__device__ __forceinline__ void dot_step_w4(const uint4& q, float sc, float zz, const uint16_t* xs,
                                            const float* xsum, int K, int k, float* acc) {
    uint32_t qd[4] = {q.x, q.y, q.z, q.w};
    float part[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) part[r] = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t c = qd[d];
        const uint32_t p0 = and_or(c, 0x000f000fu, 0x43004300u);
        const uint32_t p1 = and_or(c >> 4, 0x000f000fu, 0x43004300u);
        const uint32_t p2 = and_or(c >> 8, 0x000f000fu, 0x43004300u);
        const uint32_t p3 = and_or(c >> 12, 0x000f000fu, 0x43004300u);
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            uint4 xv = *reinterpret_cast<const uint4*>(xs + r * K + k + 8 * w4_chunk(k >> 5, d));
            float s = part[r];
            s = dot2_bf16(p0, xv.x, s);
            s = dot2_bf16(p1, xv.y, s);
            s = dot2_bf16(p2, xv.z, s);
            s = dot2_bf16(p3, xv.w, s);
            part[r] = s;
        }
    }
    const float z128 = 128.0f + zz;
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] += sc * (part[r] - z128 * xsum[r * (K / 32) + k / 32]);
}

// MLX affine 4-bit: 32 inputs (half a 64-input group) per lane step; same
// widening and LDS layout as dot_step_w4.
template <int NR>
__device__ __forceinline__ void dot_step_affine(const uint4& q, float sc, float bias, const uint16_t* xs,
                                                const float* xsum, int K, int k, float* acc) {
    uint32_t qd[4] = {q.x, q.y, q.z, q.w};
    float part[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) part[r] = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t c = qd[d];
        const uint32_t p0 = and_or(c, 0x000f000fu, 0x43004300u);
        const uint32_t p1 = and_or(c >> 4, 0x000f000fu, 0x43004300u);
        const uint32_t p2 = and_or(c >> 8, 0x000f000fu, 0x43004300u);
        const uint32_t p3 = and_or(c >> 12, 0x000f000fu, 0x43004300u);
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            uint4 xv = *reinterpret_cast<const uint4*>(xs + r * K + k + 8 * w4_chunk(k >> 5, d));
            float s = part[r];
            s = dot2_bf16(p0, xv.x, s);
            s = dot2_bf16(p1, xv.y, s);
            s = dot2_bf16(p2, xv.z, s);
            s = dot2_bf16(p3, xv.w, s);
            part[r] = s;
        }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const float X = xsum[r * (K / 32) + k / 32];
        acc[r] += fmaf(sc, part[r] - 128.0f * X, bias * X);
    }
}

// Two E2M1 codes (byte B of c) -> two exact bf16 values, in input order.
template <int B>
__device__ __forceinline__ uint32_t fp4x2_bf16(uint32_t c) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, B));
}

// NVFP4: 32 inputs (two 16-input blocks, scales s0 and s1) per lane step; the
// rows in LDS in their plain order.
template <int NR>
__device__ __forceinline__ void dot_step_nv(const uint4& q, float s0, float s1, const uint16_t* xs, int K,
                                            int k, float* acc) {
    const uint32_t qd[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        float part[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) part[r] = 0.0f;
#pragma unroll
        for (int dd = 0; dd < 2; ++dd) {
            const int d = 2 * blk + dd;
            const uint32_t c = qd[d];
            const uint32_t p0 = fp4x2_bf16<0>(c), p1 = fp4x2_bf16<1>(c);
            const uint32_t p2 = fp4x2_bf16<2>(c), p3 = fp4x2_bf16<3>(c);
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const uint4 xv = *reinterpret_cast<const uint4*>(xs + r * K + k + 8 * d);
                float s = part[r];
                s = dot2_bf16(p0, xv.x, s);
                s = dot2_bf16(p1, xv.y, s);
                s = dot2_bf16(p2, xv.z, s);
                s = dot2_bf16(p3, xv.w, s);
                part[r] = s;
            }
        }
        const float sc = blk ? s1 : s0;
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[r] = fmaf(sc, part[r], acc[r]);
    }
}

// Per-group arrays of row `row` (of K inputs) at lane step k: W4A16 (scale,
// zero) and MLX affine (scale, bias) as bf16 bits; NVFP4 the two E4M3 bytes
// of the step's blocks in s.
template <int FMT>
__device__ __forceinline__ void load_scales(const uint16_t* sb, const uint16_t* zb, size_t row, int K, int k,
                                            uint32_t* s, uint32_t* z) {
    if constexpr (FMT == 1) {
        *s = sb[row * (K / 32) + k / 32];
        *z = zb[row * (K / 32) + k / 32];
    } else if constexpr (FMT == 2) {
        *s = sb[row * (K / 64) + k / 64];
        *z = zb[row * (K / 64) + k / 64];
    } else {
        *s = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(sb) + row * (K / 16) + k / 16);
        *z = 0;
    }
}

// One 32-input lane step of a 4-bit format; !ok (a step past the row) adds
// nothing.
template <int FMT, int NR>
__device__ __forceinline__ void quant_step(const uint4& q, uint32_t s, uint32_t z, bool ok, const uint16_t* xs,
                                           const float* xsum, int K, int k, float* acc) {
    if constexpr (FMT == 1) {
        dot_step_w4<NR>(q, ok ? bf16_bits_to_f32(s) : 0.0f, bf16_bits_to_f32(z), xs, xsum, K, k, acc);
    } else if constexpr (FMT == 2) {
        dot_step_affine<NR>(q, ok ? bf16_bits_to_f32(s) : 0.0f, ok ? bf16_bits_to_f32(z) : 0.0f, xs, xsum, K, k,
                            acc);
    } else {
        // (converted unconditionally: a conversion under the condition would
        // become a branch)
        const float f0 = __builtin_amdgcn_cvt_f32_fp8(s, 0), f1 = __builtin_amdgcn_cvt_f32_fp8(s, 1);
        dot_step_nv<NR>(q, ok ? f0 : 0.0f, ok ? f1 : 0.0f, xs, K, k, acc);
    }
}

// ---- gate/up ---------------------------------------------------------------

// One work item: intermediate columns c0 .. c0+15 of group g; wave w owns
// columns c0 + 2w and c0 + 2w + 1 (its gate row and its up row each).
// Loads are never predicated: a lane step past the end of the row reloads the
// row's first chunk and its weights are zeroed, so every load of a block is in
// flight at once (a predicated load would make the compiler wait for the
// previous one).  CB = lane steps per block (bf16: 512 inputs per step).
template <int FMT, int NR, int CB>
__device__ void gateup_item(const ExpertArgs& a, const Group& g, int c0, const uint16_t* xs,
                            const float* xsum) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool shared = g.expert < 0;
    const int Ig = shared ? a.Is : a.I;
    const int H = a.H;
    for (int cc = 0; cc < 2; ++cc) {
        const int c = c0 + 2 * wave + cc;
        float ag[NR], au[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) ag[r] = au[r] = 0.0f;
        if (FMT == 0) {
            const uint16_t* gr = shared ? a.swgu + (size_t)c * H
                                        : a.wgu + ((size_t)g.expert * 2 * Ig + c) * H;
            const uint16_t* ur = gr + (size_t)Ig * H;
            const int nch = (H + 511) / 512;
            for (int q0 = 0; q0 < nch; q0 += CB) {
                uint4 wg[CB], wu[CB];
                int kk[CB];
                bool ok[CB];
#pragma unroll
                for (int qq = 0; qq < CB; ++qq) {
                    const int k = 512 * (q0 + qq) + 8 * lane;
                    ok[qq] = (q0 + qq < nch) && (k < H);
                    kk[qq] = ok[qq] ? k : 0;
                    wg[qq] = wload(gr + kk[qq]);
                    wu[qq] = wload(ur + kk[qq]);
                }
#pragma unroll
                for (int qq = 0; qq < CB; ++qq) {
                    const uint4 z = make_uint4(0, 0, 0, 0);
                    dot_step_bf16<NR>(ok[qq] ? wg[qq] : z, xs, H, kk[qq], ag);
                    dot_step_bf16<NR>(ok[qq] ? wu[qq] : z, xs, H, kk[qq], au);
                }
            }
        } else {
            const size_t grow = (size_t)g.expert * 2 * Ig + c, urow = grow + Ig;
            const uint8_t* gq = a.qgu + grow * (H / 2);
            const uint8_t* uq = a.qgu + urow * (H / 2);
            constexpr int CB4 = 3;
            const int nch = (H + 2047) / 2048;
            for (int q0 = 0; q0 < nch; q0 += CB4) {
                uint4 qg[CB4], qu[CB4];
                uint32_t sg[CB4], zg[CB4], su[CB4], zu[CB4];
                int kk[CB4];
                bool ok[CB4];
#pragma unroll
                for (int qq = 0; qq < CB4; ++qq) {
                    const int k = 2048 * (q0 + qq) + 32 * lane;
                    ok[qq] = (q0 + qq < nch) && (k < H);
                    kk[qq] = ok[qq] ? k : 0;
                    qg[qq] = wload(gq + kk[qq] / 2);
                    qu[qq] = wload(uq + kk[qq] / 2);
                    load_scales<FMT>(a.sgu, a.zgu, grow, H, kk[qq], &sg[qq], &zg[qq]);
                    load_scales<FMT>(a.sgu, a.zgu, urow, H, kk[qq], &su[qq], &zu[qq]);
                }
#pragma unroll
                for (int qq = 0; qq < CB4; ++qq) {
                    quant_step<FMT, NR>(qg[qq], sg[qq], zg[qq], ok[qq], xs, xsum, H, kk[qq], ag);
                    quant_step<FMT, NR>(qu[qq], su[qq], zu[qq], ok[qq], xs, xsum, H, kk[qq], au);
                }
            }
        }
        // NVFP4: the gate and up matrix scales multiply the finished sums
        float mg = 1.0f, mu = 1.0f;
        if (FMT == 3 && !shared) {
            mg = a.ggu[2 * (size_t)g.expert];
            mu = a.ggu[2 * (size_t)g.expert + 1];
        }
        uint16_t* hout = shared ? a.h_s : a.h_r + (size_t)g.row0 * a.I;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            float gs_ = wave_sum(ag[r]);
            float us_ = wave_sum(au[r]);
            if (FMT == 3) {
                gs_ *= mg;
                us_ *= mu;
            }
            if (lane == r) hout[(size_t)r * Ig + c] = f32_to_bf16_bits(silu_mul(gs_, us_));
        }
    }
}

// MAXNR: the most rows a group of the launch has (1 at T = 1: the one-row
// kernels need fewer registers, so two or three blocks fit on a CU).
template <int FMT, int CB, int MAXNR>
__device__ __forceinline__ void gateup_dispatch_rows(const ExpertArgs& a, const Group& g, int c0,
                                                     const uint16_t* xs, const float* xsum) {
    if constexpr (MAXNR == 1) {
        gateup_item<FMT, 1, CB>(a, g, c0, xs, xsum);
        return;
    }
    switch (g.n) {
        case 1: gateup_item<FMT, 1, CB>(a, g, c0, xs, xsum); break;
        case 2: gateup_item<FMT, 2, CB>(a, g, c0, xs, xsum); break;
        case 3: gateup_item<FMT, 3, CB>(a, g, c0, xs, xsum); break;
        case 4: gateup_item<FMT, 4, CB>(a, g, c0, xs, xsum); break;
        case 5: gateup_item<FMT, 5, CB>(a, g, c0, xs, xsum); break;
        case 6: gateup_item<FMT, 6, CB>(a, g, c0, xs, xsum); break;
        case 7: gateup_item<FMT, 7, CB>(a, g, c0, xs, xsum); break;
        default: gateup_item<FMT, 8, CB>(a, g, c0, xs, xsum); break;
    }
}

// ---- overlapped path: bf16 groups of 1 or 2 rows (the decode case) --------
//
// A work item's critical path used to be: group descriptor -> row tokens ->
// rows into LDS -> barrier -> weight loads.  Here the next item's descriptor
// and tokens are fetched during the current item, and the rows of a new group
// are loaded into registers before the item's weight loads are issued and
// written to one of two LDS buffers while those loads are in flight (a plain
// s_barrier, not __syncthreads, whose fence would wait for them).  The two
// buffers alternate per staging, so a block needs no barrier before writing
// the next group's rows: the previous staging's barrier already ordered every
// read of the buffer being replaced.

struct ItemMeta {
    Group g;
    int gi, tile, tok0, tok1;
};

__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

__device__ __forceinline__ ItemMeta load_meta(const ExpertArgs& a, int it, int nrouted, int TR);

// Returns the next item's descriptor (fetched once this item's first loads are
// in flight), or this item's when there is no next one.
template <int NR, int CB>
__device__ ItemMeta gateup_fast(const ExpertArgs& a, const ItemMeta& m, bool restage, uint16_t* xb,
                                bool has_next, int itn, int nrouted, int TR) {
    ItemMeta mn = m;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const Group& g = m.g;
    const bool shared = g.expert < 0;
    const int Ig = shared ? a.Is : a.I;
    const int H = a.H;
    const int c8n = H / 8;
    const int nchunk = NR * c8n;  // <= 4 * kGemvThreads (checked by the caller)
    // up to four 16-byte chunks of the rows per thread, in named registers
    auto xchunk = [&](int i) -> uint4 {
        const int idx = min(tid + kGemvThreads * i, nchunk - 1);
        const int r = idx / c8n, c8 = idx - r * c8n;
        return *reinterpret_cast<const uint4*>(a.x + (size_t)(r ? m.tok1 : m.tok0) * H + 8 * c8);
    };
    auto xput = [&](int i, const uint4& v) {
        const int idx = tid + kGemvThreads * i;
        if (idx < nchunk) {
            const int r = idx / c8n, c8 = idx - r * c8n;
            *reinterpret_cast<uint4*>(xb + (size_t)r * H + 8 * c8) = v;
        }
    };
    uint4 x0, x1, x2, x3;
    if (restage) {
        x0 = xchunk(0);
        x1 = xchunk(1);
        x2 = xchunk(2);
        x3 = xchunk(3);
    }
    // H = 512 CB exactly (checked by the caller): whole rows in one block of
    // loads, no clamping, no selects
    uint16_t* hout = shared ? a.h_s : a.h_r + (size_t)g.row0 * a.I;
    const uint16_t* xl = xb + 8 * lane;
#pragma nounroll
    for (int cc = 0; cc < 2; ++cc) {
        const int c = m.tile * kGuCols + 2 * wave + cc;
        const uint16_t* gr = (shared ? a.swgu + (size_t)c * H : a.wgu + ((size_t)g.expert * 2 * Ig + c) * H) + 8 * lane;
        const uint16_t* ur = gr + (size_t)Ig * H;
        uint4 wg[CB], wu[CB];
#pragma unroll
        for (int q = 0; q < CB; ++q) {
            wg[q] = wload(gr + 512 * q);
            wu[q] = wload(ur + 512 * q);
        }
        if (cc == 0) {
            if (has_next) mn = load_meta(a, itn, nrouted, TR);
            if (restage) {
                xput(0, x0);
                xput(1, x1);
                xput(2, x2);
                xput(3, x3);
                wait_lgkm0();
                __builtin_amdgcn_s_barrier();
            }
        }
        float ag[NR], au[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) ag[r] = au[r] = 0.0f;
#pragma unroll
        for (int q = 0; q < CB; ++q) {
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const uint4 xv = *reinterpret_cast<const uint4*>(xl + r * H + 512 * q);
                float sg = ag[r], su = au[r];
                sg = dot2_bf16(wg[q].x, xv.x, sg);
                sg = dot2_bf16(wg[q].y, xv.y, sg);
                sg = dot2_bf16(wg[q].z, xv.z, sg);
                sg = dot2_bf16(wg[q].w, xv.w, sg);
                su = dot2_bf16(wu[q].x, xv.x, su);
                su = dot2_bf16(wu[q].y, xv.y, su);
                su = dot2_bf16(wu[q].z, xv.z, su);
                su = dot2_bf16(wu[q].w, xv.w, su);
                ag[r] = sg;
                au[r] = su;
            }
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const float gs_ = wave_sum(ag[r]);
            const float us_ = wave_sum(au[r]);
            if (lane == r) hout[(size_t)r * Ig + c] = f32_to_bf16_bits(silu_mul(gs_, us_));
        }
    }
    return mn;
}

__device__ __forceinline__ ItemMeta load_meta(const ExpertArgs& a, int it, int nrouted, int TR) {
    ItemMeta m;
    if (it < nrouted * TR) {
        m.gi = it / TR;
        m.tile = it - m.gi * TR;
    } else {
        m.gi = nrouted;
        m.tile = it - nrouted * TR;
    }
    m.g = a.groups[a.gemv_list[m.gi]];
    const bool sh = m.g.expert < 0;
    m.tok0 = sh ? 0 : a.perm[m.g.row0] / a.topk;
    m.tok1 = sh ? 1 : (m.g.n > 1 ? a.perm[m.g.row0 + 1] / a.topk : m.tok0);
    return m;
}

// Work items: every GEMV group (routed groups first, the shared expert last
// when it is on this path) times its column tiles.
__device__ __forceinline__ void item_of(const ExpertArgs& a, int it, int nrouted, int TR,
                                        int* gi, int* tile) {
    if (it < nrouted * TR) {
        *gi = it / TR;
        *tile = it - *gi * TR;
    } else {
        *gi = nrouted;
        *tile = it - nrouted * TR;
    }
}

// FMT: the routed experts' format (0 bf16, 1 W4A16, 2 MLX affine, 3 NVFP4);
// the shared expert is bf16 in every format.
// Launch bounds of the one-row kernels, in waves per SIMD: 6 (at most 80
// registers, three blocks per CU) where that needs no spills -- the 4-bit down
// kernels and the NVFP4 gate/up kernel -- else 4 (two blocks per CU; W4A16 and
// MLX affine gate/up items hold a scale and a zero or bias per step and row).
constexpr int one_row_waves(int fmt, bool gateup) { return fmt == 0 ? 4 : (gateup && fmt != 3 ? 4 : 6); }

template <int FMT, int CB, int MAXNR>
__global__ __launch_bounds__(kGemvThreads, MAXNR == 1 ? one_row_waves(FMT, true) : 1) void gateup_gemv_kernel(ExpertArgs a, int lds_rows) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
    float* xsum = reinterpret_cast<float*>(smem + (size_t)lds_rows * a.H * 2);
    const int ngv = a.plan_counts[0];
    if (ngv == 0) return;
    const bool sh_last = a.groups[a.gemv_list[ngv - 1]].expert < 0;
    const int nrouted = ngv - (sh_last ? 1 : 0);
    const int TR = a.I / kGuCols, TS = sh_last && !a.shared_gu_done ? a.Is / kGuCols : 0;
    const int total = nrouted * TR + TS;
    // Items are dealt round-robin: at any moment the blocks stream neighbouring
    // column tiles of the same experts, so HBM sees a few long sequential runs
    // rather than one run per block.
    int it = blockIdx.x;
    if (it >= total) return;
    const bool fast_ok = 2 * (a.H / 8) <= 4 * kGemvThreads && a.H == 512 * CB;
    ItemMeta m = load_meta(a, it, nrouted, TR);
    int cur = -1, buf = 0;
    // the one row staged by the synchronous path (2 token + 4-bit layout), or
    // -1: one-row groups of the same token (every group when T = 1) reuse it
    int staged = -1;
    for (;;) {
        const int itn = it + gridDim.x;
        const bool has_next = itn < total;
        ItemMeta mn = m;
        const Group& g = m.g;
        const bool w4 = FMT != 0 && g.expert >= 0;
        // the 4-bit layout of staged rows (pairwise-permuted, with per-32
        // sums) for W4A16 and MLX affine; NVFP4 reads them in plain order
        const bool perm = w4 && FMT != 3;
        if (!w4 && g.n <= 2 && fast_ok) {
            const bool restage = m.gi != cur;
            if (restage) buf ^= 1;
            uint16_t* xb = xs + (size_t)buf * 2 * a.H;
            if (MAXNR == 1 || g.n == 1)
                mn = gateup_fast<1, CB>(a, m, restage, xb, has_next, itn, nrouted, TR);
            else if constexpr (MAXNR > 1)
                mn = gateup_fast<2, CB>(a, m, restage, xb, has_next, itn, nrouted, TR);
            cur = m.gi;
            staged = -1;  // its buffers overlap the synchronous staging area
        } else {
            // rows staged synchronously across the whole LDS area
            const int key = g.n == 1 ? 2 * m.tok0 + (perm ? 1 : 0) : -1;
            if (key < 0 || key != staged) {
                __syncthreads();  // a fast-path item before may still read its buffer
                stage_rows(a, g, false, a.H, g.n, perm, xs, xsum);
                __syncthreads();
                staged = key;
            }
            if (has_next) mn = load_meta(a, itn, nrouted, TR);
            if (w4)
                gateup_dispatch_rows<FMT, CB, MAXNR>(a, g, m.tile * kGuCols, xs, xsum);
            else
                gateup_dispatch_rows<0, CB, MAXNR>(a, g, m.tile * kGuCols, xs, xsum);
            // The next item overwrites these rows only if it stages others
            // (or takes the fast path, whose buffers overlap them); one-row
            // groups of the same token and format keep them, and need no
            // barrier (every 4-bit item at T = 1).
            const bool w4n = FMT != 0 && mn.g.expert >= 0;
            const bool keeps = has_next && mn.g.n == 1 && key >= 0 &&
                               2 * mn.tok0 + (w4n && FMT != 3 ? 1 : 0) == key &&
                               !(!w4n && mn.g.n <= 2 && fast_ok);
            if (!keeps) __syncthreads();
            cur = -1;
        }
        if (!has_next) break;
        it = itn;
        m = mn;
    }
}

// ---- down ------------------------------------------------------------------

// One work item: output columns n0 .. n0+63 of group g; wave w owns 8 of them,
// streamed as passes of UP rows of the down weight (UP = 4: 16 loads in
// flight for a bf16 row of K = 2048; each column's arithmetic is the same
// whatever UP).
template <int FMT, int NR, int UP = 4>
__device__ void down_item(const ExpertArgs& a, const Group& g, int n0, const uint16_t* xs,
                          const float* xsum) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool shared = g.expert < 0;
    const int K = shared ? a.Is : a.I;
    const int H = a.H;
    constexpr int U = UP;
    constexpr int CW = kDnCols / kGemvWaves;  // columns per wave
    for (int pass = 0; pass < CW / U; ++pass) {
    const int cbase = n0 + CW * wave + U * pass;
    float acc[U][NR];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[u][r] = 0.0f;
    if (FMT == 0 && K == 512 * 4) {
        // rows of exactly 4 lane steps (K = 2048): no clamping, no selects
        const uint16_t* wrow = (shared ? a.swd : a.wd + (size_t)g.expert * H * K) + (size_t)cbase * K + 8 * lane;
        const uint16_t* xl = xs + 8 * lane;
        uint4 wv[U][4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int u = 0; u < U; ++u) wv[u][q] = wload(wrow + (size_t)u * K + 512 * q);
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const uint4 xv = *reinterpret_cast<const uint4*>(xl + r * K + 512 * q);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    float t = acc[u][r];
                    t = dot2_bf16(wv[u][q].x, xv.x, t);
                    t = dot2_bf16(wv[u][q].y, xv.y, t);
                    t = dot2_bf16(wv[u][q].z, xv.z, t);
                    t = dot2_bf16(wv[u][q].w, xv.w, t);
                    acc[u][r] = t;
                }
            }
    } else if (FMT == 0) {
        const uint16_t* wbase = shared ? a.swd : a.wd + (size_t)g.expert * H * K;
        constexpr int CB = 4;
        const int nch = (K + 511) / 512;
        for (int q0 = 0; q0 < nch; q0 += CB) {
            uint4 wv[U][CB];
            int kk[CB];
            bool ok[CB];
#pragma unroll
            for (int qq = 0; qq < CB; ++qq) {
                const int k = 512 * (q0 + qq) + 8 * lane;
                ok[qq] = (q0 + qq < nch) && (k < K);
                kk[qq] = ok[qq] ? k : 0;
#pragma unroll
                for (int u = 0; u < U; ++u)
                    wv[u][qq] = wload(wbase + (size_t)(cbase + u) * K + kk[qq]);
            }
#pragma unroll
            for (int qq = 0; qq < CB; ++qq) {
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    uint4 xv = *reinterpret_cast<const uint4*>(xs + r * K + kk[qq]);
                    if (!ok[qq]) xv = make_uint4(0, 0, 0, 0);
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        float s = acc[u][r];
                        s = dot2_bf16(wv[u][qq].x, xv.x, s);
                        s = dot2_bf16(wv[u][qq].y, xv.y, s);
                        s = dot2_bf16(wv[u][qq].z, xv.z, s);
                        s = dot2_bf16(wv[u][qq].w, xv.w, s);
                        acc[u][r] = s;
                    }
                }
            }
        }
    } else {
        const size_t rbase = (size_t)g.expert * H;
        const int nch = (K + 2047) / 2048;
        for (int q = 0; q < nch; ++q) {
            uint4 qv[U];
            uint32_t sv[U], zv[U];
            const int k = 2048 * q + 32 * lane;
            const bool ok = k < K;
            const int kq = ok ? k : 0;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const size_t row = rbase + cbase + u;
                qv[u] = wload(a.qd + row * (K / 2) + kq / 2);
                load_scales<FMT>(a.sd, a.zd, row, K, kq, &sv[u], &zv[u]);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) quant_step<FMT, NR>(qv[u], sv[u], zv[u], ok, xs, xsum, K, kq, acc[u]);
        }
    }
    // NVFP4: the down matrix scale multiplies the finished sums
    const float md = FMT == 3 && !shared ? a.gd[g.expert] : 1.0f;
    float* yout = shared ? a.y_s : a.y_r + (size_t)g.row0 * H;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            float v = wave_sum(acc[u][r]);
            if (FMT == 3) v *= md;
            if (lane == ((u * NR + r) & 63)) yout[(size_t)r * H + cbase + u] = v;
        }
    }
}

// A bf16 item of a group of one or two rows with K = 2048 (every routed
// group at decode): the group's rows, when they change, are read into
// registers and written to LDS buffer xb (one of two, alternating) after the
// first pass's weight loads are issued, so the row fetch and the barrier
// overlap the weight stream.  Same per-column order as down_item.
template <int NR>
__device__ void down_fast(const ExpertArgs& a, const Group& g, int n0, bool restage, uint16_t* xb) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool shared = g.expert < 0;
    constexpr int K = 512 * 4;
    constexpr int c8n = K / 8;
    static_assert(NR * c8n <= kGemvThreads, "one 16-byte chunk of the rows per thread");
    const int H = a.H;
    constexpr int U = kDnCols / kGemvWaves / 2;
    uint4 xc = make_uint4(0, 0, 0, 0);
    const int r_ = tid / c8n, c8 = tid - r_ * c8n;
    if (restage && tid < NR * c8n) {
        const uint16_t* src = shared ? a.h_s + (size_t)r_ * K : a.h_r + (size_t)(g.row0 + r_) * K;
        xc = *reinterpret_cast<const uint4*>(src + 8 * c8);
    }
    const uint16_t* xl = xb + 8 * lane;
#pragma nounroll
    for (int pass = 0; pass < 2; ++pass) {
        const int cbase = n0 + 2 * U * wave + U * pass;
        const uint16_t* wrow = (shared ? a.swd : a.wd + (size_t)g.expert * H * K) + (size_t)cbase * K + 8 * lane;
        uint4 wv[U][4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int u = 0; u < U; ++u) wv[u][q] = wload(wrow + (size_t)u * K + 512 * q);
        if (pass == 0 && restage) {
            if (tid < NR * c8n) *reinterpret_cast<uint4*>(xb + (size_t)r_ * K + 8 * c8) = xc;
            wait_lgkm0();
            __builtin_amdgcn_s_barrier();
        }
        float acc[U][NR];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < NR; ++r) acc[u][r] = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const uint4 xv = *reinterpret_cast<const uint4*>(xl + r * K + 512 * q);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    float t = acc[u][r];
                    t = dot2_bf16(wv[u][q].x, xv.x, t);
                    t = dot2_bf16(wv[u][q].y, xv.y, t);
                    t = dot2_bf16(wv[u][q].z, xv.z, t);
                    t = dot2_bf16(wv[u][q].w, xv.w, t);
                    acc[u][r] = t;
                }
            }
        float* yout = shared ? a.y_s : a.y_r + (size_t)g.row0 * H;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const float v = wave_sum(acc[u][r]);
                if (lane == ((u * NR + r) & 63)) yout[(size_t)r * H + cbase + u] = v;
            }
    }
}

template <int FMT, int MAXNR>
__device__ __forceinline__ void down_dispatch_rows(const ExpertArgs& a, const Group& g, int n0,
                                                   const uint16_t* xs, const float* xsum) {
    if constexpr (MAXNR == 1) {
        down_item<FMT, 1, FMT == 0 ? 2 : 4>(a, g, n0, xs, xsum);
        return;
    }
    switch (g.n) {
        case 1: down_item<FMT, 1>(a, g, n0, xs, xsum); break;
        case 2: down_item<FMT, 2>(a, g, n0, xs, xsum); break;
        case 3: down_item<FMT, 3>(a, g, n0, xs, xsum); break;
        case 4: down_item<FMT, 4>(a, g, n0, xs, xsum); break;
        case 5: down_item<FMT, 5>(a, g, n0, xs, xsum); break;
        case 6: down_item<FMT, 6>(a, g, n0, xs, xsum); break;
        case 7: down_item<FMT, 7>(a, g, n0, xs, xsum); break;
        default: down_item<FMT, 8>(a, g, n0, xs, xsum); break;
    }
}

template <int FMT, int MAXNR>
__global__ __launch_bounds__(kGemvThreads, MAXNR == 1 ? one_row_waves(FMT, false) : 1) void down_gemv_kernel(ExpertArgs a, int lds_rows,
                                                                                    int kmax) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
    float* xsum = reinterpret_cast<float*>(smem + (size_t)lds_rows * kmax * 2);
    const int ngv = a.plan_counts[0];
    if (ngv == 0) return;
    const bool sh_last = a.groups[a.gemv_list[ngv - 1]].expert < 0;
    const int nrouted = ngv - (sh_last ? 1 : 0);
    const int TR = a.H / kDnCols;
    const int total = (nrouted + (sh_last ? 1 : 0)) * TR;
    // fcur: the group in the current fast-path buffer; scur: the group staged
    // across the LDS area by the synchronous path (which overlaps the fast
    // path's buffers, so each path forgets the other's rows)
    int fcur = -1, scur = -1, buf = 0;
    bool prev_slow = false;
    for (int it = blockIdx.x; it < total; it += gridDim.x) {
        const int gi = it / TR, tile = it - gi * TR;
        const Group g = a.groups[a.gemv_list[gi]];
        const bool w4 = FMT != 0 && g.expert >= 0;
        const int K = g.expert < 0 ? a.Is : a.I;
        // (not in the 4-bit kernels: their registers would spill)
        if (FMT == 0 && g.n <= 2 && K == 512 * 4) {
            if (prev_slow) __syncthreads();  // the synchronous item's LDS reads are done
            const bool restage = gi != fcur;
            if (restage) buf ^= 1;
            uint16_t* xb = xs + (size_t)buf * 2 * K;
            if (MAXNR == 1 || g.n == 1)
                down_fast<1>(a, g, tile * kDnCols, restage, xb);
            else if constexpr (MAXNR > 1)
                down_fast<2>(a, g, tile * kDnCols, restage, xb);
            fcur = gi;
            scur = -1;
            prev_slow = false;
            continue;
        }
        if (gi != scur) {
            __syncthreads();
            stage_rows(a, g, true, K, g.n, w4 && FMT != 3, xs, xsum);
            __syncthreads();
            scur = gi;
        }
        if (w4)
            down_dispatch_rows<FMT, MAXNR>(a, g, tile * kDnCols, xs, xsum);
        else
            down_dispatch_rows<0, MAXNR>(a, g, tile * kDnCols, xs, xsum);
        fcur = -1;
        prev_slow = true;
    }
}

// ---- one row: the down projection with the combine folded in -------------
//
// At T = 1 with 4-bit routed experts and K = I = Is = 2048 (one 4-bit lane
// step per weight row), the token-major form ([P2] "Per MoE layer": the rows
// come back as one weighted sum per token): wave w of block b owns output
// column c = 8 b + w, loads that column's row of every pick's down matrix and
// of the shared expert's, reduces each exactly as down_item does (same staged
// layout -- pairwise-permuted with per-32 sums for W4A16 and MLX affine, plain
// for NVFP4 -- same lane steps, same helpers, same wave sums) and adds them in
// pick order as combine_kernel does, then the shared output, then the
// residual -- bit for
// bit the unfused pair of launches, without the per-pick outputs' round trip
// and the combine's launch.  All in-band picks' rows of h (slots 0..N_in-1,
// T = 1) and the shared row are staged once per block, every load in flight
// before the first LDS write.
constexpr int kOneMaxPicks = 8;

template <int FMT>
__global__ __launch_bounds__(kGemvThreads, 4) void down_combine_one_kernel(ExpertArgs a, const int32_t* __restrict__ ids,
                                                                           const int32_t* __restrict__ pos,
                                                                           const float* __restrict__ wts, int k,
                                                                           const uint16_t* __restrict__ res,
                                                                           int has_shared, float* __restrict__ out) {
    constexpr int K = 2048, C8N = K / 8, GN = K / 32;
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                         // [kOneMaxPicks + 1][K]
    float* xsum = reinterpret_cast<float*>(smem + (kOneMaxPicks + 1) * K * 2);  // [kOneMaxPicks][K / 32]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.H;
    int p[kOneMaxPicks], nin = 0;
#pragma unroll
    for (int j = 0; j < kOneMaxPicks; ++j) {
        p[j] = j < k ? pos[j] : -1;
        nin += p[j] >= 0 ? 1 : 0;
    }
    // staging: chunk i of the routed rows (slot i / C8N, permuted as
    // stage_rows does) or of the shared row (plain); every load first
    constexpr int PER = ((kOneMaxPicks + 1) * C8N + kGemvThreads - 1) / kGemvThreads;
    uint4 v[PER];
    const int nchunk = (nin + (has_shared ? 1 : 0)) * C8N;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int idx = tid + u * kGemvThreads;
        const int r = idx / C8N, c8 = idx - r * C8N;
        const uint16_t* src = r < nin ? a.h_r + (size_t)r * a.I : a.h_s;
        v[u] = idx < nchunk ? *reinterpret_cast<const uint4*>(src + 8 * c8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int idx = tid + u * kGemvThreads;
        if (idx >= nchunk) continue;
        const int r = idx / C8N, c8 = idx - r * C8N;
        uint4 w = v[u];
        int dst = c8;
        uint16_t* row = xs + (size_t)(r < nin ? r : kOneMaxPicks) * K;
        if (r < nin && FMT != 3) {
            uint4 q;
            q.x = (w.x & 0xffffu) | (w.z << 16);
            q.y = (w.x >> 16) | (w.z & 0xffff0000u);
            q.z = (w.y & 0xffffu) | (w.w << 16);
            q.w = (w.y >> 16) | (w.w & 0xffff0000u);
            w = q;
            dst = (c8 & ~3) | w4_chunk(c8 >> 2, c8 & 3);
        }
        *reinterpret_cast<uint4*>(row + 8 * dst) = w;
    }
    __syncthreads();
    // per-32 sums of the routed rows, as stage_rows forms them (NVFP4 reads
    // its rows in plain order and uses no sums)
    for (int idx = tid; FMT != 3 && idx < nin * GN; idx += kGemvThreads) {
        const int r = idx / GN, gi = idx - r * GN;
        const uint4* src = reinterpret_cast<const uint4*>(xs + (size_t)r * K + 32 * gi);
        float sum = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 w = src[w4_chunk(gi, q)];
            sum += bf16_lo(w.x) + bf16_hi(w.x);
            sum += bf16_lo(w.y) + bf16_hi(w.y);
            sum += bf16_lo(w.z) + bf16_hi(w.z);
            sum += bf16_lo(w.w) + bf16_hi(w.w);
        }
        xsum[r * GN + gi] = sum;
    }
    __syncthreads();

    const int c = blockIdx.x * kGemvWaves + wave;
    if (c >= H) return;
    // every pick's row of column c (picks outside the band read expert 0's,
    // unused), then the shared row, all in flight at once
    uint4 qv[kOneMaxPicks];
    uint32_t sv[kOneMaxPicks], zv[kOneMaxPicks];
    int ej[kOneMaxPicks];
#pragma unroll
    for (int j = 0; j < kOneMaxPicks; ++j) {
        ej[j] = p[j] >= 0 ? ids[j] : 0;
        const size_t row = (size_t)ej[j] * H + c;
        qv[j] = wload(a.qd + row * (K / 2) + 16 * lane);
        load_scales<FMT>(a.sd, a.zd, row, K, 32 * lane, &sv[j], &zv[j]);
    }
    // (no shared expert: any valid address, unused)
    const uint16_t* swr = has_shared ? a.swd + (size_t)c * K : reinterpret_cast<const uint16_t*>(a.qd);
    uint4 wv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) wv[q] = wload(swr + 512 * q + 8 * lane);

    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < kOneMaxPicks; ++j) {
        if (p[j] < 0) continue;  // wave-uniform
        float part[1] = {0.0f};
        quant_step<FMT, 1>(qv[j], sv[j], zv[j], true, xs + (size_t)(p[j] < 0 ? 0 : p[j]) * K,
                           xsum + (size_t)(p[j] < 0 ? 0 : p[j]) * GN, K, 32 * lane, part);
        float y = wave_sum(part[0]);
        if (FMT == 3) y *= a.gd[ej[j]];
        acc = __builtin_fmaf(wts[j], y, acc);
    }
    if (has_shared) {
        const uint16_t* xl = xs + (size_t)kOneMaxPicks * K + 8 * lane;
        float t = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 xv = *reinterpret_cast<const uint4*>(xl + 512 * q);
            t = dot2_bf16(wv[q].x, xv.x, t);
            t = dot2_bf16(wv[q].y, xv.y, t);
            t = dot2_bf16(wv[q].z, xv.z, t);
            t = dot2_bf16(wv[q].w, xv.w, t);
        }
        acc = acc + wave_sum(t);
    }
    if (res) acc = acc + bf16_bits_to_f32(res[c]);
    if (lane == 0) out[c] = acc;
}

bool down_combine_one_ok(const ExpertArgs& a, int k, bool has_shared) {
    return a.T == 1 && a.fmt != 0 && k <= kOneMaxPicks && a.I == 2048 && (!has_shared || a.Is == 2048) &&
           a.H % kGemvWaves == 0;
}

void launch_down_combine_one(const ExpertArgs& a, const int32_t* ids, const int32_t* pos, const float* wts, int k,
                             const uint16_t* res, bool has_shared, float* out, hipStream_t st) {
    const size_t lds = (size_t)(kOneMaxPicks + 1) * 2048 * 2 + (size_t)kOneMaxPicks * (2048 / 32) * 4;
    const int grid = a.H / kGemvWaves;
    auto go = [&](auto fmt) {
        constexpr int F = decltype(fmt)::value;
        allow_lds(down_combine_one_kernel<F>, lds);
        down_combine_one_kernel<F><<<grid, kGemvThreads, lds, st>>>(a, ids, pos, wts, k, res, has_shared ? 1 : 0, out);
    };
    switch (a.fmt) {
        case 2: go(std::integral_constant<int, 2>{}); break;
        case 3: go(std::integral_constant<int, 3>{}); break;
        default: go(std::integral_constant<int, 1>{}); break;
    }
}

// blocks per CU: three for the one-row kernels bounded to 6 waves per SIMD
// when their LDS allows
static int gemv_grid(size_t lds, int num_cu, long long ub, bool six_waves = false) {
    int occ = six_waves && lds <= 53 * 1024 ? 3 : (lds <= 64 * 1024 ? 2 : 1);
    long long g = (long long)num_cu * occ;
    if (ub < g) g = ub;
    return (int)(g < 1 ? 1 : g);
}

template <int FMT, int CB, int MAXNR>
static void launch_gateup_fmt(const ExpertArgs& a, int grid, size_t lds, int lds_rows, hipStream_t st) {
    allow_lds(gateup_gemv_kernel<FMT, CB, MAXNR>, lds);
    gateup_gemv_kernel<FMT, CB, MAXNR><<<grid, kGemvThreads, lds, st>>>(a, lds_rows);
}

// 4-bit experts at T = 1 take the one-row kernels; their bf16 path, for the
// shared expert when the top-k launch has not done it, loads at most 4 lane
// steps at a time to stay within the registers of two or three blocks per CU.
template <int CB>
static void launch_gateup_cb(const ExpertArgs& a, int grid, size_t lds, int lds_rows,
                             hipStream_t st) {
    constexpr int CB1 = CB < 4 ? CB : 4;
    const bool one = a.T == 1;
    switch (a.fmt) {
        case 1:
            one ? launch_gateup_fmt<1, CB1, 1>(a, grid, lds, lds_rows, st)
                : launch_gateup_fmt<1, CB, 8>(a, grid, lds, lds_rows, st);
            break;
        case 2:
            one ? launch_gateup_fmt<2, CB1, 1>(a, grid, lds, lds_rows, st)
                : launch_gateup_fmt<2, CB, 8>(a, grid, lds, lds_rows, st);
            break;
        case 3:
            one ? launch_gateup_fmt<3, CB1, 1>(a, grid, lds, lds_rows, st)
                : launch_gateup_fmt<3, CB, 8>(a, grid, lds, lds_rows, st);
            break;
        default: launch_gateup_fmt<0, CB, 8>(a, grid, lds, lds_rows, st); break;
    }
}

void launch_gateup_gemv(const ExpertArgs& a, int max_groups, int num_cu, hipStream_t st) {
    const int max_rows = a.T < kSmallRows ? a.T : kSmallRows;
    // rows of LDS: the largest group, and at least two buffers of two rows
    const int lds_rows = max_rows > 4 ? max_rows : 4;
    const size_t lds = (size_t)lds_rows * a.H * 2 + (a.fmt ? (size_t)max_rows * (a.H / 32) * 4 : 0);
    const int tiles = (a.I > a.Is ? a.I : a.Is) / kGuCols;
    const int grid = gemv_grid(lds, num_cu, (long long)max_groups * tiles, a.T == 1 && one_row_waves(a.fmt, true) == 6);
    // lane steps per load block for bf16 rows: the whole row when it has at
    // most 12 steps of 512 inputs (H <= 6144)
    const int nch = (a.H + 511) / 512;
    if (nch <= 4)
        launch_gateup_cb<4>(a, grid, lds, lds_rows, st);
    else if (nch <= 8)
        launch_gateup_cb<8>(a, grid, lds, lds_rows, st);
    else
        launch_gateup_cb<12>(a, grid, lds, lds_rows, st);
}

void launch_down_gemv(const ExpertArgs& a, int max_groups, int num_cu, hipStream_t st) {
    const int max_rows = a.T < kSmallRows ? a.T : kSmallRows;
    const int kmax = a.I > a.Is ? a.I : a.Is;
    // rows of LDS: the largest group, and at least two buffers of two rows
    const int lds_rows = max_rows > 4 ? max_rows : 4;
    const size_t lds = (size_t)lds_rows * kmax * 2 + (a.fmt ? (size_t)max_rows * (kmax / 32) * 4 : 0);
    const int grid = gemv_grid(lds, num_cu, (long long)max_groups * (a.H / kDnCols),
                               a.T == 1 && one_row_waves(a.fmt, false) == 6);
    auto go = [&](auto fmt) {
        constexpr int F = decltype(fmt)::value;
        if (a.T == 1) {  // one-row kernels: two or three blocks per CU
            allow_lds(down_gemv_kernel<F, 1>, lds);
            down_gemv_kernel<F, 1><<<grid, kGemvThreads, lds, st>>>(a, lds_rows, kmax);
        } else {
            allow_lds(down_gemv_kernel<F, 8>, lds);
            down_gemv_kernel<F, 8><<<grid, kGemvThreads, lds, st>>>(a, lds_rows, kmax);
        }
    };
    switch (a.fmt) {
        case 1: go(std::integral_constant<int, 1>{}); break;
        case 2: go(std::integral_constant<int, 2>{}); break;
        case 3: go(std::integral_constant<int, 3>{}); break;
        default: go(std::integral_constant<int, 0>{}); break;
    }
}

}  // namespace moe
