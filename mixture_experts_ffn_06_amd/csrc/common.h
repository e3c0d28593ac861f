// common.h -- device helpers and the internal plan shared by the kernels of
// libmoeffn.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;
// Groups of at most this many rows take the bandwidth-bound GEMV path; larger
// groups take the MFMA path.
constexpr int kSmallRows = 8;
// MFMA tile: rows of the group x weight rows x reduction depth.
constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBK = 64;
// GEMV work items: gate/up covers 16 intermediate columns (16 gate + 16 up
// weight rows), down covers 64 output columns.
constexpr int kGuCols = 16;
constexpr int kDnCols = 64;
// Rows per dispatch block (four waves of 64 rows).
constexpr int kDispatchRows = 256;

// One expert group of the dispatch: a routed expert of the band (expert >= 0)
// or the shared expert (expert == -1).
struct Group {
    int32_t expert;  // global expert id, or -1 for the shared expert
    int32_t row0;    // first row of the group in perm order (0 for the shared expert)
    int32_t n;       // rows in the group
    int32_t pad;
};

// Pointers and sizes every expert kernel needs.  Built on the host per call.
struct ExpertArgs {
    // rows
    const uint16_t* x;  // bf16 [T, H]
    int32_t T, H, topk;
    // routed experts
    int32_t I;
    int32_t fmt;                // 0 bf16, 1 W4A16 (G 32), 2 MLX affine (G 64), 3 NVFP4 (G 16)
    const uint16_t* wgu;        // bf16 [E, 2I, H]
    const uint16_t* wd;         // bf16 [E, H, I]
    const uint8_t* qgu;         // [E, 2I, H/2]
    const uint16_t* sgu;        // [E, 2I, H/G] (NVFP4: E4M3 bytes)
    const uint16_t* zgu;
    const uint8_t* qd;          // [E, H, I/2]
    const uint16_t* sd;         // [E, H, I/G] (NVFP4: E4M3 bytes)
    const uint16_t* zd;
    const float* ggu;           // NVFP4 matrix scales [E, 2] (gate, up), else null
    const float* gd;            // NVFP4 matrix scales [E], else null
    // shared expert (bf16)
    int32_t Is;
    const uint16_t* swgu;       // [2Is, H]
    const uint16_t* swd;        // [H, Is]
    // plan (device, written by the dispatch)
    const Group* groups;        // [nb + 1]
    const int32_t* gemv_list;   // group indices on the GEMV path
    const int32_t* mfma_list;   // four lists of (group, m0) pairs: 128-, 64-, 32- and 256-row tiles
    int32_t mfma_cap;           // capacity of each list
    const int32_t* plan_counts; // [0] GEMV groups, [1..4] tiles of 128, 64, 32, 256 rows
    const int32_t* perm;        // [T*topk]
    // scratch
    uint16_t* h_r;  // bf16 [T*topk, I]  (perm order)
    uint16_t* h_s;  // bf16 [T, Is]
    float* y_r;     // fp32 [T*topk, H] (perm order)
    float* y_s;     // fp32 [T, H]
    // the shared expert's h was computed by the top-k/dispatch launch (its
    // gate/up GEMV items are skipped)
    int32_t shared_gu_done;
};

// The shared expert's gate/up run by extra blocks of the top-k/dispatch
// launch (T <= kSmallRows, H a multiple of 512): it depends on no routing
// decision, so its weight stream overlaps the routing's latency chain.
struct SharedGateUp {
    const uint16_t* x;  // bf16 [T, H] (the normed rows when a norm is given)
    const uint16_t* w;  // bf16 [2 Is, H]: gate rows, then up rows
    uint16_t* h;        // bf16 [T, Is]
    int32_t T, H, Is;
    int32_t blocks;     // blocks beyond the first; 0: not done there
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even fp32 -> bf16 bits (hardware convert on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
    return g / (1.0f + __expf(-g)) * u;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// acc + a.lo*b.lo + a.hi*b.hi with a, b packed bf16 pairs.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Sum over the 64 lanes of a wave, in a fixed order: four DPP steps sum each
// row of 16 lanes (pairs, quads, halves, rows: every lane of a row ends with
// the row's sum), then (row0 + row1) + (row2 + row3) from lanes 0, 16, 32, 48.
// Every lane gets the sum.  DPP moves stay in the VALU, so the chain is short.
template <int CTRL>
__device__ __forceinline__ float dpp_term(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_term<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_term<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_term<0x141>(v);  // row_half_mirror
    v += dpp_term<0x140>(v);  // row_mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

// Weight loads.  Every weight byte is read once per call, so the loads carry
// the non-temporal hint (the `nt` cache-policy bit): the lines are not kept
// in preference to reused data.  Measured on the decode GEMVs: 6.0 -> 6.8
// TB/s.
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 wload(const void* p) {
    const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Allow a kernel more than 64 KiB of dynamic LDS (gfx950 has 160 KiB per
// CU): the attribute is raised only when a call needs more than was set
// before for that kernel on this device (a host-side table, moe_ffn.cpp),
// so the steady state makes no runtime call.
void allow_lds_once(const void* kernel, size_t bytes);
template <typename F>
inline void allow_lds(F* kernel, size_t bytes) {
    if (bytes > 64 * 1024) allow_lds_once(reinterpret_cast<const void*>(kernel), bytes);
}

// Host-side launchers (one per kernel family).
void launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps, int T, int H, uint16_t* xn,
                    hipStream_t st);
void launch_router_logits(const uint16_t* x, const float* wr, const float* bias, int T, int H,
                          int E, float* logits, hipStream_t st);
// sigmoid = 0: softmax over the picks of biased logits; 1: picks by
// sigmoid + bias of unbiased logits, raw-score weights (topk.h)
void launch_router_topk(const float* logits, const float* bias, int sigmoid, int T, int E, int k,
                        int32_t* ids, float* w, hipStream_t st);
// Batches of at most 16 rows: top-k and the dispatch in one block, and the
// shared expert's gate/up in sg.blocks more blocks of the same launch.
void launch_topk_dispatch_small(const float* logits, const float* bias, int sigmoid, int E, float* wts,
                                int32_t* ids, int T, int k,
                                int lo, int hi, bool has_shared, int32_t* counts, int32_t* offsets,
                                int32_t* perm, int32_t* pos, Group* groups, int32_t* gemv_list,
                                int32_t* mfma_list, int mfma_cap, int32_t* plan_counts,
                                const SharedGateUp& sg, hipStream_t st);
void launch_dispatch(const int32_t* ids, int T, int k, int lo, int hi, bool has_shared,
                     int32_t* blkcnt, int32_t* counts, int32_t* offsets, int32_t* perm,
                     int32_t* pos, Group* groups, int32_t* gemv_list, int32_t* mfma_list,
                     int mfma_cap, int32_t* plan_counts, hipStream_t st);
void launch_gateup_gemv(const ExpertArgs& a, int max_groups, int num_cu, hipStream_t st);
void launch_down_gemv(const ExpertArgs& a, int max_groups, int num_cu, hipStream_t st);
// T = 1, 4-bit routed experts, K = I = Is = 2048, at most 8 picks: the down
// projection with the pick-order combine folded in (bit for bit the pair of
// down_gemv and combine launches); down_combine_one_ok says when it applies.
bool down_combine_one_ok(const ExpertArgs& a, int k, bool has_shared);
void launch_down_combine_one(const ExpertArgs& a, const int32_t* ids, const int32_t* pos, const float* wts, int k,
                             const uint16_t* res, bool has_shared, float* out, hipStream_t st);
// bf16 experts: the direct-to-LDS pipelined tiles, one launch for the
// 256-row tiles and one for the 128-, 64- and 32-row tiles (gate/up or
// down).  With 4-bit experts these launches run the (bf16) shared expert's
// tiles only.
void launch_mfma_pipe(const ExpertArgs& a, bool gateup, int num_cu, hipStream_t st);
// 4-bit experts: the same pipeline with the codes dequantized in LDS, tiles
// of 128 (and 256 as two halves), 64 and 32 rows; then the shared expert.
void launch_mfma_w4(const ExpertArgs& a, bool gateup, int num_cu, hipStream_t st);
void launch_combine(const float* y_r, const float* y_s, const uint16_t* res, const int32_t* pos, const float* w,
                    int T, int H, int k, float* out, hipStream_t st);
void launch_combine_tree(const float* y_r, const float* y_s, const uint16_t* res, const int32_t* ids, const int32_t* pos,
                         const float* w, int T, int H, int k, int node_level, float* out,
                         hipStream_t st);

// The sum of band partials: order 0 = rank order over part[0..nparts-1];
// order 1 = the canonical tree, as nops pushes of part op_part[o] (-1: a
// +0.0 node) at level op_l0[o], merged up to level op_l1[o]; the result is
// the entry at root_level.
constexpr int kMaxParts = 64;
constexpr int kMaxReduceOps = 96;
struct ReduceProgram {
    const float* part[kMaxParts];
    int8_t op_part[kMaxReduceOps];
    uint8_t op_l0[kMaxReduceOps];
    uint8_t op_l1[kMaxReduceOps];
    int nparts, nops, order, root_level;
};
void launch_reduce(const ReduceProgram& pg, const float* y_s, const uint16_t* res, size_t n,
                   float* y, int num_cu, hipStream_t st);

}  // namespace moe
