// dispatch.hip -- group the in-band picks by expert: histogram, prefix sum,
// a stable permutation (rows ascending within an expert) and its inverse,
// plus the work lists of the expert kernels.  Integer only: the result does
// not depend on scheduling, and it matches a host grouping byte for byte.
//
// [P1] "GLM-5.2 multi-GPU: expert-parallel sharding + the resident-fit
// benchmark", "What landed": each rank contributes only the picks it owns;
// its lever table: batched expert dispatch (one grouped call instead of a
// loop over experts).  [P5] "GLM-5.3-Flash and full GLM-5.3 on the native
// CUDA engine (tracker) #593": the device grouping plan is byte-equal to the
// host routing.
//
// Method: rows are cut into blocks of 256 (four waves of 64 rows).  In each
// wave, bit r of mask[e] is set when row r picked expert e (LDS integer
// atomics: the result does not depend on their order).  A pick's slot is the
// expert's offset + the picks of earlier blocks (scanned in block order) + the
// picks of earlier waves of the block + popcount(mask[e] below row r).
#include "common.h"
#include "topk.h"

namespace moe {

__device__ __forceinline__ void build_masks(unsigned long long* masks, const int32_t* ids, int T,
                                            int k, int lo, int nb) {
    const int tid = threadIdx.x;
    for (int i = tid; i < 4 * nb; i += blockDim.x) masks[i] = 0ull;
    __syncthreads();
    const int t = blockIdx.x * kDispatchRows + tid;
    const int wave = tid >> 6, lane = tid & 63;
    if (t < T) {
        for (int j = 0; j < k; ++j) {
            int e = ids[(size_t)t * k + j] - lo;
            if (e >= 0 && e < nb) atomicOr(&masks[wave * nb + e], 1ull << lane);
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t* __restrict__ ids,
                                                             int T, int k, int lo, int nb,
                                                             int32_t* __restrict__ blkcnt) {
    extern __shared__ unsigned long long masks[];
    build_masks(masks, ids, T, k, lo, nb);
    for (int e = threadIdx.x; e < nb; e += blockDim.x) {
        int c = __popcll(masks[e]) + __popcll(masks[nb + e]) + __popcll(masks[2 * nb + e]) +
                __popcll(masks[3 * nb + e]);
        blkcnt[(size_t)blockIdx.x * nb + e] = c;
    }
}

// Inclusive sum over the lanes of a wave (lane l gets v_0 + .. + v_l): four
// row shifts sum within each row of 16 lanes, then two row broadcasts carry
// the row totals (DPP moves: no LDS round trip per step).
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
    return v;
}

// Exclusive scans of N values over the 1024 threads of a block at once
// (integer sums: the result does not depend on the order): wave scans, then
// wave 0 scans the 16 wave totals.  s_tmp holds 17 N ints.
template <int N>
__device__ void block_exclusive_scan_n(const int (&v)[N], int (&res)[N], int (&total)[N], int* s_tmp) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int inc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) inc[i] = wave_incl_scan(v[i]);
    if (lane == 63)
#pragma unroll
        for (int i = 0; i < N; ++i) s_tmp[wave * N + i] = inc[i];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int w = wave_incl_scan(lane < 16 ? s_tmp[lane * N + i] : 0);
            if (lane < 16) s_tmp[lane * N + i] = w;  // inclusive over waves
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int before = wave ? s_tmp[(wave - 1) * N + i] : 0;
        res[i] = before + inc[i] - v[i];
        total[i] = s_tmp[15 * N + i];
    }
    __syncthreads();
}

__device__ __forceinline__ int block_exclusive_scan(int v, int* s_tmp, int* total) {
    const int vv[1] = {v};
    int r[1], t[1];
    block_exclusive_scan_n<1>(vv, r, t, s_tmp);
    *total = t[0];
    return r[0];
}

// Groups and work lists.  Thread i owns groups 2i and 2i+1 with row counts
// cnt[] and first rows run[]; group nb is the shared expert when present.
__device__ void build_plan(const int cnt[2], const int run[2], int nb, int T, int lo,
                           bool has_shared, Group* __restrict__ groups,
                           int32_t* __restrict__ gemv_list, int32_t* __restrict__ mfma_list,
                           int mfma_cap, int32_t* __restrict__ plan_counts, int* s_tmp) {
    const int tid = threadIdx.x;
    // A group of 1..8 rows goes to the GEMV path; one of 9..32, 33..64 or
    // 65..128 rows is one tile of 32, 64 or 128 rows; a larger one is cut into
    // 256-row tiles, the last one partial.  Every group is in exactly one
    // list, so one launch reads each expert's weights.
    int n[2], gv[2], t256[2], t128[2], t64[2], t32[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int e = 2 * tid + q;
        n[q] = 0;
        if (e < nb) {
            n[q] = cnt[q];
            groups[e] = Group{lo + e, run[q], cnt[q], 0};
        } else if (e == nb && has_shared) {
            n[q] = T;
            groups[e] = Group{-1, 0, T, 0};
        }
        const int nn = n[q];
        gv[q] = (nn >= 1 && nn <= kSmallRows) ? 1 : 0;
        t32[q] = (nn > kSmallRows && nn <= 32) ? 1 : 0;
        t64[q] = (nn > 32 && nn <= 64) ? 1 : 0;
        t128[q] = (nn > 64 && nn <= 128) ? 1 : 0;
        t256[q] = nn > 128 ? (nn + 255) / 256 : 0;
    }
    const int cnts[5] = {gv[0] + gv[1], t256[0] + t256[1], t128[0] + t128[1], t64[0] + t64[1],
                         t32[0] + t32[1]};
    int offs[5], tots[5];
    block_exclusive_scan_n<5>(cnts, offs, tots, s_tmp);
    int gv0 = offs[0], o256 = offs[1], o128 = offs[2], o64 = offs[3], o32 = offs[4];
    const int ngv = tots[0], n256 = tots[1], n128 = tots[2], n64 = tots[3], n32 = tots[4];
    int32_t* l128 = mfma_list;
    int32_t* l64 = mfma_list + 2 * (size_t)mfma_cap;
    int32_t* l32 = mfma_list + 4 * (size_t)mfma_cap;
    int32_t* l256 = mfma_list + 6 * (size_t)mfma_cap;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int e = 2 * tid + q;
        if (gv[q]) gemv_list[gv0] = e;
        gv0 += gv[q];
        for (int m = 0; m < t256[q]; ++m) {
            l256[2 * (o256 + m)] = e;
            l256[2 * (o256 + m) + 1] = m * 256;
        }
        o256 += t256[q];
        if (t128[q]) {
            l128[2 * o128] = e;
            l128[2 * o128 + 1] = 0;
        }
        o128 += t128[q];
        if (t64[q]) {
            l64[2 * o64] = e;
            l64[2 * o64 + 1] = 0;
        }
        o64 += t64[q];
        if (t32[q]) {
            l32[2 * o32] = e;
            l32[2 * o32 + 1] = 0;
        }
        o32 += t32[q];
    }
    if (tid == 0) {
        plan_counts[0] = ngv;
        plan_counts[1] = n128;
        plan_counts[2] = n64;
        plan_counts[3] = n32;
        plan_counts[4] = n256;
    }
}


// One block of 1024 threads; thread i owns groups 2i and 2i+1 (group nb is the
// shared expert when present).
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(
    int nblk, int nb, int T, bool has_shared, int32_t* __restrict__ blkcnt,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, Group* __restrict__ groups,
    int32_t* __restrict__ gemv_list, int32_t* __restrict__ mfma_list, int mfma_cap,
    int32_t* __restrict__ plan_counts, int lo) {
    __shared__ int s_tmp[17 * 5];
    const int tid = threadIdx.x;
    int cnt[2], run[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int e = 2 * tid + q;
        int r = 0;
        if (e < nb) {
            for (int b = 0; b < nblk; ++b) {
                int c = blkcnt[(size_t)b * nb + e];
                blkcnt[(size_t)b * nb + e] = r;
                r += c;
            }
        }
        cnt[q] = r;
    }
    int total;
    int off0 = block_exclusive_scan(cnt[0] + cnt[1], s_tmp, &total);
    run[0] = off0;
    run[1] = off0 + cnt[0];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int e = 2 * tid + q;
        if (e < nb) {
            counts[e] = cnt[q];
            offsets[e] = run[q];
            for (int b = 0; b < nblk; ++b) blkcnt[(size_t)b * nb + e] += run[q];
        }
    }
    if (tid == 0) offsets[nb] = total;

    build_plan(cnt, run, nb, T, lo, has_shared, groups, gemv_list, mfma_list, mfma_cap,
               plan_counts, s_tmp);
}

__global__ __launch_bounds__(256) void dispatch_place_kernel(const int32_t* __restrict__ ids,
                                                             int T, int k, int lo, int nb,
                                                             const int32_t* __restrict__ base,
                                                             int32_t* __restrict__ perm,
                                                             int32_t* __restrict__ pos) {
    extern __shared__ unsigned long long masks[];
    build_masks(masks, ids, T, k, lo, nb);
    const int tid = threadIdx.x;
    const int t = blockIdx.x * kDispatchRows + tid;
    const int wave = tid >> 6, lane = tid & 63;
    if (t >= T) return;
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int j = 0; j < k; ++j) {
        const int p = t * k + j;
        int e = ids[p] - lo;
        if (e >= 0 && e < nb) {
            int slot = base[(size_t)blockIdx.x * nb + e];
            for (int w = 0; w < wave; ++w) slot += __popcll(masks[w * nb + e]);
            slot += __popcll(masks[wave * nb + e] & below);
            perm[slot] = p;
            pos[p] = slot;
        } else {
            pos[p] = -1;
        }
    }
}

// All of the dispatch in one block when every row fits in one block of 256
// rows (decode): masks, counts, scan, plan and placement without a kernel
// boundary in between.  1024 threads; threads 0..255 own the rows of the
// masks, the placement takes one thread per pick.
__device__ __forceinline__ void dispatch_small_body(
    const int32_t* __restrict__ ids, int T, int k, int lo, int nb, bool has_shared,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ pos, Group* __restrict__ groups, int32_t* __restrict__ gemv_list,
    int32_t* __restrict__ mfma_list, int mfma_cap, int32_t* __restrict__ plan_counts) {
    extern __shared__ unsigned long long masks[];  // [4][nb], then int offsets[nb + 1]
    int* s_off = reinterpret_cast<int*>(masks + 4 * nb);
    __shared__ int s_tmp[17 * 5];
    build_masks(masks, ids, T, k, lo, nb);
    const int tid = threadIdx.x;
    int cnt[2], run[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int e = 2 * tid + q;
        cnt[q] = e < nb ? __popcll(masks[e]) + __popcll(masks[nb + e]) + __popcll(masks[2 * nb + e]) +
                              __popcll(masks[3 * nb + e])
                        : 0;
    }
    int total;
    const int off0 = block_exclusive_scan(cnt[0] + cnt[1], s_tmp, &total);
    run[0] = off0;
    run[1] = off0 + cnt[0];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int e = 2 * tid + q;
        if (e < nb) {
            counts[e] = cnt[q];
            offsets[e] = run[q];
            s_off[e] = run[q];
        }
    }
    if (tid == 0) offsets[nb] = total;
    build_plan(cnt, run, nb, T, lo, has_shared, groups, gemv_list, mfma_list, mfma_cap,
               plan_counts, s_tmp);  // its scans hold barriers: s_off is visible
    // one thread per pick: its slot is the expert's offset + the picks of
    // earlier rows (earlier waves' masks, then the bits below its row)
    for (int p = tid; p < T * k; p += blockDim.x) {
        const int t = p / k;
        const int e = ids[p] - lo;
        if (e >= 0 && e < nb) {
            const int wave = t >> 6, row = t & 63;
            int slot = s_off[e];
            for (int w = 0; w < wave; ++w) slot += __popcll(masks[w * nb + e]);
            slot += __popcll(masks[wave * nb + e] & ((1ull << row) - 1ull));
            perm[slot] = p;
            pos[p] = slot;
        } else {
            pos[p] = -1;
        }
    }
}

__global__ __launch_bounds__(1024) void dispatch_small_kernel(
    const int32_t* __restrict__ ids, int T, int k, int lo, int nb, bool has_shared,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ pos, Group* __restrict__ groups, int32_t* __restrict__ gemv_list,
    int32_t* __restrict__ mfma_list, int mfma_cap, int32_t* __restrict__ plan_counts) {
    dispatch_small_body(ids, T, k, lo, nb, has_shared, counts, offsets, perm, pos, groups, gemv_list,
                        mfma_list, mfma_cap, plan_counts);
}

// The shared expert's gate/up for NR rows in one block of 16 waves: each wave
// takes gate/up column pairs c = wave * nblocks + block, then c + 16 nblocks,
// ... (so every block has work when the columns are few), with the rows staged
// in LDS by direct global->LDS loads issued ahead of the weights.  A wave's
// first weight loads are issued before the staging's wait and barrier, and
// each next column's first loads before the current column's lane sums.  A column's two dots follow the GEMV path's order: lane l
// accumulates the inputs 512 q + 8 l .. +7 over q = 0, 1, .. (dot2 pairs in
// order), then the lanes are summed by wave_sum.
template <int NR>
__device__ void shared_gateup_rows(const SharedGateUp& s, int block, int nblocks) {
    extern __shared__ uint4 xs4[];
    uint16_t* xs = reinterpret_cast<uint16_t*>(xs4);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = s.H, c8n = H / 8;
    constexpr int QB = 6;  // lane steps of 512 inputs per block of loads
    const int nq = H / 512;
    uint4 wg[QB], wu[QB];
    auto issue = [&](int c, int q0) {
        const uint16_t* gr = s.w + (size_t)c * H + 8 * lane;
        const uint16_t* ur = gr + (size_t)s.Is * H;
#pragma unroll
        for (int qq = 0; qq < QB; ++qq) {
            const int q = q0 + qq < nq ? q0 + qq : nq - 1;  // past the row: reload, unused
            wg[qq] = wload(gr + 512 * q);
            wu[qq] = wload(ur + 512 * q);
        }
    };
    int c = wave * nblocks + block;
    const int nwaves = blockDim.x >> 6;
    const int step = nblocks * nwaves;
    // The rows (contiguous, NR * H / 8 16-byte chunks: a multiple of 64 since
    // H is a multiple of 512) go straight to LDS, 64 chunks per wave load,
    // before the weight loads; each wave then waits until only its weight
    // loads are in flight (loads return in issue order), and a plain barrier
    // (no fence: it would wait for the weights too) makes the rows visible.
    typedef __attribute__((address_space(3))) unsigned char lds_byte;
    lds_byte* xl8 = (lds_byte*)xs4;
    for (int c0 = 64 * wave; c0 < NR * c8n; c0 += 64 * nwaves)
        __builtin_amdgcn_global_load_lds(s.x + (size_t)(c0 + lane) * 8, xl8 + (size_t)c0 * 16, 16, 0, 0);
    // the wait below counts on every row load issuing before the weight loads
    __builtin_amdgcn_sched_barrier(0);
    const bool first = c < s.Is;
    if (first) {
        issue(c, 0);
        // (0xf << 8) | (7 << 4): lgkm and exp counts unconstrained; vmcnt 2 QB
        __builtin_amdgcn_s_waitcnt((2 * QB & 0xf) | (0x7 << 4) | (0xf << 8) | (((2 * QB) >> 4) << 14));
    } else {
        __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xf << 8));
    }
    __builtin_amdgcn_s_barrier();
    // no read of the staged rows may move above the barrier (a compiler-only
    // memory barrier: it emits no wait for the weight loads in flight)
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    const uint16_t* xl = xs + 8 * lane;
    while (c < s.Is) {
        float ag[NR], au[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) ag[r] = au[r] = 0.0f;
        for (int q0 = 0; q0 < nq; q0 += QB) {
            if (q0 > 0) issue(c, q0);
#pragma unroll
            for (int qq = 0; qq < QB; ++qq) {
                if (q0 + qq >= nq) break;  // wave-uniform
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    const uint4 xv = *reinterpret_cast<const uint4*>(xl + (size_t)r * H + 512 * (q0 + qq));
                    float sg = ag[r], su = au[r];
                    sg = dot2_bf16(wg[qq].x, xv.x, sg);
                    sg = dot2_bf16(wg[qq].y, xv.y, sg);
                    sg = dot2_bf16(wg[qq].z, xv.z, sg);
                    sg = dot2_bf16(wg[qq].w, xv.w, sg);
                    su = dot2_bf16(wu[qq].x, xv.x, su);
                    su = dot2_bf16(wu[qq].y, xv.y, su);
                    su = dot2_bf16(wu[qq].z, xv.z, su);
                    su = dot2_bf16(wu[qq].w, xv.w, su);
                    ag[r] = sg;
                    au[r] = su;
                }
            }
        }
        const int cn = c + step;
        if (cn < s.Is) issue(cn, 0);
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const float g = wave_sum(ag[r]);
            const float u = wave_sum(au[r]);
            if (lane == r) s.h[(size_t)r * s.Is + c] = f32_to_bf16_bits(silu_mul(g, u));
        }
        c = cn;
    }
}

__device__ void shared_gateup_block(const SharedGateUp& s, int block, int nblocks) {
    switch (s.T) {
        case 1: shared_gateup_rows<1>(s, block, nblocks); break;
        case 2: shared_gateup_rows<2>(s, block, nblocks); break;
        case 3: shared_gateup_rows<3>(s, block, nblocks); break;
        case 4: shared_gateup_rows<4>(s, block, nblocks); break;
        case 5: shared_gateup_rows<5>(s, block, nblocks); break;
        case 6: shared_gateup_rows<6>(s, block, nblocks); break;
        case 7: shared_gateup_rows<7>(s, block, nblocks); break;
        default: shared_gateup_rows<8>(s, block, nblocks); break;
    }
}

// Batches of at most 16 rows: top-k (wave t takes row t) and the dispatch in
// block 0; the picks go to the outputs and to LDS, where the dispatch reads
// them.  Blocks 1 .. sg.blocks compute the shared expert's gate/up meanwhile.
template <int PER>
__global__ __launch_bounds__(1024) void topk_dispatch_small_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int sigmoid, int E,
    float* __restrict__ wts, int32_t* __restrict__ ids,
    int T, int k, int lo, int nb, bool has_shared, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ pos,
    Group* __restrict__ groups, int32_t* __restrict__ gemv_list, int32_t* __restrict__ mfma_list,
    int mfma_cap, int32_t* __restrict__ plan_counts, SharedGateUp sg) {
    if (blockIdx.x > 0) {
        shared_gateup_block(sg, blockIdx.x - 1, sg.blocks);
        return;
    }
    __shared__ int32_t s_ids[16 * 16];  // rows x picks (at most 16 each)
    const int wave = threadIdx.x >> 6;
    if (wave < T) topk_row<PER>(logits, bias, sigmoid, wave, E, k, ids, wts, s_ids);
    __syncthreads();
    dispatch_small_body(s_ids, T, k, lo, nb, has_shared, counts, offsets, perm, pos, groups, gemv_list,
                        mfma_list, mfma_cap, plan_counts);
}

void launch_topk_dispatch_small(const float* logits, const float* bias, int sigmoid, int E, float* wts,
                                int32_t* ids, int T, int k,
                                int lo, int hi, bool has_shared, int32_t* counts, int32_t* offsets,
                                int32_t* perm, int32_t* pos, Group* groups, int32_t* gemv_list,
                                int32_t* mfma_list, int mfma_cap, int32_t* plan_counts,
                                const SharedGateUp& sg, hipStream_t st) {
    const int nb = hi - lo;
    size_t lds = sizeof(unsigned long long) * 4 * (size_t)nb + sizeof(int) * ((size_t)nb + 1);
    if (sg.blocks > 0 && (size_t)sg.T * sg.H * 2 > lds) lds = (size_t)sg.T * sg.H * 2;
    const int per = (E + 63) / 64;
#define MOE_TOPK_DISPATCH(P)                                                                          \
    do {                                                                                              \
        allow_lds(topk_dispatch_small_kernel<P>, lds);                                                \
        topk_dispatch_small_kernel<P><<<1 + sg.blocks, 1024, lds, st>>>(                              \
            logits, bias, sigmoid, E, wts, ids, T, k, lo, nb, has_shared, counts, offsets, perm, pos, \
            groups, gemv_list, mfma_list, mfma_cap, plan_counts, sg);                                 \
    } while (0)
    if (per <= 1)
        MOE_TOPK_DISPATCH(1);
    else if (per <= 2)
        MOE_TOPK_DISPATCH(2);
    else if (per <= 4)
        MOE_TOPK_DISPATCH(4);
    else if (per <= 8)
        MOE_TOPK_DISPATCH(8);
    else
        MOE_TOPK_DISPATCH(16);
#undef MOE_TOPK_DISPATCH
}

void launch_dispatch(const int32_t* ids, int T, int k, int lo, int hi, bool has_shared,
                     int32_t* blkcnt, int32_t* counts, int32_t* offsets, int32_t* perm,
                     int32_t* pos, Group* groups, int32_t* gemv_list, int32_t* mfma_list,
                     int mfma_cap, int32_t* plan_counts, hipStream_t st) {
    const int nb = hi - lo;
    const int nblk = (T + kDispatchRows - 1) / kDispatchRows;
    const size_t lds = sizeof(unsigned long long) * 4 * (size_t)nb;
    if (nblk == 1) {
        dispatch_small_kernel<<<1, 1024, lds + sizeof(int) * ((size_t)nb + 1), st>>>(
            ids, T, k, lo, nb, has_shared, counts, offsets, perm, pos, groups, gemv_list, mfma_list,
            mfma_cap, plan_counts);
        return;
    }
    dispatch_count_kernel<<<nblk, kDispatchRows, lds, st>>>(ids, T, k, lo, nb, blkcnt);
    dispatch_scan_kernel<<<1, 1024, 0, st>>>(nblk, nb, T, has_shared, blkcnt, counts, offsets,
                                             groups, gemv_list, mfma_list, mfma_cap, plan_counts,
                                             lo);
    dispatch_place_kernel<<<nblk, kDispatchRows, lds, st>>>(ids, T, k, lo, nb, blkcnt, perm, pos);
}

}  // namespace moe
