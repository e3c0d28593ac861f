// moe_ffn.cpp -- the C ABI of libmoeffn.so: argument checks (all before the
// first enqueue: [P1] "GLM-5.2 multi-GPU: expert-parallel sharding + the
// resident-fit benchmark", gates table, fail-closed plans), workspace layout,
// and the stage launches on the caller's stream.
#include "../../include/moe_ffn.h"

#include <hip/hip_runtime.h>

#include <math.h>
#include <mutex>
#include <string.h>

#include "common.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

// Byte offsets of the scratch buffers inside the workspace.
struct Layout {
    size_t logits, ids, w, counts, offsets, perm, pos, blkcnt, groups, gemv_list, mfma_list,
        plan_counts, h_r, h_s, y_r, y_s, xn, total;
};

int max_mfma_tiles(int T, int E, int k) {
    // tiles of one height over all groups <= (picks + shared rows) / 128 + groups
    return (int)(((long long)T * k + T) / moe::kBM) + E + 2;
}

Layout make_layout(int T, int H, int E, int I, int Is, int k) {
    Layout L;
    size_t o = 0;
    const size_t Tk = (size_t)T * k;
    const size_t nblk = ((size_t)T + moe::kDispatchRows - 1) / moe::kDispatchRows;
    L.logits = o; o += align_up((size_t)T * E * 4);
    L.ids = o; o += align_up(Tk * 4);
    L.w = o; o += align_up(Tk * 4);
    L.counts = o; o += align_up((size_t)E * 4);
    L.offsets = o; o += align_up(((size_t)E + 1) * 4);
    L.perm = o; o += align_up(Tk * 4);
    L.pos = o; o += align_up(Tk * 4);
    L.blkcnt = o; o += align_up(nblk * E * 4);
    L.groups = o; o += align_up(((size_t)E + 1) * sizeof(moe::Group));
    L.gemv_list = o; o += align_up(((size_t)E + 1) * 4);
    L.mfma_list = o; o += align_up(4 * (size_t)max_mfma_tiles(T, E, k) * 8);
    L.plan_counts = o; o += align_up(32);
    L.h_r = o; o += align_up(Tk * I * 2);
    L.h_s = o; o += align_up((size_t)T * (Is > 0 ? Is : 0) * 2);
    L.y_r = o; o += align_up(Tk * H * 4);
    L.y_s = o; o += align_up((size_t)T * H * 4);
    L.xn = o; o += align_up((size_t)T * H * 2);
    L.total = o;
    return L;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Size checks shared by moe_ffn and moe_ffn_workspace_bytes, in the order
// the header documents: shapes, then top-k, then format.
int32_t check_sizes(int32_t T, int32_t H, int32_t E, int32_t I, int32_t Is, int32_t topk,
                    int32_t fmt) {
    if (T < 1 || T > MOE_MAX_T || H < 256 || H % 256 != 0 || I < 64 || I % 64 != 0 ||
        (Is != 0 && (Is < 64 || Is % 64 != 0)) || E < 1 || E > MOE_MAX_E)
        return MOE_E_SHAPE;
    if (topk < 1 || topk > E || topk > MOE_MAX_TOPK) return MOE_E_TOPK;
    if (fmt != MOE_BF16 && fmt != MOE_W4A16 && fmt != MOE_AFFINE4 && fmt != MOE_NVFP4) return MOE_E_FORMAT;
    // MLX affine rows of bf16 scales (and biases) are K / 64 entries, read in
    // 4-byte pieces: K a multiple of 128 keeps them whole and aligned
    if (fmt == MOE_AFFINE4 && I % 128 != 0) return MOE_E_SHAPE;
    return MOE_OK;
}

// Inputs per scale group of a 4-bit format (0: bf16).
int group_of(int fmt) {
    return fmt == MOE_W4A16 ? 32 : (fmt == MOE_AFFINE4 ? 64 : (fmt == MOE_NVFP4 ? 16 : 0));
}

// The 4-bit arrays a format needs, in the order q, s, z of gate/up, q, s, z of
// down, then the NVFP4 matrix scales (z unused by NVFP4, which needs g).
int needed_arrays(const moe_experts* ex, const void** out) {
    const bool nv = ex->fmt == MOE_NVFP4;
    const void* all[8] = {ex->q_gate_up, ex->s_gate_up, nv ? nullptr : ex->z_gate_up, ex->q_down, ex->s_down,
                          nv ? nullptr : ex->z_down, nv ? ex->g_gate_up : nullptr, nv ? ex->g_down : nullptr};
    const bool need[8] = {true, true, !nv, true, true, !nv, nv, nv};
    int n = 0;
    for (int i = 0; i < 8; ++i)
        if (need[i]) out[n++] = all[i];
    return n;
}

struct DeviceInfo {
    bool known = false;
    bool gfx950 = false;
    int num_cu = 0;
};

std::mutex g_dev_mu;
DeviceInfo g_dev[64];

// Per-device properties, queried once per device (a read-only cache).
int32_t device_info(int* num_cu) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_E_HIP;
    if (dev < 0 || dev >= 64) return MOE_E_DEVICE;
    std::lock_guard<std::mutex> lock(g_dev_mu);
    DeviceInfo& d = g_dev[dev];
    if (!d.known) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_E_HIP;
        d.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        d.num_cu = prop.multiProcessorCount;
        d.known = true;
    }
    if (!d.gfx950) return MOE_E_DEVICE;
    *num_cu = d.num_cu;
    return MOE_OK;
}

// The workspace of moe_ffn_static: one array per GPU, loaded with the code
// object and held until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: its address on each device
// comes from hipGetSymbolAddress (static_scratch below).
static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch[64];

// The device address of `scratch` on the current device, looked up once per
// device with that device current.
int32_t static_scratch(void** ptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_E_HIP;
    if (dev < 0 || dev >= 64) return MOE_E_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_E_HIP;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return MOE_OK;
}

// Kernels whose dynamic-LDS limit was raised: the largest size set per
// kernel and device.
std::mutex g_lds_mu;
struct LdsEntry {
    const void* kernel;
    int dev;
    size_t bytes;
};
LdsEntry g_lds[64];
int g_nlds = 0;

// Level of the smallest canonical-tree node containing [lo, hi).
int tree_level(int lo, int hi) {
    int L = 0;
    while ((lo >> L) != ((hi - 1) >> L)) ++L;
    return L;
}

}  // namespace

namespace moe {

void allow_lds_once(const void* kernel, size_t bytes) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return;
    std::lock_guard<std::mutex> lock(g_lds_mu);
    LdsEntry* e = nullptr;
    for (int i = 0; i < g_nlds; ++i)
        if (g_lds[i].kernel == kernel && g_lds[i].dev == dev) e = &g_lds[i];
    if (e && e->bytes >= bytes) return;
    // on failure the error stays pending and the call reports MOE_E_HIP
    if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) !=
        hipSuccess)
        return;
    if (!e && g_nlds < 64) {
        e = &g_lds[g_nlds++];
        e->kernel = kernel;
        e->dev = dev;
    }
    if (e) e->bytes = bytes;
}

}  // namespace moe

extern "C" size_t moe_ffn_workspace_bytes(int32_t T, int32_t H, int32_t E, int32_t I, int32_t Is,
                                          int32_t topk, int32_t fmt) {
    if (check_sizes(T, H, E, I, Is, topk, fmt) != MOE_OK) return 0;
    return make_layout(T, H, E, I, Is, topk).total;
}

extern "C" const char* moe_ffn_strerror(int32_t code) {
    switch (code) {
        case MOE_OK: return "ok";
        case MOE_E_NULL: return "a required pointer is NULL";
        case MOE_E_SHAPE: return "unsupported or inconsistent sizes";
        case MOE_E_DIM: return "router expert count differs from the experts' count";
        case MOE_E_BAND: return "expert band is empty or outside [0, E)";
        case MOE_E_TOPK: return "topk must be in [1, min(E, 16)]";
        case MOE_E_FORMAT: return "unknown expert weight format or group size";
        case MOE_E_WORKSPACE: return "workspace missing or too small";
        case MOE_E_ALIGN: return "a pointer is not 16-byte aligned";
        case MOE_E_HIP: return "HIP runtime error while enqueuing";
        case MOE_E_DEVICE: return "the current device is not a gfx950 GPU";
        case MOE_E_COMBINE: return "unknown combine mode or reduce order";
        case MOE_E_ROUTER: return "unknown router mode";
        case MOE_E_SCRATCH: return "sizes need more scratch than moe_ffn_static's array holds";
        default: return "unknown error code";
    }
}

namespace {

// The layer for moe_ffn and moe_ffn_static.  static_ws: the workspace is
// this device's `scratch` array instead of out->workspace.
int32_t run_layer(const moe_x* x, const moe_router* router_w, const moe_experts* experts,
                  const moe_shared* shared, int32_t band_lo, int32_t band_hi, int32_t topk,
                  const moe_out* out, void* stream, bool static_ws) {
    // ---- argument checks: nothing is enqueued before all of them pass ----
    if (!x || !router_w || !experts || !out) return MOE_E_NULL;
    if (!x->ptr || !router_w->w || !out->y) return MOE_E_NULL;
    const int fmt = experts->fmt;
    const void* qarr[8] = {};
    int nq = 0;
    if (fmt == MOE_BF16) {
        if (!experts->w_gate_up || !experts->w_down) return MOE_E_NULL;
    } else if (group_of(fmt) > 0) {
        nq = needed_arrays(experts, qarr);
        for (int i = 0; i < nq; ++i)
            if (!qarr[i]) return MOE_E_NULL;
    } else {
        return MOE_E_FORMAT;
    }
    if (shared && (!shared->w_gate_up || !shared->w_down)) return MOE_E_NULL;

    const int T = x->T, H = x->H, E = experts->E, I = experts->I;
    const int Is = shared ? shared->Is : 0;
    if (router_w->H != H || experts->H != H || (shared && shared->H != H)) return MOE_E_SHAPE;
    if (shared && Is <= 0) return MOE_E_SHAPE;
    if (router_w->E != E) return MOE_E_DIM;
    if (router_w->mode != MOE_ROUTER_SOFTMAX && router_w->mode != MOE_ROUTER_SIGMOID)
        return MOE_E_ROUTER;
    {
        const int32_t rc = check_sizes(T, H, E, I, Is, topk, fmt);
        if (rc != MOE_OK) return rc;
    }
    if (fmt != MOE_BF16 && experts->group != group_of(fmt)) return MOE_E_FORMAT;
    if (band_lo < 0 || band_hi > E || band_lo >= band_hi) return MOE_E_BAND;
    if (out->combine != MOE_COMBINE_PICK && out->combine != MOE_COMBINE_TREE) return MOE_E_COMBINE;
    if (x->norm_w && !(x->eps >= 0.0f && x->eps < INFINITY)) return MOE_E_SHAPE;

    const bool bf = fmt == MOE_BF16;
    for (int i = 0; i < nq; ++i)
        if (!aligned16(qarr[i])) return MOE_E_ALIGN;
    const void* ptrs[] = {x->ptr, router_w->w, router_w->bias,
                          bf ? experts->w_gate_up : nullptr, bf ? experts->w_down : nullptr,
                          shared ? shared->w_gate_up : nullptr, shared ? shared->w_down : nullptr,
                          out->y, out->topk_ids, out->topk_w, out->counts, out->offsets,
                          out->perm, out->pos, static_ws ? nullptr : out->workspace,
                          out->y_shared, out->y_picks, x->norm_w, out->xn};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MOE_E_ALIGN;

    const Layout L = make_layout(T, H, E, I, Is, topk);
    if (static_ws) {
        if (L.total > (size_t)MOE_STATIC_SCRATCH_BYTES) return MOE_E_SCRATCH;
    } else if (!out->workspace || out->workspace_bytes < L.total) {
        return MOE_E_WORKSPACE;
    }

    int num_cu = 0;
    {
        int32_t rc = device_info(&num_cu);
        if (rc != MOE_OK) return rc;
    }
    void* ws_base = out->workspace;
    if (static_ws) {
        int32_t rc = static_scratch(&ws_base);
        if (rc != MOE_OK) return rc;
    }

    // ---- enqueue ----
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    unsigned char* ws = static_cast<unsigned char*>(ws_base);
    float* logits = reinterpret_cast<float*>(ws + L.logits);
    int32_t* ids = out->topk_ids ? out->topk_ids : reinterpret_cast<int32_t*>(ws + L.ids);
    float* wts = out->topk_w ? out->topk_w : reinterpret_cast<float*>(ws + L.w);
    int32_t* counts = out->counts ? out->counts : reinterpret_cast<int32_t*>(ws + L.counts);
    int32_t* offsets = out->offsets ? out->offsets : reinterpret_cast<int32_t*>(ws + L.offsets);
    int32_t* perm = out->perm ? out->perm : reinterpret_cast<int32_t*>(ws + L.perm);
    int32_t* pos = out->pos ? out->pos : reinterpret_cast<int32_t*>(ws + L.pos);
    int32_t* blkcnt = reinterpret_cast<int32_t*>(ws + L.blkcnt);
    moe::Group* groups = reinterpret_cast<moe::Group*>(ws + L.groups);
    int32_t* gemv_list = reinterpret_cast<int32_t*>(ws + L.gemv_list);
    int32_t* mfma_list = reinterpret_cast<int32_t*>(ws + L.mfma_list);
    int32_t* plan_counts = reinterpret_cast<int32_t*>(ws + L.plan_counts);

    void* const* ev = out->stage_events;
    auto mark = [&](int slot) {
        if (ev) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(ev[slot]), st);
    };

    (void)hipGetLastError();  // clear a stale error so the check below sees only ours

    const int nb = band_hi - band_lo;
    const bool has_shared = shared != nullptr;
    mark(MOE_EV_ROUTER);
    // the layer runs on the normed rows when a norm weight is given; the
    // residual is always the raw rows
    const uint16_t* xin = static_cast<const uint16_t*>(x->ptr);
    if (x->norm_w) {
        uint16_t* xn = out->xn ? static_cast<uint16_t*>(out->xn) : reinterpret_cast<uint16_t*>(ws + L.xn);
        moe::launch_rmsnorm(xin, static_cast<const uint16_t*>(x->norm_w), x->eps, T, H, xn, st);
        xin = xn;
    }
    // softmax: the bias shifts the logits; sigmoid: it steers the selection
    // only and joins at the top-k
    const int sigmoid = router_w->mode == MOE_ROUTER_SIGMOID ? 1 : 0;
    moe::launch_router_logits(xin, router_w->w,
                              sigmoid ? nullptr : router_w->bias, T, H, E, logits, st);
    const float* sel_bias = sigmoid ? router_w->bias : nullptr;
    mark(MOE_EV_TOPK);
    const int mfma_cap = max_mfma_tiles(T, E, topk);
    // With at most kSmallRows rows the shared expert is a GEMV group; its
    // gate/up then runs inside the top-k/dispatch launch (its rows staged in
    // at most 128 KiB of LDS).
    moe::SharedGateUp sg;
    memset(&sg, 0, sizeof sg);
    if (has_shared && T <= moe::kSmallRows && H % 512 == 0 && (size_t)T * H * 2 <= 128 * 1024) {
        sg.x = xin;
        sg.w = static_cast<const uint16_t*>(shared->w_gate_up);
        sg.h = reinterpret_cast<uint16_t*>(ws + L.h_s);
        sg.T = T;
        sg.H = H;
        sg.Is = Is;
        // one block per remaining CU (its LDS holds the rows: one block per
        // CU), fewer when there are fewer column pairs than blocks
        const int free_cu = num_cu - 1 > 1 ? num_cu - 1 : 1;
        sg.blocks = Is < free_cu ? (Is > 0 ? Is : 1) : free_cu;
    }
    if (T <= 16) {
        // block 0: top-k (a wave per row) and the dispatch
        mark(MOE_EV_DISPATCH);
        moe::launch_topk_dispatch_small(logits, sel_bias, sigmoid, E, wts, ids, T, topk, band_lo, band_hi, has_shared, counts,
                                        offsets, perm, pos, groups, gemv_list, mfma_list, mfma_cap,
                                        plan_counts, sg, st);
    } else {
        moe::launch_router_topk(logits, sel_bias, sigmoid, T, E, topk, ids, wts, st);
        mark(MOE_EV_DISPATCH);
        moe::launch_dispatch(ids, T, topk, band_lo, band_hi, has_shared, blkcnt, counts, offsets, perm,
                             pos, groups, gemv_list, mfma_list, mfma_cap, plan_counts, st);
    }

    moe::ExpertArgs a;
    memset(&a, 0, sizeof a);
    a.x = xin;
    a.T = T;
    a.H = H;
    a.topk = topk;
    a.I = I;
    a.fmt = fmt;
    a.wgu = static_cast<const uint16_t*>(experts->w_gate_up);
    a.wd = static_cast<const uint16_t*>(experts->w_down);
    a.qgu = experts->q_gate_up;
    a.sgu = static_cast<const uint16_t*>(experts->s_gate_up);
    a.zgu = static_cast<const uint16_t*>(experts->z_gate_up);
    a.qd = experts->q_down;
    a.sd = static_cast<const uint16_t*>(experts->s_down);
    a.zd = static_cast<const uint16_t*>(experts->z_down);
    a.ggu = fmt == MOE_NVFP4 ? experts->g_gate_up : nullptr;
    a.gd = fmt == MOE_NVFP4 ? experts->g_down : nullptr;
    a.Is = Is;
    a.swgu = shared ? static_cast<const uint16_t*>(shared->w_gate_up) : nullptr;
    a.swd = shared ? static_cast<const uint16_t*>(shared->w_down) : nullptr;
    a.groups = groups;
    a.gemv_list = gemv_list;
    a.mfma_list = mfma_list;
    a.mfma_cap = mfma_cap;
    a.plan_counts = plan_counts;
    a.perm = perm;
    a.h_r = reinterpret_cast<uint16_t*>(ws + L.h_r);
    a.h_s = reinterpret_cast<uint16_t*>(ws + L.h_s);
    // the expert outputs land in the caller's export buffers when given
    a.y_r = out->y_picks ? out->y_picks : reinterpret_cast<float*>(ws + L.y_r);
    const bool shared_apart = has_shared && out->y_shared;
    a.y_s = shared_apart ? out->y_shared : reinterpret_cast<float*>(ws + L.y_s);
    a.shared_gu_done = sg.blocks > 0 ? 1 : 0;

    // Groups on each path: a group has at most T rows (a row picks an expert
    // at most once), so with T <= 8 nothing reaches the MFMA path.
    const long long picks = (long long)T * topk;
    const int max_groups = (int)((picks < nb ? picks : nb) + (has_shared ? 1 : 0));
    const bool mfma_possible = T > moe::kSmallRows;

    mark(MOE_EV_GU_GEMV);
    moe::launch_gateup_gemv(a, max_groups, num_cu, st);
    mark(MOE_EV_GU_MFMA);
    if (mfma_possible) {
        if (fmt == MOE_BF16)
            moe::launch_mfma_pipe(a, true, num_cu, st);
        else
            moe::launch_mfma_w4(a, true, num_cu, st);
    }
    // one row, 4-bit experts, pick order, no per-pick or shared outputs
    // asked for: the down projection and the combine in one launch
    const bool fused_one = out->combine == MOE_COMBINE_PICK && !out->y_picks && !shared_apart &&
                           moe::down_combine_one_ok(a, topk, has_shared);
    const uint16_t* res = out->residual ? static_cast<const uint16_t*>(x->ptr) : nullptr;
    mark(MOE_EV_DN_GEMV);
    if (fused_one)
        moe::launch_down_combine_one(a, ids, pos, wts, topk, res, has_shared, out->y, st);
    else
        moe::launch_down_gemv(a, max_groups, num_cu, st);
    mark(MOE_EV_DN_MFMA);
    if (mfma_possible) {
        if (fmt == MOE_BF16)
            moe::launch_mfma_pipe(a, false, num_cu, st);
        else
            moe::launch_mfma_w4(a, false, num_cu, st);
    }
    mark(MOE_EV_COMBINE);
    const float* add_s = has_shared && !shared_apart ? a.y_s : nullptr;
    if (out->combine == MOE_COMBINE_TREE)
        moe::launch_combine_tree(a.y_r, add_s, res, ids, pos, wts, T, H, topk,
                                 tree_level(band_lo, band_hi), out->y, st);
    else if (!fused_one)  // (the fused launch has combined)
        moe::launch_combine(a.y_r, add_s, res, pos, wts, T, H, topk, out->y, st);
    mark(MOE_EV_END);

    if (hipGetLastError() != hipSuccess) return MOE_E_HIP;
    return MOE_OK;
}

}  // namespace

extern "C" int32_t moe_ffn(const moe_x* x, const moe_router* router_w, const moe_experts* experts,
                           const moe_shared* shared, int32_t band_lo, int32_t band_hi,
                           int32_t topk, const moe_out* out, void* stream) {
    return run_layer(x, router_w, experts, shared, band_lo, band_hi, topk, out, stream, false);
}

extern "C" int32_t moe_ffn_static(const moe_x* x, const moe_router* router_w,
                                  const moe_experts* experts, const moe_shared* shared,
                                  int32_t band_lo, int32_t band_hi, int32_t topk,
                                  const moe_out* out, void* stream) {
    return run_layer(x, router_w, experts, shared, band_lo, band_hi, topk, out, stream, true);
}

extern "C" int32_t moe_ffn_reduce(const float* const* parts, int32_t nparts, const int32_t* band_lo,
                                  const int32_t* band_hi, int32_t E, int32_t order,
                                  const float* y_shared, const void* residual, int32_t T, int32_t H,
                                  float* y, void* stream) {
    if (!parts || !y) return MOE_E_NULL;
    if (order != MOE_REDUCE_RANK && order != MOE_REDUCE_TREE) return MOE_E_COMBINE;
    if (nparts < 1 || nparts > MOE_MAX_PARTS || T < 1 || T > MOE_MAX_T || H < 256 || H % 256 != 0)
        return MOE_E_SHAPE;
    for (int p = 0; p < nparts; ++p) {
        if (!parts[p]) return MOE_E_NULL;
        if (!aligned16(parts[p])) return MOE_E_ALIGN;
    }
    if (!aligned16(y) || (y_shared && !aligned16(y_shared)) || (residual && !aligned16(residual)))
        return MOE_E_ALIGN;

    moe::ReduceProgram pg;
    memset(&pg, 0, sizeof pg);
    pg.nparts = nparts;
    pg.order = order;
    for (int p = 0; p < nparts; ++p) pg.part[p] = parts[p];
    if (order == MOE_REDUCE_TREE) {
        if (!band_lo || !band_hi) return MOE_E_NULL;
        if (E < 1 || E > MOE_MAX_E) return MOE_E_SHAPE;
        // every band a node clipped to [0, E), in order, and so their union
        auto is_node = [&](int lo, int hi, int* lev) {
            if (lo < 0 || hi > E || lo >= hi) return false;
            const int L = tree_level(lo, hi);
            const int end = lo + (1 << L);
            *lev = L;
            return ((lo >> L) << L) == lo && (end < E ? end : E) == hi;
        };
        int ulev = 0;
        if (!is_node(band_lo[0], band_hi[nparts - 1], &ulev)) return MOE_E_BAND;
        int cursor = band_lo[0];
        uint32_t occ = 0;
        auto push = [&](int part, int lev) {
            if (pg.nops >= moe::kMaxReduceOps) return false;
            int l1 = lev;
            while (occ >> l1 & 1u) occ &= ~(1u << l1++);
            occ |= 1u << l1;
            pg.op_part[pg.nops] = (int8_t)part;
            pg.op_l0[pg.nops] = (uint8_t)lev;
            pg.op_l1[pg.nops] = (uint8_t)l1;
            pg.nops += 1;
            return true;
        };
        for (int p = 0; p < nparts; ++p) {
            int lev = 0;
            if (band_lo[p] != cursor || !is_node(band_lo[p], band_hi[p], &lev)) return MOE_E_BAND;
            if (!push(p, lev)) return MOE_E_SHAPE;
            cursor = band_lo[p] + (1 << lev);  // the node's end (past E for the last one)
        }
        // the union's node past the last part: +0.0 nodes, largest first
        const int uend = band_lo[0] + (1 << ulev);
        while (cursor < uend) {
            int lev = 0;
            while (((cursor >> (lev + 1)) << (lev + 1)) == cursor && cursor + (2 << lev) <= uend) ++lev;
            if (!push(-1, lev)) return MOE_E_SHAPE;
            cursor += 1 << lev;
        }
        pg.root_level = ulev;
        if (occ != (1u << ulev)) return MOE_E_BAND;  // not one node: unreachable for a valid tiling
    }

    int num_cu = 0;
    {
        int32_t rc = device_info(&num_cu);
        if (rc != MOE_OK) return rc;
    }
    (void)hipGetLastError();
    moe::launch_reduce(pg, y_shared, static_cast<const uint16_t*>(residual), (size_t)T * H, y,
                       num_cu, reinterpret_cast<hipStream_t>(stream));
    if (hipGetLastError() != hipSuccess) return MOE_E_HIP;
    return MOE_OK;
}

// ---- tensor-parallel slices ----------------------------------------------------

extern "C" int32_t moe_tp_shares(int32_t dim, int32_t unit, int32_t ranks, int32_t* shares) {
    if (!shares) return MOE_E_NULL;
    if (unit < 1 || dim < unit || dim % unit != 0 || ranks < 1 || ranks > dim / unit)
        return MOE_E_SHAPE;
    const int units = dim / unit;
    for (int r = 0; r < ranks; ++r) shares[r] = (units / ranks + (r < units % ranks ? 1 : 0)) * unit;
    return MOE_OK;
}

namespace {

// bytes [b0, b0 + nb) of every row of `rows` rows of `row_bytes` bytes
hipError_t copy_cols(void* dst, const void* src, size_t rows, size_t row_bytes, size_t b0, size_t nb,
                     hipStream_t st) {
    return hipMemcpy2DAsync(dst, nb, static_cast<const unsigned char*>(src) + b0, row_bytes, nb, rows,
                            hipMemcpyDeviceToDevice, st);
}

// gate rows [lo, hi) and up rows [I + lo, I + hi) of E blocks of 2I rows
hipError_t copy_gate_up(void* dst, const void* src, size_t E, size_t I, size_t lo, size_t hi,
                        size_t row_bytes, hipStream_t st) {
    const size_t n = hi - lo;
    // each destination block holds n gate rows then n up rows: two strided
    // copies with a destination pitch of 2n rows
    hipError_t e = hipMemcpy2DAsync(dst, 2 * n * row_bytes,
                                    static_cast<const unsigned char*>(src) + lo * row_bytes,
                                    2 * I * row_bytes, n * row_bytes, E, hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return e;
    return hipMemcpy2DAsync(static_cast<unsigned char*>(dst) + n * row_bytes, 2 * n * row_bytes,
                            static_cast<const unsigned char*>(src) + (I + lo) * row_bytes,
                            2 * I * row_bytes, n * row_bytes, E, hipMemcpyDeviceToDevice, st);
}

}  // namespace

extern "C" int32_t moe_tp_slice_experts(const moe_experts* src, int32_t i_lo, int32_t i_hi,
                                        const moe_experts* dst, void* stream) {
    if (!src || !dst) return MOE_E_NULL;
    const int fmt = src->fmt;
    if (fmt != MOE_BF16 && group_of(fmt) == 0) return MOE_E_FORMAT;
    const int G = group_of(fmt);
    if (dst->fmt != fmt || (G > 0 && (src->group != G || dst->group != G))) return MOE_E_FORMAT;
    const int E = src->E, H = src->H, I = src->I;
    // whole 64-column units, 128 for MLX affine (whose experts need I % 128 == 0)
    const int unit = fmt == MOE_AFFINE4 ? 128 : 64;
    if (E < 1 || E > MOE_MAX_E || H < 256 || H % 256 != 0 || I < unit || I % unit != 0)
        return MOE_E_SHAPE;
    if (i_lo < 0 || i_hi > I || i_lo >= i_hi || i_lo % unit != 0 || i_hi % unit != 0) return MOE_E_SHAPE;
    if (dst->E != E || dst->H != H || dst->I != i_hi - i_lo) return MOE_E_SHAPE;
    const void* need_src[8] = {src->w_gate_up, src->w_down};
    const void* need_dst[8] = {dst->w_gate_up, dst->w_down};
    int nneed = 2;
    if (G > 0) {
        nneed = needed_arrays(src, need_src);
        needed_arrays(dst, need_dst);
    }
    for (int i = 0; i < nneed; ++i) {
        if (!need_src[i] || !need_dst[i]) return MOE_E_NULL;
        if (!aligned16(need_src[i]) || !aligned16(need_dst[i])) return MOE_E_ALIGN;
    }
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const size_t n = (size_t)(i_hi - i_lo);
    hipError_t e = hipSuccess;
    if (fmt == MOE_BF16) {
        e = copy_gate_up(const_cast<void*>(dst->w_gate_up), src->w_gate_up, E, I, i_lo, i_hi, (size_t)H * 2, st);
        if (e == hipSuccess)
            e = copy_cols(const_cast<void*>(dst->w_down), src->w_down, (size_t)E * H, (size_t)I * 2, (size_t)i_lo * 2,
                          n * 2, st);
    } else {
        // bytes of a per-group array per input: a bf16 per G inputs, or an
        // E4M3 byte per 16 (NVFP4)
        const size_t per = fmt == MOE_NVFP4 ? 16 : (size_t)G / 2;  // inputs per byte
        auto cu = [&](const void* d, const void* s_, size_t row_bytes) {
            if (e == hipSuccess) e = copy_gate_up(const_cast<void*>(d), s_, E, I, i_lo, i_hi, row_bytes, st);
        };
        auto cd = [&](const void* d, const void* s_, size_t in_per_byte) {
            if (e == hipSuccess)
                e = copy_cols(const_cast<void*>(d), s_, (size_t)E * H, (size_t)I / in_per_byte,
                              (size_t)i_lo / in_per_byte, n / in_per_byte, st);
        };
        cu(dst->q_gate_up, src->q_gate_up, (size_t)H / 2);
        cu(dst->s_gate_up, src->s_gate_up, (size_t)H / per);
        cd(dst->q_down, src->q_down, 2);
        cd(dst->s_down, src->s_down, per);
        if (fmt == MOE_NVFP4) {
            // the matrix scales belong to whole matrices: every slice keeps them
            if (e == hipSuccess)
                e = hipMemcpyAsync(const_cast<float*>(dst->g_gate_up), src->g_gate_up, (size_t)E * 2 * 4,
                                   hipMemcpyDeviceToDevice, st);
            if (e == hipSuccess)
                e = hipMemcpyAsync(const_cast<float*>(dst->g_down), src->g_down, (size_t)E * 4,
                                   hipMemcpyDeviceToDevice, st);
        } else {
            cu(dst->z_gate_up, src->z_gate_up, (size_t)H / per);
            cd(dst->z_down, src->z_down, per);
        }
    }
    if (e != hipSuccess) return MOE_E_HIP;
    return MOE_OK;
}

extern "C" int32_t moe_tp_slice_shared(const moe_shared* src, int32_t i_lo, int32_t i_hi,
                                       const moe_shared* dst, void* stream) {
    if (!src || !dst || !src->w_gate_up || !src->w_down || !dst->w_gate_up || !dst->w_down)
        return MOE_E_NULL;
    const int H = src->H, Is = src->Is;
    if (H < 256 || H % 256 != 0 || Is < 64 || Is % 64 != 0) return MOE_E_SHAPE;
    if (i_lo < 0 || i_hi > Is || i_lo >= i_hi || i_lo % 64 != 0 || i_hi % 64 != 0) return MOE_E_SHAPE;
    if (dst->H != H || dst->Is != i_hi - i_lo) return MOE_E_SHAPE;
    if (!aligned16(src->w_gate_up) || !aligned16(src->w_down) || !aligned16(dst->w_gate_up) ||
        !aligned16(dst->w_down))
        return MOE_E_ALIGN;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const size_t n = (size_t)(i_hi - i_lo);
    hipError_t e = copy_gate_up(const_cast<void*>(dst->w_gate_up), src->w_gate_up, 1, Is, i_lo, i_hi, (size_t)H * 2, st);
    if (e == hipSuccess)
        e = copy_cols(const_cast<void*>(dst->w_down), src->w_down, (size_t)H, (size_t)Is * 2, (size_t)i_lo * 2, n * 2, st);
    if (e != hipSuccess) return MOE_E_HIP;
    return MOE_OK;
}
