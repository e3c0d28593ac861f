/*
 * moe_ffn.h -- C ABI of libmoeffn.so: one routed mixture-of-experts FFN layer,
 * restricted to an expert band, on an AMD Instinct MI355X (gfx950).
 *
 * Pages this interface follows (titles as published):
 *   [P1] "GLM-5.2 multi-GPU: expert-parallel sharding + the resident-fit
 *        benchmark" -- "What landed": experts partitioned into contiguous
 *        bands, a replicated router picking the same top-k on every rank,
 *        each rank contributing only the picks it owns, per-rank [H] residual
 *        partials; the gates table (band of one rank == routed monolith,
 *        fail-closed plan checks, shared-expert wrapper).
 *   [P2] "GLM-5.3-Flash on CUDA: attention on one GPU, routed experts on the
 *        Sparks (proposal) #214" -- "Per MoE layer": rows go to the expert
 *        side with their top-k ids and weights, partials are summed in rank
 *        order, the shared expert runs alongside.
 *   [P4] "GLM-5.3-Flash on CUDA over three ranks (--tp 3) ... #310" --
 *        fp32 partial rows summed in a fixed order.
 *   [P5] "GLM-5.3-Flash and full GLM-5.3 on the native CUDA engine (tracker)
 *        #593" -- fused gate/up rows 2w wide; W4A16 checkpoints; device
 *        grouping plan byte-equal to the host routing.
 *
 * What one call computes (for the band [band_lo, band_hi) of the E experts):
 *   1. router logits l[t,e] = dot(x[t,:], Wr[e,:]) + bias[e] in fp32, for ALL
 *      E experts whatever the band ([P1]: the router runs replicated), summed
 *      in a fixed order (64 lane partials over k = 256 i + 4 l + c, i outer,
 *      c inner, fused multiply-adds from +0.0, then six pairwise rounds
 *      l xor 1, 2, 4, 8, 16, 32), -0.0 normalised to +0.0;
 *   2. top-k: experts ordered by (logit descending, id ascending), the first
 *      topk in that pick order (the order is unspecified for NaN logits,
 *      which only non-finite inputs produce); weights w_j = exp(l_j - l_0) / sum_i exp(l_i -
 *      l_0) over the picks (softmax renormalised over the picks);
 *   3. dispatch of the in-band picks by expert (counts, offsets, a stable
 *      permutation ascending in row, and its inverse);
 *   4. per in-band expert: h = silu(x W_gate^T) * (x W_up^T), y = h W_down^T
 *      (SwiGLU; silu(g) = g / (1 + exp(-g)));
 *   5. out[t,:] = sum over picks j in pick order with the expert in the band
 *      of w_j * y_j, accumulated in fp32 from +0.0, then + the shared
 *      expert's output (weight 1) when `shared` is not NULL.  With
 *      moe_out.combine = MOE_COMBINE_TREE the routed sum follows the
 *      canonical tree over expert ids instead (below).
 * The full band [0, E) gives the whole layer (the routed monolith plus the
 * shared expert).  Summing the outputs of consecutive bands in band order
 * gives the whole layer up to fp32 reassociation; in tree mode, summing the
 * outputs of bands that are tree nodes along the tree (moe_ffn_reduce) gives
 * it bit for bit.
 *
 * The canonical tree ([P4] maintainer reply: every sum follows one fixed tree
 * of slices however the slices fall over ranks, so every rank holds the same
 * bits): the complete binary tree over expert ids 0..E'-1, E' the least
 * power of two >= E.  For row t, leaf e holds w_j * y_j (one fp32 product)
 * when e is the row's pick j and lies in the band, else +0.0; an inner node
 * holds left + right (fp32).  A node is the range [a 2^L, (a+1) 2^L) of
 * leaves; a call returns the value of the smallest node containing
 * [band_lo, band_hi).  Bands that are nodes (clipped to [0, E)) are the
 * pieces moe_ffn_reduce can add back together exactly; every contiguous band
 * is a run of such nodes.
 *
 * Memory: every pointer is device memory owned by the caller, contiguous
 * row-major, 16-byte aligned.  The library never allocates device memory;
 * scratch lives in the caller's workspace (moe_ffn) or in one static array
 * per GPU (moe_ffn_static).  Its only host-side state is write-once, per
 * device and under a lock: the device's properties, the address of the
 * static array, and the dynamic-LDS limit set per kernel and device
 * (hipFuncSetAttribute, called again only for a larger size).
 * Execution: all work is enqueued asynchronously on `stream`; nothing is
 * copied back to the host and nothing waits for the GPU.  Calls on different
 * streams need different workspaces.
 * Errors: every argument check runs before the first enqueue; on error
 * nothing is enqueued and no output is written ([P1] gates table:
 * fail-closed).  Runs are bit-identical from call to call for the same
 * inputs (no floating-point atomics; every reduction has a fixed order).
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define MOE_OK 0
#define MOE_E_NULL (-1)      /* a required pointer is NULL */
#define MOE_E_SHAPE (-2)     /* T < 1 or too large; H differs between arguments; H % 256 != 0;
                                I or Is not a positive multiple of 64 (I of MOE_AFFINE4
                                experts: of 128); E > MOE_MAX_E */
#define MOE_E_DIM (-3)       /* router E != experts E ([P1]: plan.Dim != NumExperts) */
#define MOE_E_BAND (-4)      /* band_lo < 0, band_hi > E or band_lo >= band_hi */
#define MOE_E_TOPK (-5)      /* topk < 1, topk > E or topk > MOE_MAX_TOPK */
#define MOE_E_FORMAT (-6)    /* unknown weight format, or a group size other than the format's */
#define MOE_E_WORKSPACE (-7) /* workspace NULL or smaller than moe_ffn_workspace_bytes() */
#define MOE_E_ALIGN (-8)     /* a pointer is not 16-byte aligned */
#define MOE_E_HIP (-9)       /* the HIP runtime reported an error while enqueuing */
#define MOE_E_DEVICE (-10)   /* the current device is not a gfx950 GPU */
#define MOE_E_COMBINE (-11)  /* unknown combine mode or reduce order */
#define MOE_E_ROUTER (-12)   /* unknown router mode */
#define MOE_E_SCRATCH (-13)  /* moe_ffn_static: the sizes need more than MOE_STATIC_SCRATCH_BYTES */

#define MOE_MAX_TOPK 16
#define MOE_MAX_PARTS 64 /* partials one moe_ffn_reduce call adds */
#define MOE_MAX_E 1024
#define MOE_MAX_T (1 << 20)

/* Expert weight formats ([P5] "The pieces, in order": the family's 4-bit
 * checkpoints -- W4A16, MLX affine 4-bit, NVIDIA's NVFP4 read as stored; [P4]
 * comments: NVFP4's 16-input groups, MLX's 64).  Activations stay bf16. */
#define MOE_BF16 0    /* bf16 weights */
#define MOE_W4A16 1   /* 4-bit unsigned codes, bf16 scale and zero per 32 inputs */
#define MOE_AFFINE4 2 /* MLX affine: 4-bit unsigned codes, bf16 scale and bias per 64 inputs */
#define MOE_NVFP4 3   /* FP4 E2M1 codes, FP8 E4M3 scale per 16 inputs, fp32 scale per matrix */

/* Rows: x is bf16 [T, H].  With norm_w (bf16 [H]) the layer runs on the
 * RMSNorm of the rows ([P2] "Per MoE layer": the expert side receives the
 * normed rows; [P5] "What exists now": rmsnorm is a fixed-order fp32 glue
 * kernel whose inv_rms(0) is about 316, i.e. eps = 1e-5): per row, the sum of
 * squares in the router's fixed order (step 1 below), ms = ss / H,
 * inv = 1 / sqrt(ms + eps) (correctly rounded), xn = bf16((x * inv) * norm_w)
 * (round to nearest even); router and experts read xn.  eps must be finite
 * and >= 0 (else MOE_E_SHAPE). */
typedef struct moe_x {
    const void* ptr; /* bf16 [T, H] */
    int32_t T, H;
    const void* norm_w; /* bf16 [H] or NULL: no norm */
    float eps;
} moe_x;

/* Router modes. */
#define MOE_ROUTER_SOFTMAX 0 /* steps 1-2 above: the bias shifts the logits */
#define MOE_ROUTER_SIGMOID 1 /* sigmoid + bias top-k, raw-score weights */

/* Router: fp32 gate weight [E, H] and an optional fp32 per-expert bias [E].
 * MOE_ROUTER_SOFTMAX: the bias is added to the logits before selection and
 * weighting.  MOE_ROUTER_SIGMOID ([P5] "What exists now": GLM's glm_route is
 * sigmoid + bias top-k with raw-score weights): score s_e = sigmoid(l_e) of
 * the unbiased logit; experts are ordered by (s_e + bias_e descending, id
 * ascending, -0.0 as +0.0); the weight of a pick is its raw score s_e, not
 * renormalised.  The selection turns on fp32 values, so the sigmoid is fixed
 * step by step: exp_c(x) = p(r) * 2^n with n = rint(x * log2(e)) (fp32
 * product, ties to even), r = fma(-n, ln2_lo, fma(-n, ln2_hi, x)) where
 * ln2_hi = 0.693145751953125 and ln2_lo is the fp32 value nearest
 * ln 2 - ln2_hi, p(r) the Taylor terms 1/i! (i = 6..0, nearest fp32) in
 * Horner form with fused multiply-adds; exp_c(x) = +inf for x > 88.8 and +0
 * for x < -104; sigmoid(l) = 1 / (1 + exp_c(-l)), IEEE fp32 operations. */
typedef struct moe_router {
    const float* w;    /* fp32 [E, H] */
    const float* bias; /* fp32 [E] or NULL */
    int32_t E, H;
    int32_t mode; /* MOE_ROUTER_SOFTMAX or MOE_ROUTER_SIGMOID */
} moe_router;

/* Routed experts, all E of them (the band selects which ones run).
 * MOE_BF16:  w_gate_up bf16 [E, 2I, H] -- rows 0..I-1 are the gate
 *            projection, rows I..2I-1 the up projection ([P5]: the fused
 *            gate/up rows are 2w wide); w_down bf16 [E, H, I].
 * The 4-bit formats store two codes per byte, the even input index in the low
 * nibble: q_gate_up uint8 [E, 2I, H/2], q_down uint8 [E, H, I/2] (gate rows
 * first, as above), with per-group arrays of G consecutive inputs:
 * MOE_W4A16:   G = 32; s_gate_up, z_gate_up bf16 [E, 2I, H/32], s_down,
 *              z_down bf16 [E, H, I/32]; weight = (code - zero) * scale.
 * MOE_AFFINE4: G = 64 (MLX affine 4-bit); s_* bf16 scales, z_* bf16 biases,
 *              [E, 2I, H/64] and [E, H, I/64]; weight = scale * code + bias;
 *              I a multiple of 128 (whole 4-byte pieces of the down arrays).
 * MOE_NVFP4:   G = 16 (NVIDIA's NVFP4 as stored); a code is an FP4 E2M1
 *              value (bit 3 sign, bits 2..1 exponent with bias 1, bit 0
 *              mantissa; exponent 0 gives 0 or 0.5); s_gate_up uint8
 *              [E, 2I, H/16] and s_down uint8 [E, H, I/16] are FP8 E4M3
 *              scales (bias 7, exponent 0 subnormal, 0x7f / 0xff NaN);
 *              g_gate_up fp32 [E, 2] (each expert's gate, then up matrix
 *              scale) and g_down fp32 [E]; weight = e2m1(code) * e4m3(scale)
 *              * matrix scale; z_* unused.
 * group must equal the format's G (ignored for MOE_BF16).  Unused pointers of
 * the other formats are ignored. */
typedef struct moe_experts {
    int32_t E, H, I;
    int32_t fmt;   /* MOE_BF16, MOE_W4A16, MOE_AFFINE4 or MOE_NVFP4 */
    int32_t group; /* 32, 64 or 16 for the 4-bit formats; ignored for MOE_BF16 */
    const void* w_gate_up;
    const void* w_down;
    const uint8_t* q_gate_up;
    const void* s_gate_up;
    const void* z_gate_up;
    const uint8_t* q_down;
    const void* s_down;
    const void* z_down;
    const float* g_gate_up; /* MOE_NVFP4: fp32 [E, 2] */
    const float* g_down;    /* MOE_NVFP4: fp32 [E] */
} moe_experts;

/* Shared expert (unrouted, weight 1, every row): bf16 w_gate_up [2Is, H]
 * (gate rows first), w_down [H, Is]. */
typedef struct moe_shared {
    int32_t Is, H;
    const void* w_gate_up;
    const void* w_down;
} moe_shared;

/* Event slots recorded on the stream when moe_out.stage_events is set: slot
 * s is recorded just before stage s is enqueued (also when the stage has no
 * work for this call), and slot MOE_EV_END after the last stage. */
#define MOE_EV_ROUTER 0   /* router logits */
#define MOE_EV_TOPK 1     /* top-k and weights */
#define MOE_EV_DISPATCH 2 /* histogram, scan, permutation, tile lists */
#define MOE_EV_GU_GEMV 3  /* gate/up + SwiGLU, groups of <= 8 rows */
#define MOE_EV_GU_MFMA 4  /* gate/up + SwiGLU, groups of > 8 rows (MFMA) */
#define MOE_EV_DN_GEMV 5  /* down projection, groups of <= 8 rows */
#define MOE_EV_DN_MFMA 6  /* down projection, groups of > 8 rows (MFMA) */
#define MOE_EV_COMBINE 7  /* weighted sum in pick order + shared */
#define MOE_EV_END 8
#define MOE_NUM_EVENTS 9

/* Order of the routed sum (moe_out.combine). */
#define MOE_COMBINE_PICK 0 /* pick order (descending logit), fp32 fused multiply-adds */
#define MOE_COMBINE_TREE 1 /* the canonical tree over expert ids */

/* Outputs.  y is required and fully overwritten (rows with no in-band pick
 * and no shared expert become +0.0).  The other outputs are optional exports
 * of the routing and dispatch (NULL = not exported):
 *   topk_ids int32 [T, topk] and topk_w fp32 [T, topk], in pick order;
 *   counts int32 [nb], offsets int32 [nb + 1] (nb = band_hi - band_lo);
 *   perm int32 [T*topk]: entries 0..N_in-1 hold t*topk + j of the in-band
 *        picks grouped by expert (band order), rows ascending within an
 *        expert; entries past N_in = offsets[nb] are left unspecified;
 *   pos int32 [T*topk]: the index of pick t*topk + j in perm, or -1 when the
 *        pick is outside the band.
 * workspace: device scratch of at least moe_ffn_workspace_bytes() bytes.
 * stage_events: NULL, or MOE_NUM_EVENTS hipEvent_t handles (created by the
 *        caller) recorded at the stage boundaries, for timing.
 * y_shared: NULL, or fp32 [T, H]: the shared expert's output is written
 *        there and not added to y (for moe_ffn_reduce, which adds it after
 *        the partials); ignored without a shared expert.
 * y_picks: NULL, or fp32 [T*topk, H]: row i receives the expert output of
 *        pick perm[i] before weighting (rows past N_in unspecified).
 * combine: MOE_COMBINE_PICK (0) or MOE_COMBINE_TREE.
 * residual: nonzero adds the raw rows x (not the normed ones) to y last, after
 *        the shared expert ([P2]: the partials are the rows' residual updates).
 * xn: NULL, or bf16 [T, H] receiving the normed rows (only with norm_w). */
typedef struct moe_out {
    float* y; /* fp32 [T, H] */
    int32_t* topk_ids;
    float* topk_w;
    int32_t* counts;
    int32_t* offsets;
    int32_t* perm;
    int32_t* pos;
    void* workspace;
    size_t workspace_bytes;
    void* const* stage_events;
    float* y_shared;
    float* y_picks;
    int32_t combine;
    int32_t residual;
    void* xn;
} moe_out;

/* Run the layer for the band [band_lo, band_hi) on `stream` (a hipStream_t;
 * NULL = the null stream).  shared may be NULL.  Returns MOE_OK or a
 * negative MOE_E_* code. */
int32_t moe_ffn(const moe_x* x, const moe_router* router_w, const moe_experts* experts,
                const moe_shared* shared, int32_t band_lo, int32_t band_hi, int32_t topk,
                const moe_out* out, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): moe_ffn
 * with its scratch in a static array of MOE_STATIC_SCRATCH_BYTES bytes per
 * GPU instead of a caller's workspace.  The array is part of the library's
 * code object: each GPU the library runs on holds it from the first use
 * until the process ends.  Arguments, results and errors are moe_ffn's,
 * except that out->workspace and out->workspace_bytes are ignored and sizes
 * whose workspace (moe_ffn_workspace_bytes) exceeds the array return
 * MOE_E_SCRATCH before anything is enqueued.  It calls no allocating routine.
 * Nothing in the array has to start at zero: every call writes each scratch
 * value before reading it, so the previous call's contents do no harm.  All
 * calls on one GPU share the array: calls that overlap on one GPU (on
 * different streams, or from several threads without ordering) race and
 * must be serialised by the caller. */
#define MOE_STATIC_SCRATCH_BYTES (32u << 20)
int32_t moe_ffn_static(const moe_x* x, const moe_router* router_w, const moe_experts* experts,
                       const moe_shared* shared, int32_t band_lo, int32_t band_hi, int32_t topk,
                       const moe_out* out, void* stream);

/* Workspace bytes a call with these sizes needs (Is = 0: no shared expert).
 * Returns 0 for sizes moe_ffn would reject. */
size_t moe_ffn_workspace_bytes(int32_t T, int32_t H, int32_t E, int32_t I, int32_t Is,
                               int32_t topk, int32_t fmt);

/* Orders of moe_ffn_reduce. */
#define MOE_REDUCE_RANK 0 /* ((p_0 + p_1) + p_2) + ...: rank (band) order */
#define MOE_REDUCE_TREE 1 /* along the canonical tree over expert ids */

/* The exchange step of an expert-parallel layer, on one GPU: add the fp32
 * partials of several band calls ([P2] "Per MoE layer" and [P4]: the ranks'
 * fp32 partials summed in rank order; [P4] maintainer reply: one fixed tree
 * of slices), then the shared expert's output, then a residual.
 *   parts: host array of nparts device pointers, fp32 [T, H] each
 *          (1 <= nparts <= MOE_MAX_PARTS);
 *   band_lo, band_hi: host arrays [nparts], the band of each part.  They are
 *          read only by MOE_REDUCE_TREE (may be NULL for MOE_REDUCE_RANK),
 *          where the bands must follow each other ([lo_0, hi_0), [hi_0, hi_1),
 *          ...), each must be a tree node clipped to [0, E) (its band call
 *          returned that node's value), and so must their union; y is then
 *          the value of the union's node;
 *   y_shared: NULL or fp32 [T, H], added after the partials;
 *   residual: NULL or bf16 [T, H], added last;
 *   y: fp32 [T, H] output (may be parts[0] for MOE_REDUCE_RANK).
 * Errors as for moe_ffn (MOE_E_BAND for bands that break the rule above,
 * MOE_E_COMBINE for an unknown order); nothing is enqueued on error. */
int32_t moe_ffn_reduce(const float* const* parts, int32_t nparts, const int32_t* band_lo,
                       const int32_t* band_hi, int32_t E, int32_t order, const float* y_shared,
                       const void* residual, int32_t T, int32_t H, float* y, void* stream);

/* Tensor-parallel expert slices ([P4] "GLM-5.3-Flash on CUDA over three
 * ranks (--tp 3) ... #310": every rank holds a whole-unit slice of each
 * expert's intermediate columns and returns a full-width fp32 partial; the
 * partials are added in rank order, i.e. moe_ffn_reduce with
 * MOE_REDUCE_RANK).  A rank's slice is an expert set of its own (I = its
 * share), so moe_ffn runs it unchanged; the functions below give the shares
 * and lay a rank's slice out from full weights.
 *
 * Shares of dim over ranks: whole units of `unit`, as even as it goes, the
 * remainder on the lowest ranks (the page's examples: 2048 columns in 128-wide
 * units over three ranks -> 768/640/640, in 64-wide units -> 704/704/640).
 * shares: host int32 [ranks].  MOE_E_SHAPE when dim is not a positive
 * multiple of unit, ranks < 1 or ranks > dim / unit.  Host only. */
int32_t moe_tp_shares(int32_t dim, int32_t unit, int32_t ranks, int32_t* shares);

/* Copy intermediate columns [i_lo, i_hi) of every routed expert -- gate rows
 * i_lo..i_hi-1, up rows I+i_lo..I+i_hi-1 and the same inputs of the down
 * projection (codes and per-group arrays alike for the 4-bit formats; the
 * NVFP4 matrix scales are copied whole) -- into dst, an
 * expert set of the same E, H and format with I = i_hi - i_lo whose arrays
 * the caller allocated.  i_lo and i_hi are multiples of 64 (of 128 for
 * MOE_AFFINE4) with 0 <= i_lo < i_hi <= I.  Device-to-device copies enqueued on stream; errors
 * as for moe_ffn (MOE_E_SHAPE for a slice outside the rule). */
int32_t moe_tp_slice_experts(const moe_experts* src, int32_t i_lo, int32_t i_hi,
                             const moe_experts* dst, void* stream);

/* The same for the shared expert: columns [i_lo, i_hi) of Is. */
int32_t moe_tp_slice_shared(const moe_shared* src, int32_t i_lo, int32_t i_hi,
                            const moe_shared* dst, void* stream);

/* A static, human-readable message for a return code. */
const char* moe_ffn_strerror(int32_t code);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_H */
