/*
 * moe_oracle.c -- plain, slow CPU oracle for one routed mixture-of-experts FFN
 * layer restricted to an expert band.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code, header or table with the HIP
 * library; it is written from the method's definition, one row at a time.
 *
 * Pages cited (titles as published):
 *   [P1] "GLM-5.2 multi-GPU: expert-parallel sharding + the resident-fit
 *        benchmark" (fak note)
 *   [P2] "GLM-5.3-Flash on CUDA: attention on one GPU, routed experts on the
 *        Sparks (proposal) #214"
 *   [P4] "GLM-5.3-Flash on CUDA over three ranks (--tp 3) ... #310"
 *   [P5] "GLM-5.3-Flash and full GLM-5.3 on the native CUDA engine (tracker)
 *        #593"
 *
 * Precision: the router logits are fp32 in a fixed reduction order (they
 * decide integers -- the top-k ids -- so both sides take that decision in the
 * same precision and order).  Everything after the selection (softmax
 * weights, SwiGLU, down projection, weighted sum, shared expert) is fp64.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC  (no contraction:
 * every fp32 fused multiply-add below is an explicit fmaf).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_EINVAL (-1)

/* bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits. */
static float bf16_to_f32(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* ------------------------------------------------------------------------ */
/* Router logits.                                                             */
/*                                                                            */
/* [P1] "What landed": the router runs replicated on every rank and picks the */
/* same top-k, so every rank must compute bit-identical logits.  [P5] "What   */
/* exists now" describes the GLM glue as fp32 fixed-order reductions, and     */
/* [P4] (maintainer reply) requires every sum to follow one fixed tree.  The  */
/* fixed order used here (called R-order) is:                                 */
/*   64 partial sums p_l, l = 0..63, each starting at +0.0;                   */
/*   for i = 0..H/256-1 (outer), c = 0..3 (inner):                            */
/*       p_l = fmaf(x[256 i + 4 l + c], w[256 i + 4 l + c], p_l)              */
/*   then six pairwise rounds s = 1,2,4,8,16,32: p_l <- p_l + p_(l xor s);     */
/*   the dot is p_0.  logit = dot + bias (one fp32 add), -0.0 becomes +0.0.   */
/* ------------------------------------------------------------------------ */
float oracle_dot_r(const float* x, const float* w, int H)
{
    float p[64], q[64];
    for (int l = 0; l < 64; ++l) p[l] = 0.0f;
    for (int i = 0; i < H / 256; ++i)
        for (int l = 0; l < 64; ++l)
            for (int c = 0; c < 4; ++c) {
                int k = 256 * i + 4 * l + c;
                p[l] = fmaf(x[k], w[k], p[l]);
            }
    for (int s = 1; s < 64; s <<= 1) {
        for (int l = 0; l < 64; ++l) q[l] = p[l] + p[l ^ s];
        for (int l = 0; l < 64; ++l) p[l] = q[l];
    }
    return p[0];
}

int oracle_router_logits(const uint16_t* x, int T, int H, const float* wr,
                         const float* bias, int E, float* logits)
{
    if (T < 0 || H <= 0 || H % 256 != 0 || E <= 0) return OR_EINVAL;
#pragma omp parallel
    {
        float* xf = (float*)malloc(sizeof(float) * (size_t)H);
#pragma omp for schedule(static)
        for (int t = 0; t < T; ++t) {
            for (int k = 0; k < H; ++k) xf[k] = bf16_to_f32(x[(size_t)t * H + k]);
            for (int e = 0; e < E; ++e) {
                float l = oracle_dot_r(xf, wr + (size_t)e * H, H);
                if (bias) l = l + bias[e];
                if (l == 0.0f) l = 0.0f; /* -0.0 -> +0.0 */
                logits[(size_t)t * E + e] = l;
            }
        }
        free(xf);
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* RMSNorm of the rows before routing.                                        */
/*                                                                            */
/* [P2] "Per MoE layer": the expert side receives the normed rows; [P5]       */
/* "What exists now" lists rmsnorm among the fixed-order fp32 glue kernels,    */
/* and its first byte-gate run found the cross-lane total reaching only some  */
/* lanes, which then ran inv_rms(0) ~ 316x -- 1/sqrt(eps) with eps = 1e-5.    */
/* Every step here is one IEEE fp32 rounding:                                 */
/*   ss  = sum of x[c]^2 in the R-order above (fused multiply-adds);          */
/*   ms  = ss / H;  inv = 1 / sqrt(ms + eps);                                 */
/*   xn[c] = bf16_rne((x[c] * inv) * g[c]).                                   */
/* ------------------------------------------------------------------------ */
static uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u); /* NaN */
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static float rms_inv(const float* xf, int H, float eps)
{
    float ss = oracle_dot_r(xf, xf, H);
    float ms = ss / (float)H;
    float r = sqrtf(ms + eps);
    return 1.0f / r;
}

/* x bf16 [T, H], gamma bf16 [H] -> xn bf16 [T, H]; inv [T] (may be NULL). */
int oracle_rmsnorm(const uint16_t* x, int T, int H, const uint16_t* gamma, float eps,
                   uint16_t* xn, float* inv)
{
    if (T < 0 || H % 256 != 0 || H <= 0) return OR_EINVAL;
    float* xf = (float*)malloc(sizeof(float) * (size_t)H);
    for (int t = 0; t < T; ++t) {
        for (int c = 0; c < H; ++c) xf[c] = bf16_to_f32(x[(size_t)t * H + c]);
        float r = rms_inv(xf, H, eps);
        if (inv) inv[t] = r;
        for (int c = 0; c < H; ++c) {
            float v = xf[c] * r;
            v = v * bf16_to_f32(gamma[c]);
            xn[(size_t)t * H + c] = f32_to_bf16_rne(v);
        }
    }
    free(xf);
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Top-k selection and renormalised weights, one row.                         */
/*                                                                            */
/* [P2] "Per MoE layer": the expert side receives the rows with their top-k   */
/* ids and weights.  The workload fixes a softmax router whose top-k weights  */
/* are renormalised to sum to one.  Order: logit descending, expert id        */
/* ascending on ties (softmax is monotone, so selecting on logits is          */
/* selecting on probabilities).  The weights are the softmax over the k picks */
/* -- the full softmax's denominator cancels in the renormalisation.          */
/* ------------------------------------------------------------------------ */
static void topk_row(const float* l, int E, int k, int32_t* ids, double* w)
{
    unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (taken[e]) continue;
            if (best < 0 || l[e] > l[best]) best = e; /* strict: ties keep lower id */
        }
        taken[best] = 1;
        ids[j] = best;
    }
    free(taken);
    double m = (double)l[ids[0]];
    double s = 0.0;
    for (int j = 0; j < k; ++j) {
        w[j] = exp((double)l[ids[j]] - m);
        s += w[j];
    }
    for (int j = 0; j < k; ++j) w[j] = w[j] / s;
}

int oracle_topk(const float* logits, int T, int E, int k, int32_t* ids, double* w)
{
    if (T < 0 || E <= 0 || k < 1 || k > E) return OR_EINVAL;
    for (int t = 0; t < T; ++t)
        topk_row(logits + (size_t)t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k);
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Sigmoid router with a selection bias.                                      */
/*                                                                            */
/* [P5] "What exists now": GLM's own router (glm_route) is sigmoid + bias     */
/* top-k with raw-score weights.  Reading: score s_e = sigmoid(l_e) of the    */
/* unbiased logit; experts are ordered by (s_e + bias_e descending, id        */
/* ascending), -0.0 counting as +0.0; the weight of pick j is its raw score   */
/* s_{id_j}, not renormalised.  The selection turns on fp32 values, so the    */
/* sigmoid is a fixed fp32 computation that both sides write out in full:     */
/*   exp_c(x): n = rint(x * log2(e)) (fp32 product, ties to even);           */
/*             r = fma(-n, LN2_HI, x); r = fma(-n, LN2_LO, r) with LN2_HI =   */
/*             0.693145751953125 (exact in 16 bits) and LN2_LO = the fp32    */
/*             value nearest ln 2 - LN2_HI;                                   */
/*             p = Horner over the Taylor terms 1/i!, i = 6 down to 0, with  */
/*             fp32 coefficients (nearest to 1/i!): p = fma(p, r, c_i);       */
/*             exp_c = p * 2^n (exact scaling; overflow to +inf);            */
/*             x > 88.8 gives +inf and x < -104 gives +0 directly.            */
/*   sigmoid_c(l) = 1 / (1 + exp_c(-l)), each operation one IEEE fp32         */
/*             rounding (correctly rounded division).                          */
/* ------------------------------------------------------------------------ */
static const float EXPC_LOG2E = 1.44269504088896341f;
static const float EXPC_LN2_HI = 0.693145751953125f;
static const float EXPC_LN2_LO = 1.42860682030941723212e-6f;

float oracle_exp_c(float x)
{
    if (x > 88.8f) return INFINITY;
    if (x < -104.0f) return 0.0f;
    float t = x * EXPC_LOG2E;
    float n = rintf(t);
    float r = fmaf(-n, EXPC_LN2_HI, x);
    r = fmaf(-n, EXPC_LN2_LO, r);
    /* 1/i! for i = 6..0, each rounded to the nearest fp32 */
    const float c[7] = {(float)(1.0 / 720.0), (float)(1.0 / 120.0), (float)(1.0 / 24.0),
                        (float)(1.0 / 6.0), 0.5f, 1.0f, 1.0f};
    float p = c[0];
    for (int i = 1; i < 7; ++i) p = fmaf(p, r, c[i]);
    return ldexpf(p, (int)n);
}

float oracle_sigmoid_c(float l)
{
    float e = oracle_exp_c(-l);
    float d = 1.0f + e;
    return 1.0f / d;
}

/* Row of unbiased logits -> k picks by (score + bias desc, id asc) and their */
/* raw scores. */
static void topk_sigmoid_row(const float* l, const float* bias, int E, int k, int32_t* ids,
                             double* w)
{
    float* key = (float*)malloc(sizeof(float) * (size_t)E);
    float* sc = (float*)malloc(sizeof(float) * (size_t)E);
    unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
    for (int e = 0; e < E; ++e) {
        sc[e] = oracle_sigmoid_c(l[e]);
        float v = bias ? sc[e] + bias[e] : sc[e];
        if (v == 0.0f) v = 0.0f;
        key[e] = v;
    }
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (taken[e]) continue;
            if (best < 0 || key[e] > key[best]) best = e; /* strict: ties keep lower id */
        }
        taken[best] = 1;
        ids[j] = best;
        w[j] = (double)sc[best];
    }
    free(key);
    free(sc);
    free(taken);
}

int oracle_topk_sigmoid(const float* logits, const float* bias, int T, int E, int k, int32_t* ids,
                        double* w)
{
    if (T < 0 || E <= 0 || k < 1 || k > E) return OR_EINVAL;
    for (int t = 0; t < T; ++t)
        topk_sigmoid_row(logits + (size_t)t * E, bias, E, k, ids + (size_t)t * k, w + (size_t)t * k);
    return OR_OK;
}


/* ------------------------------------------------------------------------ */
/* Dispatch for the band [lo, hi).                                            */
/*                                                                            */
/* [P1] "What landed": each rank contributes only the picks it owns.  The     */
/* grouping of picks by expert is the batched dispatch of [P1]'s lever table  */
/* ("batched expert dispatch"), and [P5] gates the device grouping plan as    */
/* byte-equal to the host routing.  Definition:                               */
/*   counts[e-lo]  = #{(t,j) : ids[t,j] = e}                                  */
/*   offsets       = exclusive prefix sum of counts (length nb+1)             */
/*   perm          = for e = lo..hi-1, then t ascending, then j: t*k + j      */
/*   pos[t*k + j]  = index of that pick in perm, or -1 outside the band.      */
/* Returns the number of in-band picks, or OR_EINVAL.                         */
/* ------------------------------------------------------------------------ */
int oracle_dispatch(const int32_t* ids, int T, int k, int lo, int hi,
                    int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos)
{
    if (T < 0 || k < 1 || lo < 0 || hi <= lo) return OR_EINVAL;
    int nb = hi - lo;
    for (int e = 0; e < nb; ++e) counts[e] = 0;
    for (int p = 0; p < T * k; ++p) {
        int e = ids[p];
        if (e >= lo && e < hi) counts[e - lo] += 1;
    }
    offsets[0] = 0;
    for (int e = 0; e < nb; ++e) offsets[e + 1] = offsets[e] + counts[e];
    for (int p = 0; p < T * k; ++p) pos[p] = -1;
    int cursor = 0;
    for (int e = lo; e < hi; ++e)
        for (int t = 0; t < T; ++t)
            for (int j = 0; j < k; ++j)
                if (ids[t * k + j] == e) {
                    perm[cursor] = t * k + j;
                    pos[t * k + j] = cursor;
                    cursor += 1;
                }
    return cursor;
}

/* ------------------------------------------------------------------------ */
/* The canonical tree over expert ids.                                        */
/*                                                                            */
/* [P4] (maintainer reply): every sum follows one fixed tree of slices,       */
/* however the slices fall over ranks, so all ranks hold the same bits.  The  */
/* tree used here is the complete binary tree over expert ids 0..E'-1, E' the */
/* least power of two >= E.  A row's leaf e holds its weighted expert output  */
/* w_j * y_j when e is its pick j inside the band, and +0.0 otherwise (the    */
/* leaves E..E'-1 are always +0.0); an inner node holds left + right.  A band */
/* call returns the value of the smallest node containing its band.  Below,   */
/* a node with no leaf set is +0.0 (the sum of +0.0 leaves), every other      */
/* node is the sum of its two children, computed as written: the plain dense  */
/* definition, with the shortcut for empty nodes only.                        */
/* ------------------------------------------------------------------------ */

/* Level of the smallest node containing [lo, hi): the least L such that lo  */
/* and hi-1 agree above bit L-1.  Its first leaf is lo with the low L bits    */
/* cleared. */
int oracle_tree_node(int E, int lo, int hi, int* node_lo, int* level)
{
    if (E < 1 || lo < 0 || hi > E || lo >= hi) return OR_EINVAL;
    int L = 0;
    while ((lo >> L) != ((hi - 1) >> L)) L += 1;
    *node_lo = (lo >> L) << L;
    *level = L;
    return OR_OK;
}

/* Value of node [node_lo, node_lo + 2^level) for one column: ids[i] are the  */
/* leaf positions of the set leaves, vals[i] their fp32 values (ids distinct, */
/* any order). */
static float tree_value_f(int node_lo, int level, const int32_t* ids, const float* vals, int m)
{
    int size = 1 << level;
    int found = -1, cnt = 0;
    for (int i = 0; i < m; ++i)
        if (ids[i] >= node_lo && ids[i] < node_lo + size) {
            found = i;
            cnt += 1;
        }
    if (cnt == 0) return 0.0f;
    if (level == 0) return vals[found];
    float left = tree_value_f(node_lo, level - 1, ids, vals, m);
    float right = tree_value_f(node_lo + size / 2, level - 1, ids, vals, m);
    return left + right;
}

/* The same tree in fp64, for the layer below. */
static double tree_value_d(int node_lo, int level, const int32_t* ids, const double* vals, int m)
{
    int size = 1 << level;
    int found = -1, cnt = 0;
    for (int i = 0; i < m; ++i)
        if (ids[i] >= node_lo && ids[i] < node_lo + size) {
            found = i;
            cnt += 1;
        }
    if (cnt == 0) return 0.0;
    if (level == 0) return vals[found];
    double left = tree_value_d(node_lo, level - 1, ids, vals, m);
    double right = tree_value_d(node_lo + size / 2, level - 1, ids, vals, m);
    return left + right;
}

/* Node values for n columns: vals is [m, n] (row i = leaf ids[i]), out [n]. */
int oracle_tree_value(const int32_t* ids, const float* vals, int m, int node_lo, int level,
                      size_t n, float* out)
{
    if (m < 0 || level < 0 || level > 20) return OR_EINVAL;
    float* col = (float*)malloc(sizeof(float) * (size_t)(m > 0 ? m : 1));
    for (size_t c = 0; c < n; ++c) {
        for (int i = 0; i < m; ++i) col[i] = vals[(size_t)i * n + c];
        out[c] = tree_value_f(node_lo, level, ids, col, m);
    }
    free(col);
    return OR_OK;
}

/* Value of node [nlo, nlo + 2^lev) from parts whose nodes tile it: part p    */
/* covers node (plo[p], plev[p]); a node past E with no part is +0.0. */
static float merge_value(int nlo, int lev, int E, int nparts, const int* plo, const int* plev,
                         const float* const* parts, size_t c)
{
    for (int p = 0; p < nparts; ++p)
        if (plo[p] == nlo && plev[p] == lev) return parts[p][c];
    if (nlo >= E) return 0.0f;
    if (lev == 0) return 0.0f; /* unreachable for a valid tiling */
    float left = merge_value(nlo, lev - 1, E, nparts, plo, plev, parts, c);
    float right = merge_value(nlo + (1 << (lev - 1)), lev - 1, E, nparts, plo, plev, parts, c);
    return left + right;
}

/* Sum of band partials along the canonical tree.  Part p is the output of a */
/* band call for [lo[p], hi[p]); the bands must tile a range [U_lo, U_hi) in  */
/* order, each band must be its node clipped to [0, E), and so must the       */
/* range.  out = value of the range's node (+ shared, when not NULL, last);   */
/* parts, shared and out are [n] each.  Returns OR_EINVAL for other bands.   */
int oracle_tree_merge(int E, int nparts, const int32_t* lo, const int32_t* hi,
                      const float* const* parts, const float* shared, size_t n, float* out)
{
    if (nparts < 1) return OR_EINVAL;
    int* plo = (int*)malloc(sizeof(int) * (size_t)nparts);
    int* plev = (int*)malloc(sizeof(int) * (size_t)nparts);
    int ok = 1;
    for (int p = 0; p < nparts && ok; ++p) {
        if (oracle_tree_node(E, lo[p], hi[p], &plo[p], &plev[p]) != OR_OK) ok = 0;
        else if (plo[p] != lo[p]) ok = 0;
        else {
            int end = plo[p] + (1 << plev[p]);
            if ((end < E ? end : E) != hi[p]) ok = 0;
        }
        if (ok && p > 0 && lo[p] != hi[p - 1]) ok = 0;
    }
    int ulo = 0, ulev = 0;
    if (ok && oracle_tree_node(E, lo[0], hi[nparts - 1], &ulo, &ulev) != OR_OK) ok = 0;
    if (ok) {
        int end = ulo + (1 << ulev);
        if (ulo != lo[0] || (end < E ? end : E) != hi[nparts - 1]) ok = 0;
    }
    if (ok)
        for (size_t c = 0; c < n; ++c) {
            float v = merge_value(ulo, ulev, E, nparts, plo, plev, parts, c);
            out[c] = shared ? v + shared[c] : v;
        }
    free(plo);
    free(plev);
    return ok ? OR_OK : OR_EINVAL;
}

/* Sum of rank partials in rank order.  [P4] (maintainer reply and the      */
/* --tp 3 comments): each rank returns a full-width fp32 partial and the      */
/* partials are added in rank order, so the sum is a left fold: ((p0 + p1) +  */
/* p2) + ..., each addition one fp32 rounding; the shared expert's output     */
/* (when not NULL) is added after the partials and the bf16 residual (when    */
/* not NULL, widened exactly) last.  parts [nparts][n], out [n].             */
int oracle_rank_merge(int nparts, const float* const* parts, const float* shared, const uint16_t* residual,
                      size_t n, float* out)
{
    if (nparts < 1) return OR_EINVAL;
    for (size_t c = 0; c < n; ++c) {
        float v = parts[0][c];
        for (int p = 1; p < nparts; ++p) v = v + parts[p][c];
        if (shared) v = v + shared[c];
        if (residual) v = v + bf16_to_f32(residual[c]);
        out[c] = v;
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Tensor-parallel shares.                                                    */
/*                                                                            */
/* [P4] (proposal and comments): a dimension splits in whole units, as evenly */
/* as it goes, with the remainder on the lowest ranks.  units = dim / unit;   */
/* rank r gets floor(units / ranks) units, plus one when r < units mod ranks. */
/* Rejects a dim that is not a positive multiple of unit and more ranks than  */
/* units (a rank would hold nothing).                                         */
/* ------------------------------------------------------------------------ */
int oracle_tp_shares(int dim, int unit, int ranks, int32_t* shares)
{
    if (unit < 1 || dim < unit || dim % unit != 0 || ranks < 1) return OR_EINVAL;
    int units = dim / unit;
    if (ranks > units) return OR_EINVAL;
    for (int r = 0; r < ranks; ++r) shares[r] = (units / ranks + (r < units % ranks ? 1 : 0)) * unit;
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Expert weights.                                                            */
/*                                                                            */
/* bf16: w_gate_up [E, 2I, H] (rows 0..I-1 gate, I..2I-1 up: [P5]'s fused     */
/*       gate/up rows are 2w wide), w_down [E, H, I].                          */
/* w4:   4-bit unsigned codes, two per byte, low nibble = even k, with a bf16 */
/*       scale s and zero z per 32-wide group along k; the weight is          */
/*       (q - z) * s.  [P5] "The pieces, in order" lists W4A16 checkpoints    */
/*       (4-bit weights, 16-bit activations) on the family; [P4] names the    */
/*       group units.                                                         */
/* ------------------------------------------------------------------------ */
/* affine4: MLX's affine 4-bit format ([P5] "The pieces, in order": MLX      */
/*       affine 4-bit checkpoints; [P4] comments: MLX's 64-input groups):     */
/*       4-bit unsigned codes packed as above, a bf16 scale s and bias b per  */
/*       64-wide group along k; the weight is s * q + b.                      */
/* nvfp4: NVIDIA's NVFP4 read as stored ([P5]: NVFP4 checkpoint read as      */
/*       stored, W4A16; [P4] comments: NVFP4's 16-input groups): each 4-bit  */
/*       code is an FP4 E2M1 value (sign bit 3, exponent bits 2..1 with bias  */
/*       1, mantissa bit 0; exponent 0 is subnormal: 0 or 0.5), packed two    */
/*       per byte with the even k in the low nibble; one FP8 E4M3 scale per   */
/*       16-wide group along k (sign, 4 exponent bits with bias 7, 3 mantissa */
/*       bits; exponent 0 subnormal; the all-ones pattern is NaN) and one     */
/*       fp32 scale per matrix (the gate, up and down matrices of an expert   */
/*       each have their own); the weight is fp4(q) * e4m3(s) * g.           */
typedef struct {
    int32_t fmt; /* 0 = bf16, 1 = w4 (group 32), 2 = affine4 (group 64), 3 = nvfp4 (group 16) */
    int32_t E, H, I;
    const uint16_t* w_gate_up;
    const uint16_t* w_down;
    const uint8_t* q_gate_up;
    const uint16_t* s_gate_up; /* w4 and affine4: bf16; nvfp4: E4M3 bytes */
    const uint16_t* z_gate_up; /* w4: zero points; affine4: biases; nvfp4: unused */
    const uint8_t* q_down;
    const uint16_t* s_down;
    const uint16_t* z_down;
    const float* g_gate_up; /* nvfp4: fp32 [E, 2] (gate, up) */
    const float* g_down;    /* nvfp4: fp32 [E] */
} oracle_experts;

/* Row n of a [rows, K] matrix of expert e, as doubles. */
static void bf16_row(const uint16_t* base, size_t rows, int K, int e, int n, double* out)
{
    const uint16_t* r = base + ((size_t)e * rows + (size_t)n) * (size_t)K;
    for (int k = 0; k < K; ++k) out[k] = (double)bf16_to_f32(r[k]);
}

static void w4_row(const uint8_t* q, const uint16_t* s, const uint16_t* z, size_t rows, int K,
                   int e, int n, double* out)
{
    size_t row = (size_t)e * rows + (size_t)n;
    const uint8_t* qr = q + row * (size_t)(K / 2);
    const uint16_t* sr = s + row * (size_t)(K / 32);
    const uint16_t* zr = z + row * (size_t)(K / 32);
    for (int k = 0; k < K; ++k) {
        uint8_t byte = qr[k / 2];
        int code = (k % 2 == 0) ? (byte & 0xF) : (byte >> 4);
        double sc = (double)bf16_to_f32(sr[k / 32]);
        double zr_ = (double)bf16_to_f32(zr[k / 32]);
        out[k] = ((double)code - zr_) * sc;
    }
}

static int code_at(const uint8_t* qr, int k)
{
    uint8_t byte = qr[k / 2];
    return (k % 2 == 0) ? (byte & 0xF) : (byte >> 4);
}

static void affine4_row(const uint8_t* q, const uint16_t* s, const uint16_t* b, size_t rows,
                        int K, int e, int n, double* out)
{
    size_t row = (size_t)e * rows + (size_t)n;
    const uint8_t* qr = q + row * (size_t)(K / 2);
    const uint16_t* sr = s + row * (size_t)(K / 64);
    const uint16_t* br = b + row * (size_t)(K / 64);
    for (int k = 0; k < K; ++k)
        out[k] = (double)bf16_to_f32(sr[k / 64]) * (double)code_at(qr, k) +
                 (double)bf16_to_f32(br[k / 64]);
}

/* FP4 E2M1: (-1)^sign * (exponent ? (1 + m/2) * 2^(exponent - 1) : m/2). */
double oracle_fp4_e2m1(int code)
{
    int sign = (code >> 3) & 1, ex = (code >> 1) & 3, m = code & 1;
    double mag = ex ? (1.0 + 0.5 * m) * ldexp(1.0, ex - 1) : 0.5 * m;
    return sign ? -mag : mag;
}

/* FP8 E4M3: (-1)^sign * (exponent ? (1 + m/8) * 2^(exponent - 7) : m/8 * 2^-6);
 * exponent 15 with mantissa 7 is NaN (there is no infinity). */
double oracle_fp8_e4m3(int byte)
{
    int sign = (byte >> 7) & 1, ex = (byte >> 3) & 15, m = byte & 7;
    if (ex == 15 && m == 7) return NAN;
    double mag = ex ? (1.0 + m / 8.0) * ldexp(1.0, ex - 7) : (m / 8.0) * ldexp(1.0, -6);
    return sign ? -mag : mag;
}

static void nvfp4_row(const uint8_t* q, const uint8_t* s, double g, size_t rows, int K, int e,
                      int n, double* out)
{
    size_t row = (size_t)e * rows + (size_t)n;
    const uint8_t* qr = q + row * (size_t)(K / 2);
    const uint8_t* sr = s + row * (size_t)(K / 16);
    for (int k = 0; k < K; ++k)
        out[k] = oracle_fp4_e2m1(code_at(qr, k)) * oracle_fp8_e4m3(sr[k / 16]) * g;
}

static void gate_up_row(const oracle_experts* ex, int e, int n, double* out)
{
    size_t rows = 2 * (size_t)ex->I;
    if (ex->fmt == 0) bf16_row(ex->w_gate_up, rows, ex->H, e, n, out);
    else if (ex->fmt == 1) w4_row(ex->q_gate_up, ex->s_gate_up, ex->z_gate_up, rows, ex->H, e, n, out);
    else if (ex->fmt == 2)
        affine4_row(ex->q_gate_up, ex->s_gate_up, ex->z_gate_up, rows, ex->H, e, n, out);
    else /* the gate rows take the expert's gate scale, the up rows its up scale */
        nvfp4_row(ex->q_gate_up, (const uint8_t*)ex->s_gate_up,
                  (double)ex->g_gate_up[2 * (size_t)e + (n < ex->I ? 0 : 1)], rows, ex->H, e, n, out);
}

static void down_row(const oracle_experts* ex, int e, int n, double* out)
{
    size_t rows = (size_t)ex->H;
    if (ex->fmt == 0) bf16_row(ex->w_down, rows, ex->I, e, n, out);
    else if (ex->fmt == 1) w4_row(ex->q_down, ex->s_down, ex->z_down, rows, ex->I, e, n, out);
    else if (ex->fmt == 2) affine4_row(ex->q_down, ex->s_down, ex->z_down, rows, ex->I, e, n, out);
    else nvfp4_row(ex->q_down, (const uint8_t*)ex->s_down, (double)ex->g_down[e], rows, ex->I, e, n, out);
}

static double dot(const double* a, const double* b, int n)
{
    double s = 0.0;
    for (int i = 0; i < n; ++i) s += a[i] * b[i];
    return s;
}

/* ------------------------------------------------------------------------ */
/* One expert's SwiGLU FFN on one row: y = W_down (silu(W_gate x) * W_up x),  */
/* silu(g) = g / (1 + exp(-g)).  [P1] "Update (later 2026-06-29)" names the   */
/* per-expert expertSwiGLU; [P5] "What exists now" fixes the fused gate/up    */
/* rows as 2w wide.  fp64 throughout.                                          */
/* ------------------------------------------------------------------------ */
int oracle_expert_ffn(const double* x, const oracle_experts* ex, int e, double* y)
{
    if (e < 0 || e >= ex->E) return OR_EINVAL;
    int H = ex->H, I = ex->I;
    double* row = (double*)malloc(sizeof(double) * (size_t)(H > I ? H : I));
    double* h = (double*)malloc(sizeof(double) * (size_t)I);
    for (int i = 0; i < I; ++i) {
        gate_up_row(ex, e, i, row);
        double g = dot(row, x, H);
        gate_up_row(ex, e, I + i, row);
        double u = dot(row, x, H);
        h[i] = g / (1.0 + exp(-g)) * u;
    }
    for (int c = 0; c < H; ++c) {
        down_row(ex, e, c, row);
        y[c] = dot(row, h, I);
    }
    free(row);
    free(h);
    return OR_OK;
}

/* The shared expert: the same SwiGLU FFN with its own bf16 weights
 * [2Is, H] and [H, Is], applied to every row with weight 1 ([P1] gates table:
 * GLM shared-expert wrapper; [P2] "Per MoE layer": the shared expert runs
 * alongside the routed ones). */
static void shared_ffn(const double* x, const uint16_t* wgu, const uint16_t* wd, int H, int Is,
                       double* y)
{
    oracle_experts sh;
    memset(&sh, 0, sizeof sh);
    sh.fmt = 0;
    sh.E = 1;
    sh.H = H;
    sh.I = Is;
    sh.w_gate_up = wgu;
    sh.w_down = wd;
    oracle_expert_ffn(x, &sh, 0, y);
}

/* ------------------------------------------------------------------------ */
/* The layer, one row at a time.                                              */
/*                                                                            */
/* For each listed row t:                                                     */
/*   logits over all E experts whatever the band ([P1]: the router runs       */
/*   replicated and picks the same top-k); top-k ids in pick order and their  */
/*   renormalised weights; then, in pick order j = 0..k-1 and only for picks  */
/*   with lo <= id < hi ([P1]: each rank contributes only the picks it owns), */
/*   acc += w_j * FFN_{id_j}(x_t), acc starting at +0.0; then, if a shared     */
/*   expert is given, acc += FFN_shared(x_t) last.  The result is the row's    */
/*   partial residual for the band ([P1]: per-rank [H] residual partials;     */
/*   [P2]: partials summed in rank order).  combine = 1 sums the weighted     */
/*   outputs along the canonical tree instead (the value of the smallest node */
/*   containing the band, see above), then adds the shared expert.             */
/*                                                                            */
/* rows == NULL means rows 0..T-1 (nrows must equal T).  out is [nrows, H];   */
/* ids_out [nrows, k] and w_out [nrows, k] may be NULL.                        */
/* ------------------------------------------------------------------------ */
static int layer_rows(const uint16_t* x, int T, int H, const float* wr, const float* bias, int E,
                      const oracle_experts* ex, const uint16_t* sh_wgu, const uint16_t* sh_wd,
                      int Is, int use_band, int lo, int hi, int k, int combine, int router,
                      const uint16_t* gamma, float eps, int residual,
                      const int32_t* rows, int nrows, double* out, int32_t* ids_out,
                      double* w_out)
{
    if (T < 1 || H % 256 != 0 || E < 1 || k < 1 || k > E) return OR_EINVAL;
    if (combine != 0 && combine != 1) return OR_EINVAL;
    if (router != 0 && router != 1) return OR_EINVAL;
    int node_lo = 0, node_lev = 0;
    if (combine == 1 && oracle_tree_node(E, use_band ? lo : 0, use_band ? hi : E, &node_lo,
                                         &node_lev) != OR_OK)
        return OR_EINVAL;
    if (ex->E != E || ex->H != H) return OR_EINVAL;
    if (use_band && (lo < 0 || hi > E || lo >= hi)) return OR_EINVAL;
    if (!rows && nrows != T) return OR_EINVAL;
    int status = OR_OK;
    for (int r = 0; r < nrows; ++r) {
        int t = rows ? rows[r] : r;
        if (t < 0 || t >= T) return OR_EINVAL;
    }
    /* Three steps per chunk of rows, each a plain loop that OpenMP spreads
     * over the host's cores: (1) per row, the normed row, the logits and the
     * picks; (2) per (row, in-band pick) and per (row, shared expert), that
     * expert's FFN on the row -- so a few rows still keep every core busy;
     * (3) per row, the weighted sum in pick order (or along the tree), then
     * the shared expert, then the residual.  The arithmetic of each output is
     * the same as a row-at-a-time loop would do, in the same order. */
    const int slots = k + 1; /* the row's picks, then its shared expert */
    int chunk = (int)((size_t)(64u << 20) / ((size_t)slots * (size_t)H * sizeof(double)));
    if (chunk < 1) chunk = 1;
    if (chunk > nrows) chunk = nrows > 0 ? nrows : 1;
    double* xd = (double*)malloc(sizeof(double) * (size_t)chunk * H);
    double* xres = (double*)malloc(sizeof(double) * (size_t)chunk * H);
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)chunk * k);
    double* w = (double*)malloc(sizeof(double) * (size_t)chunk * k);
    double* ys = (double*)malloc(sizeof(double) * (size_t)chunk * slots * H);
    int32_t* task = (int32_t*)malloc(sizeof(int32_t) * (size_t)chunk * slots);
    const int has_shared = sh_wgu && sh_wd;
    for (int r0 = 0; r0 < nrows; r0 += chunk) {
        const int nr = nrows - r0 < chunk ? nrows - r0 : chunk;
        /* (1) routing */
#pragma omp parallel
        {
            float* xf = (float*)malloc(sizeof(float) * (size_t)H);
            float* l = (float*)malloc(sizeof(float) * (size_t)E);
#pragma omp for schedule(dynamic, 1)
            for (int i = 0; i < nr; ++i) {
                int t = rows ? rows[r0 + i] : r0 + i;
                double* xdi = xd + (size_t)i * H;
                double* xri = xres + (size_t)i * H;
                for (int c = 0; c < H; ++c) xf[c] = bf16_to_f32(x[(size_t)t * H + c]);
                if (gamma) {
                    /* the layer sees the normed rows; the residual is the raw row */
                    float ri = rms_inv(xf, H, eps);
                    for (int c = 0; c < H; ++c) {
                        xri[c] = (double)xf[c];
                        float v = xf[c] * ri;
                        v = v * bf16_to_f32(gamma[c]);
                        xf[c] = bf16_to_f32(f32_to_bf16_rne(v));
                    }
                } else {
                    for (int c = 0; c < H; ++c) xri[c] = (double)xf[c];
                }
                for (int c = 0; c < H; ++c) xdi[c] = (double)xf[c];
                for (int e = 0; e < E; ++e) {
                    float v = oracle_dot_r(xf, wr + (size_t)e * H, H);
                    if (bias && router == 0) v = v + bias[e];
                    if (v == 0.0f) v = 0.0f;
                    l[e] = v;
                }
                if (router == 0)
                    topk_row(l, E, k, ids + (size_t)i * k, w + (size_t)i * k);
                else
                    topk_sigmoid_row(l, bias, E, k, ids + (size_t)i * k, w + (size_t)i * k);
            }
            free(xf);
            free(l);
        }
        /* (2) one expert FFN per task: slot j < k is pick j (when in the
         * band), slot k the shared expert */
        int ntask = 0;
        for (int i = 0; i < nr; ++i)
            for (int j = 0; j < slots; ++j) {
                if (j < k) {
                    int e = ids[(size_t)i * k + j];
                    if (use_band && (e < lo || e >= hi)) continue;
                } else if (!has_shared) {
                    continue;
                }
                task[ntask++] = i * slots + j;
            }
#pragma omp parallel for schedule(dynamic, 1)
        for (int q = 0; q < ntask; ++q) {
            int i = task[q] / slots, j = task[q] % slots;
            double* y = ys + (size_t)task[q] * H;
            if (j < k)
                oracle_expert_ffn(xd + (size_t)i * H, ex, ids[(size_t)i * k + j], y);
            else
                shared_ffn(xd + (size_t)i * H, sh_wgu, sh_wd, H, Is, y);
        }
        /* (3) the sums */
#pragma omp parallel
        {
            double* leaf = (double*)malloc(sizeof(double) * (size_t)k * H);
            int32_t* leaf_id = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
            double* col = (double*)malloc(sizeof(double) * (size_t)k);
#pragma omp for schedule(dynamic, 1)
            for (int i = 0; i < nr; ++i) {
                const int32_t* idi = ids + (size_t)i * k;
                const double* wi = w + (size_t)i * k;
                double* acc = out + (size_t)(r0 + i) * H;
                for (int c = 0; c < H; ++c) acc[c] = 0.0;
                int m = 0;
                for (int j = 0; j < k; ++j) {
                    if (use_band && (idi[j] < lo || idi[j] >= hi)) continue;
                    const double* y = ys + ((size_t)i * slots + j) * H;
                    if (combine == 0) {
                        for (int c = 0; c < H; ++c) acc[c] += wi[j] * y[c];
                    } else {
                        for (int c = 0; c < H; ++c) leaf[(size_t)m * H + c] = wi[j] * y[c];
                        leaf_id[m++] = idi[j];
                    }
                }
                if (combine == 1)
                    for (int c = 0; c < H; ++c) {
                        for (int q = 0; q < m; ++q) col[q] = leaf[(size_t)q * H + c];
                        acc[c] = tree_value_d(node_lo, node_lev, leaf_id, col, m);
                    }
                if (has_shared) {
                    const double* y = ys + ((size_t)i * slots + k) * H;
                    for (int c = 0; c < H; ++c) acc[c] += y[c];
                }
                if (residual)
                    for (int c = 0; c < H; ++c) acc[c] += xres[(size_t)i * H + c];
                if (ids_out)
                    for (int j = 0; j < k; ++j) ids_out[(size_t)(r0 + i) * k + j] = idi[j];
                if (w_out)
                    for (int j = 0; j < k; ++j) w_out[(size_t)(r0 + i) * k + j] = wi[j];
            }
            free(leaf);
            free(leaf_id);
            free(col);
        }
    }
    free(xd);
    free(xres);
    free(ids);
    free(w);
    free(ys);
    free(task);
    return status;
}

/* The layer restricted to the expert band [lo, hi). */
int oracle_moe_ffn(const uint16_t* x, int T, int H, const float* wr, const float* bias, int E,
                   const oracle_experts* ex, const uint16_t* sh_wgu, const uint16_t* sh_wd, int Is,
                   int lo, int hi, int k, int combine, int router, const uint16_t* gamma,
                   float eps, int residual, const int32_t* rows, int nrows, double* out,
                   int32_t* ids_out, double* w_out)
{
    return layer_rows(x, T, H, wr, bias, E, ex, sh_wgu, sh_wd, Is, 1, lo, hi, k, combine, router,
                      gamma, eps, residual, rows, nrows, out, ids_out, w_out);
}

/* The routed monolith: the same layer with no band logic at all (every pick
 * contributes).  [P1] gates table: EP with one rank must equal it bit for bit. */
int oracle_moe_ffn_monolith(const uint16_t* x, int T, int H, const float* wr, const float* bias,
                            int E, const oracle_experts* ex, const uint16_t* sh_wgu,
                            const uint16_t* sh_wd, int Is, int k, const int32_t* rows, int nrows,
                            double* out)
{
    return layer_rows(x, T, H, wr, bias, E, ex, sh_wgu, sh_wd, Is, 0, 0, E, k, 0, 0, NULL, 0.0f, 0,
                      rows, nrows, out, NULL, NULL);
}

/* Dequantised weight matrix of one expert, for pins that compare the 4-bit
 * decode against a known matrix.  which = 0: gate/up [2I, H]; 1: down [H, I]. */
int oracle_expert_matrix(const oracle_experts* ex, int e, int which, double* out)
{
    if (e < 0 || e >= ex->E) return OR_EINVAL;
    if (which == 0) {
        for (int n = 0; n < 2 * ex->I; ++n) gate_up_row(ex, e, n, out + (size_t)n * ex->H);
    } else {
        for (int n = 0; n < ex->H; ++n) down_row(ex, e, n, out + (size_t)n * ex->I);
    }
    return OR_OK;
}
