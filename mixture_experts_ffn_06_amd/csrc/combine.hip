// combine.hip -- the weighted sum of each row's in-band expert outputs in pick
// order, then the shared expert, in fp32 with no atomics.
//
// [P1] "GLM-5.2 multi-GPU: expert-parallel sharding + the resident-fit
// benchmark", "What landed": per-rank [H] residual partials, each rank adding
// only the picks it owns; gates table: bit-exact when all picks sit on one
// rank.  [P2] "GLM-5.3-Flash on CUDA: attention on one GPU, routed experts on
// the Sparks (proposal) #214", "Per MoE layer": partials summed in a fixed
// (rank) order.  [P4] "GLM-5.3-Flash on CUDA over three ranks (--tp 3) ...
// #310": fp32 partial rows.
#include "common.h"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_r,
                                                     const float* __restrict__ y_s,
                                                     const int32_t* __restrict__ pos,
                                                     const float* __restrict__ w, int H, int k,
                                                     int ctiles, float* __restrict__ out) {
    const int t = blockIdx.x / ctiles;
    const int c = ((blockIdx.x - t * ctiles) * 256 + threadIdx.x) * 4;
    if (c >= H) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
        const int p = pos[(size_t)t * k + j];
        if (p < 0) continue;
        const float wj = w[(size_t)t * k + j];
        const float4 v = *reinterpret_cast<const float4*>(y_r + (size_t)p * H + c);
        acc.x = __builtin_fmaf(wj, v.x, acc.x);
        acc.y = __builtin_fmaf(wj, v.y, acc.y);
        acc.z = __builtin_fmaf(wj, v.z, acc.z);
        acc.w = __builtin_fmaf(wj, v.w, acc.w);
    }
    if (y_s) {
        const float4 v = *reinterpret_cast<const float4*>(y_s + (size_t)t * H + c);
        acc.x = acc.x + v.x;
        acc.y = acc.y + v.y;
        acc.z = acc.z + v.z;
        acc.w = acc.w + v.w;
    }
    *reinterpret_cast<float4*>(out + (size_t)t * H + c) = acc;
}

void launch_combine(const float* y_r, const float* y_s, const int32_t* pos, const float* w, int T,
                    int H, int k, float* out, hipStream_t st) {
    const int ctiles = (H / 4 + 255) / 256;
    combine_kernel<<<T * ctiles, 256, 0, st>>>(y_r, y_s, pos, w, H, k, ctiles, out);
}

}  // namespace moe
