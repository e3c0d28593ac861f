"""GPU: the one-row down projection with the combine folded in.

At T = 1 with 4-bit routed experts (K = I = Is = 2048, at most 8 picks, pick
order, no per-pick or separate shared outputs asked for) the library runs the
down projection and the pick-order combine as one token-major launch
([P2] "GLM-5.3-Flash on CUDA: attention on one GPU, routed experts on the
Sparks (proposal) #214", "Per MoE layer": each token's expert outputs come
back as one weighted sum; [P1] gates table: the fixed-order combine).  Asking
for the per-pick outputs (y_picks) runs the two separate launches instead, so
the pair of calls below compares the fused path with the unfused one: the
outputs must agree bit for bit, and both must match the oracle.
"""

import pytest
import torch

import mixture_experts_ffn_06_amd as moe
import synth
from gpu_common import OracleSide, check_routing, compare, gpu_inputs, log

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
FORMATS = ["w4", "affine4", "nvfp4"]


def _pair(w, d, lo=0, hi=None, shared=True, topk=None, residual=False):
    hi = w.E if hi is None else hi
    k = w.topk if topk is None else topk
    sh = d["shared"] if shared else None
    ex = {}
    fused = moe.moe_ffn(d["x"], d["router_w"], d["bias"], d["experts"], sh, lo, hi, k, exports=ex,
                        residual=residual)
    picks = torch.empty((k, w.H), dtype=torch.float32, device="cuda")
    plain = moe.moe_ffn(d["x"], d["router_w"], d["bias"], d["experts"], sh, lo, hi, k, y_picks=picks,
                        residual=residual)
    torch.cuda.synchronize()
    return fused, plain, ex


@pytest.mark.parametrize("fmt", FORMATS)
def test_full_size_fused_equals_unfused_and_oracle(fmt):
    w = W[f"{fmt}_t1"]
    d = gpu_inputs(w)
    fused, plain, ex = _pair(w, d)
    assert torch.equal(fused, plain), "fused one-row launch differs from down + combine"
    side = OracleSide(w, d)
    check_routing(ex, side, 0, w.E)
    compare(fused, side.layer([0], 0, w.E), f"one row {fmt}")
    again, _, _ = _pair(w, d)
    assert torch.equal(again, fused), "run-to-run bits differ"


SMALL = synth.Workload("one", T=1, H=1024, E=32, topk=8, I=2048, Is=2048)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("topk,lo,hi,shared,residual", [
    (8, 0, 32, True, False),
    (8, 0, 32, False, True),
    (4, 0, 32, True, True),
    (1, 0, 32, True, False),
    (8, 8, 24, True, False),    # some picks outside the band
    (8, 30, 32, False, False),  # most picks outside the band, maybe none inside
])
def test_small_shapes_fused_equals_unfused(fmt, topk, lo, hi, shared, residual):
    w = SMALL.with_(fmt=fmt, topk=topk)
    d = gpu_inputs(w)
    d["bias"] = (-0.1 * torch.arange(w.E, dtype=torch.float32)).cuda()
    fused, plain, ex = _pair(w, d, lo, hi, shared=shared, residual=residual)
    assert torch.equal(fused, plain), f"{fmt} k={topk} band [{lo},{hi}) shared={shared} residual={residual}"
    inband = int(((ex["topk_ids"] >= lo) & (ex["topk_ids"] < hi)).sum())
    log(f"{fmt} k={topk} band [{lo},{hi}): {inband} picks in band, bit-equal")
    if not residual:
        side = OracleSide(w, d)
        ref = side.layer([0], lo, hi, shared=shared)
        if float(ref.abs().max()) == 0:
            assert float(fused.abs().max()) == 0
        else:
            compare(fused, ref, f"one row {fmt} k={topk} [{lo},{hi})")


@pytest.mark.parametrize("fmt", FORMATS)
def test_more_than_eight_picks_take_the_separate_launches(fmt):
    # k = 12 is past the fused launch's limit: the layer still matches the oracle
    w = SMALL.with_(fmt=fmt, topk=12)
    d = gpu_inputs(w)
    fused, plain, ex = _pair(w, d)
    assert torch.equal(fused, plain)
    side = OracleSide(w, d)
    check_routing(ex, side, 0, w.E)
    compare(fused, side.layer([0], 0, w.E), f"one row {fmt} k=12")
