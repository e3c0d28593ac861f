"""GPU: the sigmoid router (selection on sigmoid(l) + bias, raw-score weights).

[P5] "GLM-5.3-Flash and full GLM-5.3 on the native CUDA engine (tracker)
#593", "What exists now": GLM's router is sigmoid + bias top-k with raw-score
weights.  The ids must match the oracle bit for bit, so the fp32 sigmoid is
fixed step by step on both sides; the exported weights (the picks' raw
scores) are compared bit for bit too.
"""

import numpy as np
import pytest
import torch

import mixture_experts_ffn_06_amd as moe
import synth
from gpu_common import OracleSide, compare, gpu_inputs, log, sample_rows
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
MID = synth.Workload("mid", T=300, H=512, E=16, topk=4, I=192, Is=128)


def _run(w, d, router="sigmoid", lo=0, hi=None, shared=True):
    ex = {}
    y = moe.moe_ffn(d["x"], d["router_w"], d["bias"], d["experts"], d["shared"] if shared else None,
                    lo, w.E if hi is None else hi, w.topk, exports=ex, router=router)
    torch.cuda.synchronize()
    return y, ex


def _oracle_routing(d, k):
    lg = orc.router_logits(d["x"].cpu(), d["router_w"].cpu(), None)
    return orc.topk_sigmoid(lg, None if d["bias"] is None else d["bias"].cpu(), k)


def _check_exact(ex, ids, wts):
    assert torch.equal(ex["topk_ids"].cpu(), ids), "ids differ from the oracle"
    gw = ex["topk_w"].cpu()
    assert torch.equal(gw.view(torch.int32), wts.float().view(torch.int32)), "raw scores differ"


def test_sigmoid_values_bit_exact_over_a_sweep():
    # row t is one-hot at column t, so logit_e = Wr[e, t] exactly; with
    # k = E = 16 every expert is a pick and its weight is sigmoid(logit)
    E, H, T = 16, 1024, 1024
    w = synth.Workload("sweep", T=T, H=H, E=E, topk=16, I=64, Is=64)
    d = gpu_inputs(w)
    x = torch.zeros(T, H, dtype=torch.bfloat16)
    x[torch.arange(T), torch.arange(T)] = 1.0
    d["x"] = x.cuda()
    g = torch.Generator().manual_seed(9)
    wr = torch.empty(E, H).uniform_(-40.0, 40.0, generator=g)
    wr[:, :64] = torch.linspace(-1e-3, 1e-3, 64)  # near zero
    wr[0, 64:80] = torch.tensor([0.0, -0.0, 88.0, -88.0, 100.0, -110.0, 1e-30, -1e-30,
                                 0.5, -0.5, 16.635532, -16.635532, 87.33654, -87.33654, 20.0, 1.0])
    d["router_w"] = wr.cuda()
    d["bias"] = None
    y, ex = _run(w, d, shared=False)
    ids, wts = _oracle_routing(d, 16)
    _check_exact(ex, ids, wts)
    log(f"{T * E} sigmoid values bit-exact")


@pytest.mark.parametrize("wname", ["mid", "decode", "prefill", "w4_t2048"])
def test_sigmoid_routing_bit_exact(wname):
    w = MID if wname == "mid" else W[wname]
    d = gpu_inputs(w)
    if d["bias"] is None:
        d["bias"] = (torch.linspace(-0.05, 0.05, w.E)).cuda()
    y, ex = _run(w, d)
    ids, wts = _oracle_routing(d, w.topk)
    _check_exact(ex, ids, wts)
    counts, offsets, perm, pos = orc.dispatch(ids, 0, w.E)
    assert torch.equal(ex["counts"].cpu()[: w.E], counts)
    assert torch.equal(ex["perm"].cpu()[: perm.numel()], perm)
    assert torch.equal(ex["pos"].cpu(), pos)
    log(f"{wname}: sigmoid routing bit-exact, largest group {int(counts.max())}")


@pytest.mark.parametrize("fmt", ["bf16", "w4"])
def test_sigmoid_layer_against_the_oracle(fmt):
    w = MID.with_(fmt=fmt)
    d = gpu_inputs(w)
    d["bias"] = (0.02 * torch.arange(w.E, dtype=torch.float32)).cuda()
    side = OracleSide(w, d)
    y, _ = _run(w, d)
    rows = list(range(w.T))
    need = set(int(e) for e in _oracle_routing(d, w.topk)[0].flatten().tolist())
    side._fetch(need)
    inputs = {"x": side.x, "router_w": side.wr, "bias": side.bias, "experts": side._experts,
              "shared": side.shared}
    ref, _, _ = orc.moe_ffn(inputs, w.E, w.I, w.Is, 0, w.E, w.topk,
                            rows=torch.tensor(rows, dtype=torch.int32), router="sigmoid")
    compare(y, ref, f"sigmoid layer {fmt}")


def test_sigmoid_decode_full_size_layer():
    w = W["decode"]
    d = gpu_inputs(w)
    d["bias"] = torch.linspace(-0.1, 0.1, w.E).cuda()
    y, ex = _run(w, d)
    side = OracleSide(w, d)
    need = set(int(e) for e in ex["topk_ids"].cpu().flatten().tolist())
    side._fetch(need)
    inputs = {"x": side.x, "router_w": side.wr, "bias": side.bias, "experts": side._experts,
              "shared": side.shared}
    ref, ids, _ = orc.moe_ffn(inputs, w.E, w.I, w.Is, 0, w.E, w.topk, router="sigmoid")
    assert torch.equal(ids, ex["topk_ids"].cpu())
    compare(y, ref, "sigmoid decode")


def test_bias_steers_selection_only():
    w = MID
    d = gpu_inputs(w)
    d["bias"] = torch.zeros(w.E).cuda()
    d["bias"][[5, 11]] = 10.0
    y, ex = _run(w, d)
    ids = ex["topk_ids"].cpu()
    assert (ids[:, :2].sort(dim=1).values == torch.tensor([5, 11], dtype=torch.int32)).all()
    lg = orc.router_logits(d["x"].cpu(), d["router_w"].cpu(), None)
    for t in range(0, w.T, 37):
        for j in range(w.topk):
            e = int(ids[t, j])
            assert float(ex["topk_w"][t, j]) == orc.sigmoid_c(float(lg[t, e]))


def test_unknown_router_mode_rejected():
    w = MID
    d = gpu_inputs(w)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_ffn(d["x"], d["router_w"], d["bias"], d["experts"], d["shared"], 0, w.E, w.topk,
                    router=7)
    assert e.value.code == -12
