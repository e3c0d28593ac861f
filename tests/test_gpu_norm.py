"""GPU: RMSNorm of the rows before routing, and the residual add.

[P2] "GLM-5.3-Flash on CUDA: attention on one GPU, routed experts on the
Sparks (proposal) #214", "Per MoE layer": the expert side receives the normed
rows.  [P5] "GLM-5.3-Flash and full GLM-5.3 on the native CUDA engine
(tracker) #593", "What exists now": rmsnorm is a fixed-order fp32 glue kernel;
its first byte-gate run found the cross-lane total reaching only some lanes
(inv_rms(0) ~ 316x).  The normed rows feed the router, so they are compared
bit for bit with the oracle's.
"""

import pytest
import torch

import mixture_experts_ffn_06_amd as moe
import synth
from gpu_common import OracleSide, compare, gpu_inputs, log, sample_rows
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
MID = synth.Workload("mid", T=300, H=512, E=16, topk=4, I=192, Is=128)


def _gamma(H, seed=1):
    g = torch.Generator().manual_seed(seed)
    return (1.0 + 0.05 * torch.randn(H, generator=g)).to(torch.bfloat16)


def _run(w, d, gamma, residual=False, combine="pick", xn=None, exports=True):
    ex = {} if exports else None
    y = moe.moe_ffn(d["x"], d["router_w"], d["bias"], d["experts"], d["shared"], 0, w.E, w.topk,
                    exports=ex, norm=gamma.cuda(), residual=residual, combine=combine, xn=xn)
    torch.cuda.synchronize()
    return y, ex


@pytest.mark.parametrize("wname", ["mid", "decode", "prefill", "w4_t2048"])
def test_normed_rows_and_ids_bit_exact(wname):
    w = MID if wname == "mid" else W[wname]
    d = gpu_inputs(w)
    gamma = _gamma(w.H)
    xn = torch.empty((w.T, w.H), dtype=torch.bfloat16, device="cuda")
    y, ex = _run(w, d, gamma, xn=xn)
    want, _ = orc.rmsnorm(d["x"].cpu(), gamma)
    assert torch.equal(xn.cpu().view(torch.int16), want.view(torch.int16)), "normed rows differ"
    lg = orc.router_logits(want, d["router_w"].cpu(), None if d["bias"] is None else d["bias"].cpu())
    ids, wts = orc.topk(lg, w.topk)
    assert torch.equal(ex["topk_ids"].cpu(), ids)
    log(f"{wname}: {w.T} normed rows and ids bit-exact")


def test_normed_rows_adversarial():
    w = MID.with_(T=64)
    d = gpu_inputs(w)
    x = d["x"].cpu().float()
    x[0] = 0.0                                    # inv_rms(0) = 1/sqrt(eps)
    x[1] = 0.0
    x[1, 252:256] = torch.tensor([3.0, -4.0, 12.0, 1.0])  # one lane's elements only
    x[2] = 0.0
    x[2, 511] = 1.0                               # the last element only
    x[3:10] *= 1e-3
    x[10:20] *= 1e3
    x[20] = 1.0                                   # constant row
    d["x"] = x.to(torch.bfloat16).cuda()
    gamma = _gamma(w.H, 2)
    xn = torch.empty((w.T, w.H), dtype=torch.bfloat16, device="cuda")
    _run(w, d, gamma, xn=xn)
    want, inv = orc.rmsnorm(d["x"].cpu(), gamma)
    assert torch.equal(xn.cpu().view(torch.int16), want.view(torch.int16))
    assert abs(float(inv[0]) - 316.2278) < 1e-3


@pytest.mark.parametrize("fmt", ["bf16", "w4", "affine4", "nvfp4"])
def test_norm_and_residual_layer_against_the_oracle(fmt):
    w = MID.with_(fmt=fmt, I=256 if fmt == "affine4" else MID.I)  # MLX affine needs I % 128 == 0
    d = gpu_inputs(w)
    gamma = _gamma(w.H, 3)
    y, ex = _run(w, d, gamma, residual=True)
    side = OracleSide(w, d)
    need = set(int(e) for e in ex["topk_ids"].cpu().flatten().tolist())
    side._fetch(need)
    inputs = {"x": side.x, "router_w": side.wr, "bias": side.bias, "experts": side._experts,
              "shared": side.shared}
    ref, ids, _ = orc.moe_ffn(inputs, w.E, w.I, w.Is, 0, w.E, w.topk, norm=gamma, residual=True)
    assert torch.equal(ids, ex["topk_ids"].cpu())
    compare(y, ref, f"norm+residual {fmt}")


def test_norm_decode_full_size_layer():
    w = W["decode"]
    d = gpu_inputs(w)
    gamma = _gamma(w.H, 4)
    y, ex = _run(w, d, gamma, residual=True)
    side = OracleSide(w, d)
    side._fetch(set(int(e) for e in ex["topk_ids"].cpu().flatten().tolist()))
    inputs = {"x": side.x, "router_w": side.wr, "bias": side.bias, "experts": side._experts,
              "shared": side.shared}
    ref, ids, _ = orc.moe_ffn(inputs, w.E, w.I, w.Is, 0, w.E, w.topk, norm=gamma, residual=True)
    assert torch.equal(ids, ex["topk_ids"].cpu())
    compare(y, ref, "norm+residual decode")


@pytest.mark.parametrize("combine", ["pick", "tree"])
def test_residual_is_added_last(combine):
    w = MID
    d = gpu_inputs(w)
    gamma = _gamma(w.H, 5)
    y0, _ = _run(w, d, gamma, residual=False, combine=combine)
    y1, _ = _run(w, d, gamma, residual=True, combine=combine)
    assert torch.equal(y1, y0 + d["x"].float())


def test_negative_eps_rejected():
    w = MID
    d = gpu_inputs(w)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_ffn(d["x"], d["router_w"], d["bias"], d["experts"], d["shared"], 0, w.E, w.topk,
                    norm=_gamma(w.H).cuda(), eps=-1.0)
    assert e.value.code == -2
