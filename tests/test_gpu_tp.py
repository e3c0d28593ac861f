"""GPU: tensor-parallel expert slices, run rank after rank on one GPU.

[P4] "GLM-5.3-Flash on CUDA over three ranks (--tp 3) ... #310": each rank
holds a whole-unit slice of every expert's intermediate columns (remainder on
the lowest ranks) and returns a full-width fp32 partial; the partials are
added in rank order.  On one GPU the ranks' slices are laid out by the library
(moe_tp_slice_*), each runs through moe_ffn at its real shape, and
moe_ffn_reduce adds the partials in rank order.
"""

import pytest
import torch

import mixture_experts_ffn_06_amd as moe
import synth
from gpu_common import OracleSide, compare, gpu_inputs, log, sample_rows
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
TPW = synth.Workload("tpw", T=120, H=512, E=16, topk=4, I=384, Is=384)


def _cpu_copy(experts):
    return {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in experts.items()}


@pytest.mark.parametrize("fmt", ["bf16", "w4"])
def test_slices_hold_the_named_columns(fmt):
    w = TPW.with_(fmt=fmt)
    d = gpu_inputs(w)
    cpu = _cpu_copy(d["experts"])
    for i_lo, i_hi in ((0, 64), (64, 320), (128, 192)):
        s = moe.tp_slice_experts(d["experts"], i_lo, i_hi)
        torch.cuda.synchronize()
        want = orc.tp_slice(cpu, i_lo, i_hi)
        for name, t in want.items():
            if isinstance(t, torch.Tensor):
                assert torch.equal(s[name].cpu(), t), (fmt, name, i_lo, i_hi)
    sh = moe.tp_slice_shared(d["shared"], 64, 192)
    torch.cuda.synchronize()
    want = orc.tp_slice({"fmt": "bf16", **{k: v.cpu() for k, v in d["shared"].items()}}, 64, 192)
    assert torch.equal(sh["w_gate_up"].cpu(), want["w_gate_up"])
    assert torch.equal(sh["w_down"].cpu(), want["w_down"])


def _rank_calls(w, d, unit, ranks):
    shares = moe.tp_shares(w.I, unit, ranks)
    sshares = moe.tp_shares(w.Is, unit, ranks)
    parts, ids = [], None
    lo = slo = 0
    for r in range(ranks):
        ex = moe.tp_slice_experts(d["experts"], lo, lo + shares[r])
        sh = moe.tp_slice_shared(d["shared"], slo, slo + sshares[r])
        exp = {}
        y = moe.moe_ffn(d["x"], d["router_w"], d["bias"], ex, sh, 0, w.E, w.topk, exports=exp)
        torch.cuda.synchronize()
        if ids is None:
            ids = exp["topk_ids"].cpu()
        assert torch.equal(exp["topk_ids"].cpu(), ids), "ranks disagree on the picks"
        parts.append(y)
        lo += shares[r]
        slo += sshares[r]
        del ex, sh
    y = moe.reduce(parts, "rank")
    torch.cuda.synchronize()
    return y, parts, shares


@pytest.mark.parametrize("fmt", ["bf16", "w4"])
@pytest.mark.parametrize("unit,ranks", [(64, 3), (128, 2), (64, 5)])
def test_tp_layer_adds_up_to_the_whole_layer(fmt, unit, ranks):
    w = TPW.with_(fmt=fmt)
    d = gpu_inputs(w)
    d["bias"] = (-0.4 * torch.arange(w.E, dtype=torch.float32)).cuda()
    y, parts, shares = _rank_calls(w, d, unit, ranks)
    log(f"{fmt} unit {unit} ranks {ranks}: shares {shares}")
    full = moe.moe_ffn(d["x"], d["router_w"], d["bias"], d["experts"], d["shared"], 0, w.E, w.topk)
    torch.cuda.synchronize()
    scale = float(full.abs().max())
    drift = float((y - full).abs().max())
    log(f"rank-order sum vs whole layer: max|d| = {drift:.3g} (max|full| {scale:.3g})")
    assert drift <= 1e-3 * scale
    side = OracleSide(w, d)
    compare(y, side.layer(list(range(w.T)), 0, w.E), f"tp {fmt} {unit}x{ranks}")
    # the rank-order sum, bit for bit the oracle's merge of the same partials
    assert torch.equal(y.cpu(), orc.rank_merge([p.cpu() for p in parts]))


def test_tp_decode_full_size_three_ranks():
    w = W["decode"]
    d = gpu_inputs(w)
    side = OracleSide(w, d)
    ref = side.layer(list(range(w.T)), 0, w.E)
    full = moe.moe_ffn(d["x"], d["router_w"], d["bias"], d["experts"], d["shared"], 0, w.E, w.topk)
    for unit in (64, 128):
        y, parts, shares = _rank_calls(w, d, unit, 3)
        log(f"decode tp3 unit {unit}: shares {shares}")
        assert shares == ([704, 704, 640] if unit == 64 else [768, 640, 640])
        compare(y, ref, f"decode tp3 unit {unit}")
        assert float((y - full).abs().max()) <= 1e-3 * float(full.abs().max())


def test_tp_rank_partial_against_the_oracle_slice():
    # one rank's partial alone is the layer of its sliced experts
    w = TPW
    d = gpu_inputs(w)
    ex = moe.tp_slice_experts(d["experts"], 128, 256)
    sh = moe.tp_slice_shared(d["shared"], 64, 128)
    y = moe.moe_ffn(d["x"], d["router_w"], d["bias"], ex, sh, 0, w.E, w.topk)
    torch.cuda.synchronize()
    ws = w.with_(I=128, Is=64)
    inputs = {"x": d["x"].cpu(), "router_w": d["router_w"].cpu(),
              "bias": None if d["bias"] is None else d["bias"].cpu(),
              "experts": orc.tp_slice(_cpu_copy(d["experts"]), 128, 256),
              "shared": {k: v for k, v in orc.tp_slice({"fmt": "bf16", **{k: v.cpu() for k, v in d["shared"].items()}}, 64, 128).items() if k != "fmt"}}
    rows = sample_rows(w.T, 12, seed=2)
    ref, _, _ = orc.moe_ffn(inputs, ws.E, ws.I, ws.Is, 0, ws.E, ws.topk,
                            rows=torch.tensor(rows, dtype=torch.int32))
    compare(y[rows], ref, "one rank's partial")


def test_slice_rejects_bad_ranges():
    w = TPW
    d = gpu_inputs(w)
    for a, b in ((0, 32), (64, 64), (320, 448), (-64, 64)):
        with pytest.raises(moe.MoeError) as e:
            moe.tp_slice_experts(d["experts"], a, b)
        assert e.value.code == -2
