"""Pins for the tensor-parallel share rule and the sliced layer in the oracle.

[P4] "GLM-5.3-Flash on CUDA over three ranks (--tp 3) ... #310": a dimension
splits in whole units, as evenly as it goes, with the remainder on the lowest
ranks; each rank returns a full-width fp32 partial and the partials are added
in rank order.  The page prints worked shares (tests/golden/tp_shares.json).
"""

import json
import os

import pytest
import torch

import synth
from oracle import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tp_shares.json")


def test_shares_printed_on_the_page():
    cases = json.load(open(GOLDEN))["cases"]
    assert len(cases) == 5
    for c in cases:
        assert orc.tp_shares(c["dim"], c["unit"], c["ranks"]) == c["shares"], c["what"]


def test_share_rule_properties():
    for unit in (1, 32, 64, 128):
        for units in range(1, 40):
            dim = units * unit
            for ranks in range(1, min(units, 9) + 1):
                s = orc.tp_shares(dim, unit, ranks)
                assert sum(s) == dim
                assert all(v % unit == 0 and v > 0 for v in s)
                assert all(a >= b for a, b in zip(s, s[1:]))  # remainder on the lowest ranks
                assert max(s) - min(s) <= unit                 # as even as it goes


def test_share_rule_rejects():
    for args in ((2000, 64, 3), (64, 64, 2), (0, 64, 1), (128, 64, 0)):
        with pytest.raises(ValueError):
            orc.tp_shares(*args)


def _slices(w, unit, ranks):
    s = orc.tp_shares(w.I, unit, ranks)
    ss = orc.tp_shares(w.Is, unit, ranks)
    lo, slo, out = 0, 0, []
    for r in range(ranks):
        out.append(((lo, lo + s[r]), (slo, slo + ss[r])))
        lo += s[r]
        slo += ss[r]
    return out


def _slice_inputs(d, sl):
    (a, b), (sa, sb) = sl
    dd = dict(d)
    dd["experts"] = orc.tp_slice(d["experts"], a, b)
    sh = orc.tp_slice({"fmt": "bf16", **d["shared"]}, sa, sb)
    dd["shared"] = {"w_gate_up": sh["w_gate_up"], "w_down": sh["w_down"]}
    return dd, b - a, sb - sa


@pytest.mark.parametrize("fmt", ["bf16", "w4", "affine4", "nvfp4"])
def test_rank_order_sum_of_slices_is_the_layer(fmt):
    # W (x) = sum over column slices of W_down[:, s] h[s]: exact in real
    # arithmetic; in fp64 the slice partials add up to the full layer up to
    # reassociation of the down-projection sums.
    w = synth.Workload("tp", T=5, H=256, E=8, topk=2, I=320, Is=192, fmt=fmt)
    d = synth.make_inputs(w, "cpu")
    full, ids, _ = orc.moe_ffn(d, w.E, w.I, w.Is, 0, w.E, w.topk)
    acc = None
    for sl in _slices(w, 64, 3):
        dd, I_r, Is_r = _slice_inputs(d, sl)
        p, ids_r, _ = orc.moe_ffn(dd, w.E, I_r, Is_r, 0, w.E, w.topk)
        assert torch.equal(ids_r, ids)  # the router is replicated: same picks
        acc = p if acc is None else acc + p
    scale = float(full.abs().max())
    assert float((acc - full).abs().max()) <= 64 * 2.0 ** -52 * scale


def test_one_rank_slice_is_the_whole_layer():
    w = synth.Workload("tp1", T=4, H=256, E=8, topk=2, I=128, Is=128)
    d = synth.make_inputs(w, "cpu")
    full, _, _ = orc.moe_ffn(d, w.E, w.I, w.Is, 0, w.E, w.topk)
    dd, I_r, Is_r = _slice_inputs(d, ((0, w.I), (0, w.Is)))
    p, _, _ = orc.moe_ffn(dd, w.E, I_r, Is_r, 0, w.E, w.topk)
    assert torch.equal(p, full)


def test_slice_keeps_the_columns_it_names():
    # bf16: gate rows i_lo..i_hi-1, up rows I+i_lo.., down inputs i_lo..
    E, I, H = 2, 128, 256
    gu = torch.arange(E * 2 * I * H, dtype=torch.float32).reshape(E, 2 * I, H)
    dn = torch.arange(E * H * I, dtype=torch.float32).reshape(E, H, I)
    s = orc.tp_slice({"fmt": "bf16", "w_gate_up": gu, "w_down": dn}, 64, 128)
    assert torch.equal(s["w_gate_up"][:, :64], gu[:, 64:128])
    assert torch.equal(s["w_gate_up"][:, 64:], gu[:, I + 64:I + 128])
    assert torch.equal(s["w_down"], dn[:, :, 64:128])
