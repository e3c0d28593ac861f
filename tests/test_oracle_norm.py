"""Pins for the oracle's RMSNorm before routing and the residual add.

[P2] "GLM-5.3-Flash on CUDA: attention on one GPU, routed experts on the
Sparks (proposal) #214", "Per MoE layer": the expert side receives the normed
rows.  [P5] "GLM-5.3-Flash and full GLM-5.3 on the native CUDA engine
(tracker) #593", "What exists now": rmsnorm is one of the fixed-order fp32
glue kernels; its first byte-gate run found the cross-lane total reaching only
some lanes, which then ran inv_rms(0) ~ 316x (1/sqrt(eps), eps = 1e-5).
"""

import math

import numpy as np
import pytest
import torch

import synth
from oracle import oracle as orc


def _bf16_ulp(v):
    v = abs(float(v))
    if v == 0:
        return 2.0 ** -133
    return 2.0 ** (math.frexp(v)[1] - 8)


def test_inv_rms_of_a_zero_row_is_the_pages_316():
    x = torch.zeros(3, 768, dtype=torch.bfloat16)
    xn, inv = orc.rmsnorm(x, torch.ones(768))
    assert torch.equal(xn, x)
    assert abs(float(inv[0]) - 316.0) < 0.5          # the page's ~316x
    assert float(inv[0]) == np.float32(1.0) / np.sqrt(np.float32(1e-5))


def test_rmsnorm_matches_the_exact_value_to_half_a_bf16_ulp():
    g = torch.Generator().manual_seed(4)
    x = (torch.randn(64, 1536, generator=g) * torch.logspace(-3, 3, 64)[:, None]).to(torch.bfloat16)
    gamma = (1.0 + 0.1 * torch.randn(1536, generator=g)).to(torch.bfloat16)
    xn, _ = orc.rmsnorm(x, gamma)
    xd = x.double()
    exact = xd / torch.sqrt(xd.pow(2).mean(1, keepdim=True) + 1e-5) * gamma.double()
    err = (xn.double() - exact).abs()
    ulp = torch.tensor([[_bf16_ulp(v) for v in row] for row in exact.tolist()], dtype=torch.float64)
    # bf16 rounding of a value correct to fp32 accuracy: within half an ulp
    # plus the fp32 error of the three steps before it
    assert bool((err <= 0.5 * ulp + 1e-6 * exact.abs()).all())
    same = (xn == exact.to(torch.bfloat16)).double().mean()
    assert float(same) > 0.999


def test_constant_rows_closed_form():
    H = 512
    for c in (1.0, 2.0, 0.5, -3.0):
        x = torch.full((1, H), c, dtype=torch.bfloat16)
        xn, inv = orc.rmsnorm(x, torch.ones(H))
        # H c^2 is exact, so ms = c^2 and inv = 1 / sqrt(c^2 + eps)
        want_inv = np.float32(1.0) / np.sqrt(np.float32(c * c) + np.float32(1e-5))
        assert float(inv[0]) == want_inv
        assert torch.equal(xn, torch.full((1, H), c * float(want_inv)).to(torch.bfloat16))


def test_energy_in_one_lanes_elements_only():
    # every nonzero element sits in the 4 elements one R-order lane owns in
    # one step: the total still reaches every element of the row
    H = 1024
    x = torch.zeros(2, H)
    x[0, 252:256] = torch.tensor([3.0, -4.0, 12.0, 0.0])   # norm 13, lane 63
    x[1, 512:516] = torch.tensor([1.0, 1.0, 1.0, 1.0])
    x = x.to(torch.bfloat16)
    xn, inv = orc.rmsnorm(x, torch.ones(H))
    for t, ss in ((0, 169.0), (1, 4.0)):
        want = 1.0 / math.sqrt(ss / H + 1e-5)
        assert abs(float(inv[t]) - want) <= 3e-7 * want  # a few fp32 roundings
    assert float(xn[0, 254]) == pytest.approx(12.0 * float(inv[0]), rel=2 ** -8)


def _inputs(w):
    d = synth.make_inputs(w, "cpu")
    g = torch.Generator().manual_seed(1)
    gamma = (1.0 + 0.05 * torch.randn(w.H, generator=g)).to(torch.bfloat16)
    return d, gamma


def test_layer_on_normed_rows_equals_layer_of_prenormed_input():
    w = synth.WORKLOADS["tiny"].with_(T=5)
    d, gamma = _inputs(w)
    a, ids_a, _ = orc.moe_ffn(d, w.E, w.I, w.Is, 0, w.E, w.topk, norm=gamma)
    xn, _ = orc.rmsnorm(d["x"], gamma)
    dd = dict(d)
    dd["x"] = xn
    b, ids_b, _ = orc.moe_ffn(dd, w.E, w.I, w.Is, 0, w.E, w.topk)
    assert torch.equal(a, b) and torch.equal(ids_a, ids_b)


def test_residual_adds_the_raw_rows_last():
    w = synth.WORKLOADS["tiny"].with_(T=5)
    d, gamma = _inputs(w)
    a, _, _ = orc.moe_ffn(d, w.E, w.I, w.Is, 0, w.E, w.topk, norm=gamma)
    b, _, _ = orc.moe_ffn(d, w.E, w.I, w.Is, 0, w.E, w.topk, norm=gamma, residual=True)
    assert torch.equal(b, a + d["x"].double())
    c, _, _ = orc.moe_ffn(d, w.E, w.I, w.Is, 0, w.E, w.topk, residual=True)
    e, _, _ = orc.moe_ffn(d, w.E, w.I, w.Is, 0, w.E, w.topk)
    assert torch.equal(c, e + d["x"].double())
