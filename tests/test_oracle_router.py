"""Pins for the oracle's sigmoid router.

[P5] "GLM-5.3-Flash and full GLM-5.3 on the native CUDA engine (tracker)
#593", "What exists now": GLM's router is sigmoid + bias top-k with raw-score
weights.  The selection turns on fp32 scores, so the sigmoid is a fixed fp32
computation (exp_c: range reduction by ln 2, the Taylor terms 1/i! up to i =
6 in Horner form with fused multiply-adds, exact scaling by 2^n; then
1 / (1 + exp_c(-l))).  Its pins: the mathematical exp and sigmoid (libm in
double) within a small ulp bound over a dense sweep, exact special values,
monotonicity, and brute-force selection.
"""

import math

import numpy as np
import pytest
import torch

import synth
from oracle import oracle as orc


def _f32_ulp(v):
    v = abs(float(np.float32(v)))
    if v == 0:
        return 2.0 ** -149
    e = math.frexp(v)[1]
    return 2.0 ** (e - 24)


def test_exp_c_within_three_ulp_of_exp():
    # the fixed fp32 evaluation reaches about 2.5 ulp at worst; a wrong term,
    # reduction constant or sign costs thousands
    xs = np.linspace(-87.0, 88.0, 20001).astype(np.float32)
    worst = 0.0
    for x in xs:
        got = orc.exp_c(float(x))
        want = math.exp(float(x))
        err = abs(got - want) / _f32_ulp(want)
        worst = max(worst, err)
    assert worst <= 3.0, worst


def test_exp_c_small_arguments_and_exact_points():
    assert orc.exp_c(0.0) == 1.0
    assert orc.exp_c(-0.0) == 1.0
    for x in (1e-8, -1e-8, 1e-4, -1e-4, 0.25, -0.25, 0.34657, -0.34657):
        got, want = orc.exp_c(x), math.exp(np.float32(x))
        assert abs(got - want) <= 3 * _f32_ulp(want)
    assert orc.exp_c(100.0) == math.inf
    assert orc.exp_c(-200.0) == 0.0


def test_sigmoid_c_values():
    assert orc.sigmoid_c(0.0) == 0.5
    assert orc.sigmoid_c(200.0) == 1.0
    assert orc.sigmoid_c(-200.0) == 0.0
    xs = np.linspace(-30.0, 30.0, 6001).astype(np.float32)
    prev = -1.0
    for x in xs:
        s = orc.sigmoid_c(float(x))
        want = 1.0 / (1.0 + math.exp(-float(x)))
        assert abs(s - want) <= 3 * _f32_ulp(want), x
        assert s >= prev  # monotone
        prev = s


def _key(l, b):
    s = np.float32(orc.sigmoid_c(float(l)))
    v = np.float32(s + np.float32(b))
    return 0.0 if v == 0 else float(v), float(s)


def test_topk_sigmoid_brute_force():
    rng = np.random.default_rng(5)
    for trial in range(30):
        E = int(rng.integers(2, 40))
        k = int(rng.integers(1, min(E, 16) + 1))
        T = 3
        lg = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32) * 3)
        if trial % 3 == 0:  # ties: repeated logits
            lg[:, ::2] = lg[:, :1]
        bias = None if trial % 2 else torch.from_numpy(rng.standard_normal(E).astype(np.float32) * 0.1)
        ids, w = orc.topk_sigmoid(lg, bias, k)
        for t in range(T):
            keys = []
            for e in range(E):
                kv, s = _key(lg[t, e], 0.0 if bias is None else bias[e])
                keys.append((-kv, e, s))
            keys.sort()
            assert ids[t].tolist() == [e for _, e, _ in keys[:k]]
            assert w[t].tolist() == [s for _, _, s in keys[:k]]


def test_bias_steers_selection_only():
    lg = torch.tensor([[0.5, -1.0, 2.0, 0.0, -3.0, 1.0]], dtype=torch.float32)
    bias = torch.tensor([0.0, 0.0, 0.0, 0.0, 10.0, 0.0], dtype=torch.float32)
    ids, w = orc.topk_sigmoid(lg, bias, 2)
    assert ids.tolist() == [[4, 2]]
    assert w[0, 0] == orc.sigmoid_c(-3.0)  # the raw score, not the biased key
    assert w[0, 1] == orc.sigmoid_c(2.0)
    ids0, w0 = orc.topk_sigmoid(lg, torch.zeros(6), 3)
    ids1, w1 = orc.topk_sigmoid(lg, None, 3)
    assert torch.equal(ids0, ids1) and torch.equal(w0, w1)


def test_sigmoid_layer_is_the_sum_of_its_picks():
    w = synth.WORKLOADS["tiny"].with_(T=4, topk=3)
    d = synth.make_inputs(w, "cpu")
    d["bias"] = torch.linspace(-0.2, 0.2, w.E)
    out, ids, wt = orc.moe_ffn(d, w.E, w.I, w.Is, 0, w.E, w.topk, router="sigmoid")
    lg = orc.router_logits(d["x"], d["router_w"], None)
    ids2, wt2 = orc.topk_sigmoid(lg, d["bias"], w.topk)
    assert torch.equal(ids, ids2) and torch.equal(wt, wt2)
    ex = orc.Experts(d["experts"], w.E, w.H, w.I)
    sh = orc.Experts({"fmt": "bf16", "w_gate_up": d["shared"]["w_gate_up"][None],
                      "w_down": d["shared"]["w_down"][None]}, 1, w.H, w.Is)
    for t in range(w.T):
        xr = d["x"][t].double()
        ref = torch.zeros(w.H, dtype=torch.float64)
        for j in range(w.topk):
            ref += wt[t, j] * orc.expert_ffn(xr, ex, int(ids[t, j]))
        ref += orc.expert_ffn(xr, sh, 0)
        assert torch.equal(out[t], ref)
