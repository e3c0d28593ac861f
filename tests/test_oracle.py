"""Pins for the CPU oracle: each test checks the oracle against something other
than itself -- hand-worked values of the fixed router order, exact sums,
library routines in the special cases that reduce to them, closed forms on
constructed weights, invariants and brute force on tiny inputs.

Pages: [P1] "GLM-5.2 multi-GPU: expert-parallel sharding + the resident-fit
benchmark" (gates table); [P2] "GLM-5.3-Flash on CUDA: attention on one GPU,
routed experts on the Sparks (proposal) #214" (Per MoE layer); [P5]
"GLM-5.3-Flash and full GLM-5.3 on the native CUDA engine (tracker) #593".
"""

import math

import numpy as np
import pytest
import torch

import synth
from oracle import oracle as orc


def bf16(a):
    return torch.as_tensor(a, dtype=torch.float32).to(torch.bfloat16)


# --------------------------------------------------------------------------
# Router: the fixed-order fp32 dot (R-order).
# --------------------------------------------------------------------------

def test_dot_r_inner_chunk_before_outer_step():
    # Lane 0 owns k = 0..3 (step i=0) then k = 256..259 (step i=1).  Its fma
    # chain is 1e8, +1 (rounds back to 1e8: ulp(1e8) = 8), ..., -1e8  -> 0.
    x = torch.zeros(512)
    x[0], x[1], x[256] = 1e8, 1.0, -1e8
    assert orc.dot_r(x, torch.ones(512)) == 0.0
    # Put the 1 in lane 1 instead (k = 4): lane 0 cancels exactly, lane 1
    # holds 1, and the pairwise rounds give exactly 1.
    x = torch.zeros(512)
    x[0], x[4], x[256] = 1e8, 1.0, -1e8
    assert orc.dot_r(x, torch.ones(512)) == 1.0


def test_dot_r_pairwise_rounds():
    # Lane 0 holds 1e8 and lanes 1..63 hold 1 each (x[4l] = 1).  Pairwise
    # rounds: s=1,2 lose the 1 and 2 added to 1e8, s=4 adds 4 (a tie, 1e8 has
    # an even significand, stays 1e8), then s=8,16,32 add 8, 16, 32 exactly:
    # 1e8 + 56.  A left-to-right sum over lanes would stay at 1e8; the exact
    # sum is 1e8 + 63.
    x = torch.zeros(256)
    x[0] = 1e8
    x[4:256:4] = 1.0
    assert orc.dot_r(x, torch.ones(256)) == 100000056.0
    # Lanes 0 and 1 cancel exactly before lane 32's 1 joins in the last round.
    x = torch.zeros(256)
    x[0], x[4], x[128] = 1e8, -1e8, 1.0
    assert orc.dot_r(x, torch.ones(256)) == 1.0


def test_dot_r_error_bound_random():
    # |dot_R - exact| <= (H/64 + 6) * 2^-24 * sum|x_k w_k| (fp32 fma chains of
    # H/64 terms then six pairwise adds), exact sum by math.fsum of exact
    # fp64 products.
    g = torch.Generator().manual_seed(5)
    for H in (256, 1024, 6144):
        for _ in range(5):
            x = torch.randn(H, generator=g).to(torch.bfloat16).float()
            w = (torch.randn(H, generator=g) * 0.02).float()
            prods = (x.double() * w.double()).tolist()
            exact = math.fsum(prods)
            bound = (H / 64 + 6) * 2.0 ** -24 * math.fsum(abs(p) for p in prods)
            assert abs(orc.dot_r(x, w) - exact) <= bound


def test_dot_r_single_term_and_every_position():
    # One nonzero product: the dot is that product exactly, wherever it sits
    # (catches a dropped or misindexed term).
    H = 512
    for k in range(H):
        x = torch.zeros(H)
        x[k] = 3.0
        w = torch.zeros(H)
        w[k] = 0.25
        assert orc.dot_r(x, w) == 0.75


def test_router_logits_bias_and_negative_zero():
    H, E = 256, 4
    x = bf16(torch.full((1, H), -1e-30))
    wr = torch.full((E, H), 1e-30)
    # Every product underflows to -0.0, so every partial sum is -0.0; the logit
    # must come back as +0.0.
    lg = orc.router_logits(x, wr, None)
    assert (lg.view(torch.int32) == 0).all()
    bias = torch.tensor([1.5, -2.0, 0.0, 0.25])
    lg = orc.router_logits(x, wr, bias)
    assert lg[0].tolist() == [1.5, -2.0, 0.0, 0.25]


# --------------------------------------------------------------------------
# Top-k and weights.
# --------------------------------------------------------------------------

def test_topk_matches_sorted_with_ties():
    g = torch.Generator().manual_seed(1)
    for E, k in ((8, 2), (16, 5), (256, 8), (64, 64)):
        # Quantised logits force many ties; -0.0 and +0.0 must tie too.
        lg = (torch.randint(-3, 4, (32, E), generator=g).float() * 0.5)
        lg[0, :4] = torch.tensor([-0.0, 0.0, -0.0, 0.0])[: min(4, E)]
        ids, _ = orc.topk(lg, k)
        for t in range(lg.shape[0]):
            ref = [e for _, e in sorted((-float(v), e) for e, v in enumerate(lg[t].tolist()))][:k]
            assert ids[t].tolist() == ref


def test_topk_uniform_logits_exact():
    # Zero router: all logits +0 -> picks 0..k-1 and weights exactly 1/k.
    x = bf16(torch.randn(3, 256))
    lg = orc.router_logits(x, torch.zeros(8, 256), None)
    ids, w = orc.topk(lg, 4)
    assert ids.tolist() == [[0, 1, 2, 3]] * 3
    assert (w == 0.25).all()


def test_topk1_weight_is_one():
    lg = torch.randn(10, 16)
    ids, w = orc.topk(lg, 1)
    assert (w == 1.0).all()
    assert ids[:, 0].tolist() == lg.argmax(dim=1).tolist()


def test_topk_all_experts_is_softmax():
    # k = E: the renormalised weights are the full softmax (library routine).
    from scipy.special import softmax

    lg = torch.randn(6, 32, generator=torch.Generator().manual_seed(3))
    ids, w = orc.topk(lg, 32)
    for t in range(6):
        sm = softmax(lg[t].double().numpy())
        np.testing.assert_allclose(w[t].numpy(), sm[ids[t].numpy()], rtol=1e-13, atol=0)


def test_topk_weights_known_ratio():
    # Logits 0 and -ln 2 -> weights 2/3 and 1/3.
    lg = torch.tensor([[0.0, -math.log(2.0), -50.0, -60.0]])
    ids, w = orc.topk(lg, 2)
    assert ids.tolist() == [[0, 1]]
    l1 = float(torch.tensor(-math.log(2.0), dtype=torch.float32))
    e = math.exp(l1)
    assert w[0].tolist() == pytest.approx([1 / (1 + e), e / (1 + e)], rel=1e-15)
    assert abs(w[0, 0].item() - 2 / 3) < 1e-7


# --------------------------------------------------------------------------
# Dispatch.
# --------------------------------------------------------------------------

def _dispatch_brute(ids, lo, hi):
    T, k = ids.shape
    picks = [(int(ids[t, j]), t, j) for t in range(T) for j in range(k) if lo <= ids[t, j] < hi]
    picks.sort()
    perm = [t * k + j for _, t, j in picks]
    counts = [sum(1 for e, _, _ in picks if e == x) for x in range(lo, hi)]
    pos = [-1] * (T * k)
    for i, p in enumerate(perm):
        pos[p] = i
    return counts, perm, pos


def _random_ids(T, E, k, g):
    return torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).to(torch.int32)


def test_dispatch_brute_force_every_band():
    g = torch.Generator().manual_seed(7)
    ids = _random_ids(13, 8, 3, g)
    for lo in range(8):
        for hi in range(lo + 1, 9):
            counts, offsets, perm, pos = orc.dispatch(ids, lo, hi)
            bc, bp, bpos = _dispatch_brute(ids, lo, hi)
            assert counts.tolist() == bc
            assert offsets.tolist() == list(np.concatenate([[0], np.cumsum(bc)]))
            assert perm.tolist() == bp
            assert pos.tolist() == bpos


def test_dispatch_invariants_large():
    g = torch.Generator().manual_seed(8)
    T, E, k = 700, 256, 8
    ids = _random_ids(T, E, k, g)
    counts, offsets, perm, pos = orc.dispatch(ids, 32, 96)
    assert int(counts.sum()) == perm.numel()
    assert offsets[0] == 0 and (offsets[1:] - offsets[:-1] == counts).all()
    # perm is a bijection onto in-band picks, rows ascend within each expert,
    # and pos inverts perm.
    inb = ((ids >= 32) & (ids < 96)).flatten()
    assert sorted(perm.tolist()) == torch.nonzero(inb).flatten().tolist()
    for e in range(64):
        seg = perm[offsets[e]: offsets[e + 1]]
        assert (ids.flatten()[seg.long()] == 32 + e).all()
        rows = (seg // k).tolist()
        assert rows == sorted(rows)
    assert (pos[perm.long()] == torch.arange(perm.numel(), dtype=torch.int32)).all()
    assert (pos[~inb] == -1).all()


def test_dispatch_all_picks_one_expert():
    ids = torch.full((50, 1), 3, dtype=torch.int32)
    counts, offsets, perm, pos = orc.dispatch(ids, 0, 8)
    assert counts.tolist() == [0, 0, 0, 50, 0, 0, 0, 0]
    assert perm.tolist() == list(range(50))


# --------------------------------------------------------------------------
# SwiGLU expert FFN on constructed weights (closed forms).
# --------------------------------------------------------------------------

def _perm_expert(H, I, pg, pu, sigma, a):
    """Expert whose gate row i selects a * x[pg[i]], up row i selects x[pu[i]],
    and down row c selects h[sigma[c]]: y[c] = silu(a x[pg[s]]) x[pu[s]], s = sigma[c]."""
    wgu = torch.zeros(2 * I, H)
    wd = torch.zeros(H, I)
    for i in range(I):
        wgu[i, pg[i]] = a
        wgu[I + i, pu[i]] = 1.0
    for c in range(H):
        wd[c, sigma[c]] = 1.0
    return wgu.to(torch.bfloat16), wd.to(torch.bfloat16)


def _silu(v):
    return v / (1.0 + math.exp(-v))


def test_expert_ffn_permutation_closed_form():
    H, I = 256, 128
    g = torch.Generator().manual_seed(11)
    pg, pu = torch.randperm(H, generator=g)[:I], torch.randperm(H, generator=g)[:I]
    sigma = torch.randint(0, I, (H,), generator=g)
    wgu, wd = _perm_expert(H, I, pg, pu, sigma, 0.5)
    ex = orc.Experts({"fmt": "bf16", "w_gate_up": wgu[None], "w_down": wd[None]}, 1, H, I)
    x = bf16(torch.randn(H, generator=g)).double()
    y = orc.expert_ffn(x, ex, 0)
    for c in range(H):
        s = int(sigma[c])
        ref = _silu(0.5 * float(x[pg[s]])) * float(x[pu[s]])
        assert y[c].item() == pytest.approx(ref, rel=1e-14, abs=1e-300)


def test_expert_ffn_linear_in_down_weights():
    H, I = 256, 64
    g = torch.Generator().manual_seed(12)
    wgu = bf16(torch.randn(1, 2 * I, H, generator=g) * 0.05)
    wd = bf16(torch.randn(1, H, I, generator=g) * 0.05)
    x = bf16(torch.randn(H, generator=g)).double()
    y1 = orc.expert_ffn(x, orc.Experts({"fmt": "bf16", "w_gate_up": wgu, "w_down": wd}, 1, H, I), 0)
    y2 = orc.expert_ffn(x, orc.Experts({"fmt": "bf16", "w_gate_up": wgu, "w_down": (wd.float() * 2).to(torch.bfloat16)}, 1, H, I), 0)
    assert torch.equal(y2, 2 * y1)


# --------------------------------------------------------------------------
# 4-bit group-affine decode: weight = (q - z) * s, low nibble = even k.
# --------------------------------------------------------------------------

def _pack(q):
    q = q.to(torch.int32)
    return (q[..., 0::2] | (q[..., 1::2] << 4)).to(torch.uint8)


def _w4(q, s, z):
    return {"fmt": "w4", "q_gate_up": _pack(q), "s_gate_up": s, "z_gate_up": z,
            "q_down": None, "s_down": None, "z_down": None}


def test_w4_unit_scale_zero_offset_is_codes():
    # s = 1, z = 0: the matrix is the codes themselves, in k order.
    N, K = 2 * 32, 64  # gate/up matrix [2I, H] with I=32, H=64
    g = torch.Generator().manual_seed(13)
    q = torch.randint(0, 16, (1, N, K), generator=g)
    s = bf16(torch.ones(1, N, K // 32))
    z = bf16(torch.zeros(1, N, K // 32))
    ex = orc.Experts(_w4(q, s, z), 1, K, N // 2)
    m = orc.expert_matrix(ex, 0, 0)
    assert torch.equal(m, q[0].double())


def test_w4_codes_equal_zero_points_vanish():
    # Integer z per group and codes equal to their group's z: every weight is 0.
    N, K = 64, 128
    zint = torch.randint(0, 16, (1, N, K // 32), generator=torch.Generator().manual_seed(14))
    q = zint.repeat_interleave(32, dim=2)
    ex = orc.Experts(_w4(q, bf16(torch.full((1, N, K // 32), 0.01)), bf16(zint.float())), 1, K, N // 2)
    assert (orc.expert_matrix(ex, 0, 0) == 0).all()


def test_w4_codes_one_above_zero_give_group_scale():
    N, K = 64, 128
    g = torch.Generator().manual_seed(15)
    zint = torch.randint(0, 15, (1, N, K // 32), generator=g)
    s = bf16(torch.rand(1, N, K // 32, generator=g) * 0.015 + 0.005)
    q = (zint + 1).repeat_interleave(32, dim=2)
    ex = orc.Experts(_w4(q, s, bf16(zint.float())), 1, K, N // 2)
    m = orc.expert_matrix(ex, 0, 0)
    assert torch.equal(m, s[0].double().repeat_interleave(32, dim=1))


# The down projection [H, I] decodes the same way along I.  Its codes, scales
# and zeros are drawn apart from the gate/up ones (other seeds, other
# values), so a down matrix read through the gate/up arrays, or with the
# scale and zero swapped, fails these.

def _w4_both(H, I, gu, dn):
    """4-bit experts (E = 1) with gate/up (q, s, z) = gu over [2I, H] and down
    (q, s, z) = dn over [H, I]."""
    return {"fmt": "w4", "q_gate_up": _pack(gu[0]), "s_gate_up": gu[1], "z_gate_up": gu[2],
            "q_down": _pack(dn[0]), "s_down": dn[1], "z_down": dn[2]}


def _w4_noise(N, K, g):
    q = torch.randint(0, 16, (1, N, K), generator=g)
    s = bf16(torch.rand(1, N, K // 32, generator=g) * 0.015 + 0.005)
    z = bf16(torch.rand(1, N, K // 32, generator=g) * 2 + 7)
    return q, s, z


def test_w4_down_unit_scale_zero_offset_is_codes():
    # s = 1, z = 0 on the down matrix: it is its codes, in input (I) order.
    H, I = 64, 96
    g = torch.Generator().manual_seed(21)
    q = torch.randint(0, 16, (1, H, I), generator=g)
    dn = (q, bf16(torch.ones(1, H, I // 32)), bf16(torch.zeros(1, H, I // 32)))
    ex = orc.Experts(_w4_both(H, I, _w4_noise(2 * I, H, g), dn), 1, H, I)
    assert torch.equal(orc.expert_matrix(ex, 0, 1), q[0].double())


def test_w4_down_codes_equal_zero_points_vanish():
    H, I = 64, 128
    g = torch.Generator().manual_seed(22)
    zint = torch.randint(0, 16, (1, H, I // 32), generator=g)
    dn = (zint.repeat_interleave(32, dim=2), bf16(torch.full((1, H, I // 32), 0.01)), bf16(zint.float()))
    ex = orc.Experts(_w4_both(H, I, _w4_noise(2 * I, H, g), dn), 1, H, I)
    assert (orc.expert_matrix(ex, 0, 1) == 0).all()
    # ... while the gate/up matrix of the same experts is not zero
    assert (orc.expert_matrix(ex, 0, 0) != 0).any()


def test_w4_down_codes_one_above_zero_give_group_scale():
    H, I = 64, 128
    g = torch.Generator().manual_seed(23)
    zint = torch.randint(0, 15, (1, H, I // 32), generator=g)
    s = bf16(torch.rand(1, H, I // 32, generator=g) * 0.015 + 0.005)
    dn = ((zint + 1).repeat_interleave(32, dim=2), s, bf16(zint.float()))
    ex = orc.Experts(_w4_both(H, I, _w4_noise(2 * I, H, g), dn), 1, H, I)
    assert torch.equal(orc.expert_matrix(ex, 0, 1), s[0].double().repeat_interleave(32, dim=1))


def test_w4_scale_and_zero_not_interchangeable():
    # One group of each matrix with scale 2 and zero 3: code 7 decodes to
    # (7 - 3) * 2 = 8, where a swapped pair would give (7 - 2) * 3 = 15.
    H, I = 256, 64
    q_gu = torch.full((1, 2 * I, H), 7)
    q_dn = torch.full((1, H, I), 7)
    gu = (q_gu, bf16(torch.full((1, 2 * I, H // 32), 2.0)), bf16(torch.full((1, 2 * I, H // 32), 3.0)))
    dn = (q_dn, bf16(torch.full((1, H, I // 32), 2.0)), bf16(torch.full((1, H, I // 32), 3.0)))
    ex = orc.Experts(_w4_both(H, I, gu, dn), 1, H, I)
    assert (orc.expert_matrix(ex, 0, 0) == 8.0).all()
    assert (orc.expert_matrix(ex, 0, 1) == 8.0).all()


def _w4_onehot(N, K, pick, zint, s):
    """4-bit [1, N, K] matrix whose row n is s[n] at input pick[n] and 0
    elsewhere: codes equal the (integer) zero everywhere except zero + 1 at
    pick[n]; scale s[n] and zero zint[n] on every group of row n."""
    q = zint[:, None].repeat(1, K).clone()
    q[torch.arange(N), pick] += 1
    return (q[None], bf16(s[:, None].repeat(1, K // 32)[None]),
            bf16(zint[:, None].repeat(1, K // 32).float()[None]))


def test_w4_expert_ffn_closed_form_through_both_matrices():
    # Gate row i = a_i e_{pg[i]}, up row i = b_i e_{pu[i]}, down row c =
    # d_c e_{sigma[c]}, all as 4-bit codes one above an integer zero:
    # y[c] = d_c silu(a_s x[pg[s]]) b_s x[pu[s]], s = sigma[c].  This runs the
    # down decode through the expert FFN itself (a down matrix read as the
    # gate/up one, transposed, or with its scale from the wrong group fails).
    H, I = 256, 64
    g = torch.Generator().manual_seed(24)
    pg, pu = torch.randint(0, H, (I,), generator=g), torch.randint(0, H, (I,), generator=g)
    sigma = torch.randint(0, I, (H,), generator=g)
    sc = bf16(torch.rand(2 * I + H, generator=g) * 0.75 + 0.25).float()
    zi = torch.randint(0, 15, (2 * I + H,), generator=g)
    gu = _w4_onehot(2 * I, H, torch.cat([pg, pu]), zi[:2 * I], sc[:2 * I])
    dn = _w4_onehot(H, I, sigma, zi[2 * I:], sc[2 * I:])
    ex = orc.Experts(_w4_both(H, I, gu, dn), 1, H, I)
    x = bf16(torch.randn(H, generator=g)).double()
    y = orc.expert_ffn(x, ex, 0)
    for c in range(H):
        s_ = int(sigma[c])
        gate = float(sc[s_]) * float(x[pg[s_]])
        up = float(sc[I + s_]) * float(x[pu[s_]])
        ref = float(sc[2 * I + c]) * _silu(gate) * up
        assert y[c].item() == pytest.approx(ref, rel=1e-14, abs=1e-300)


# --------------------------------------------------------------------------
# The whole layer on constructed weights (closed form), and the band gates.
# --------------------------------------------------------------------------

def test_layer_closed_form_two_picks_and_shared():
    # E = 4 permutation experts with distinct gate scales; zero router plus a
    # bias that fixes the picks (experts 2 then 0) and their weights (2/3, 1/3).
    H, I, E, k = 256, 128, 4, 2
    g = torch.Generator().manual_seed(16)
    wgus, wds, par = [], [], []
    for e in range(E + 1):  # the last one is the shared expert
        pg, pu = torch.randperm(H, generator=g)[:I], torch.randperm(H, generator=g)[:I]
        sigma = torch.randint(0, I, (H,), generator=g)
        a = [0.5, 1.0, 2.0, 0.25, 1.5][e]
        wgu, wd = _perm_expert(H, I, pg, pu, sigma, a)
        wgus.append(wgu)
        wds.append(wd)
        par.append((pg, pu, sigma, a))
    bias = torch.tensor([-math.log(2.0), -5.0, 0.0, -7.0])
    x = bf16(torch.randn(3, H, generator=g))
    inputs = {"x": x, "router_w": torch.zeros(E, H), "bias": bias,
              "experts": {"fmt": "bf16", "w_gate_up": torch.stack(wgus[:E]), "w_down": torch.stack(wds[:E])},
              "shared": {"w_gate_up": wgus[E], "w_down": wds[E]}}
    l1 = float(torch.tensor(-math.log(2.0), dtype=torch.float32))
    w2, w0 = 1 / (1 + math.exp(l1)), math.exp(l1) / (1 + math.exp(l1))

    def y(e, xr, c):
        pg, pu, sigma, a = par[e]
        s = int(sigma[c])
        return _silu(a * xr[int(pg[s])]) * xr[int(pu[s])]

    for lo, hi, use in ((0, 4, (2, 0)), (0, 1, (0,)), (1, 4, (2,)), (1, 2, ())):
        out, ids, w = orc.moe_ffn(inputs, E, I, I, lo, hi, k)
        assert ids.tolist() == [[2, 0]] * 3
        for t in range(3):
            xr = x[t].double().tolist()
            for c in range(0, H, 7):
                ref = 0.0
                for e in use:
                    ref += (w2 if e == 2 else w0) * y(e, xr, c)
                ref += y(E, xr, c)
                assert out[t, c].item() == pytest.approx(ref, rel=1e-12, abs=1e-12)


def _tiny(**kw):
    w = synth.WORKLOADS["tiny"].with_(**kw)
    return w, synth.make_inputs(w, "cpu")


def test_full_band_equals_monolith_bit_exact():
    # [P1] gates table: EP with one rank == routed monolith, max|delta| = 0.
    for seed in range(3):
        w, d = _tiny(seed=seed)
        full, _, _ = orc.moe_ffn(d, w.E, w.I, w.Is, 0, w.E, w.topk)
        mono = orc.moe_ffn_monolith(d, w.E, w.I, w.Is, w.topk)
        assert torch.equal(full, mono)


def _band_sum(d, w, cuts):
    acc = None
    for b, (lo, hi) in enumerate(zip(cuts[:-1], cuts[1:])):
        dd = dict(d)
        if b > 0:
            dd["shared"] = None  # the shared expert goes with the first band only
        p, _, _ = orc.moe_ffn(dd, w.E, w.I, w.Is, lo, hi, w.topk)
        acc = p.clone() if acc is None else acc + p
    return acc


def test_every_band_partition_sums_to_full():
    # [P1] gates table: EP(ranks=N) vs monolith differs by reassociation only.
    # Every contiguous partition of E = 8 experts (2^7 of them); elementwise
    # |delta| <= (k + 1) * 2^-52 * (sum_j |w_j y_j| + |shared|), bounded here
    # by (k + 1) * 2^-52 * 4 * max|out| with a generous margin.
    w, d = _tiny(T=6, topk=3)
    full = orc.moe_ffn_monolith(d, w.E, w.I, w.Is, w.topk)
    scale = float(full.abs().max())
    for mask in range(1 << 7):
        cuts = [0] + [i + 1 for i in range(7) if mask >> i & 1] + [8]
        s = _band_sum(d, w, cuts)
        assert float((s - full).abs().max()) <= 64 * 2.0 ** -52 * scale


def test_all_picks_in_one_band_exact():
    # [P1] gates table: load-imbalanced, all picks on one rank: max|delta| = 0.
    w, d = _tiny(T=5, topk=2)
    d["bias"] = torch.tensor([10.0, 10.0, 10.0, 0, 0, 0, 0, 0])
    full = orc.moe_ffn_monolith(d, w.E, w.I, w.Is, w.topk)
    s = _band_sum(d, w, [0, 3, 5, 8])
    assert torch.equal(s, full)


def test_topk1_layer_is_argmax_expert_plus_shared():
    w, d = _tiny(topk=1)
    out, ids, wt = orc.moe_ffn(d, w.E, w.I, w.Is, 0, w.E, 1)
    assert (wt == 1.0).all()
    ex = orc.Experts(d["experts"], w.E, w.H, w.I)
    sh = orc.Experts({"fmt": "bf16", "w_gate_up": d["shared"]["w_gate_up"][None],
                      "w_down": d["shared"]["w_down"][None]}, 1, w.H, w.Is)
    for t in range(w.T):
        xr = d["x"][t].double()
        ref = orc.expert_ffn(xr, ex, int(ids[t, 0])) + orc.expert_ffn(xr, sh, 0)
        assert torch.equal(out[t], ref)


def test_layer_rows_subset_matches_all_rows():
    w, d = _tiny(T=7)
    full, ids, wt = orc.moe_ffn(d, w.E, w.I, w.Is, 0, w.E, w.topk)
    rows = torch.tensor([6, 0, 3], dtype=torch.int32)
    sub, sids, swt = orc.moe_ffn(d, w.E, w.I, w.Is, 0, w.E, w.topk, rows=rows)
    assert torch.equal(sub, full[rows.long()])
    assert torch.equal(sids, ids[rows.long()])


def test_fail_closed():
    # [P1] gates table: fail-closed rejections (plan.Dim != NumExperts, empty
    # bands), plus shapes outside the fixed router order.
    w, d = _tiny()
    with pytest.raises(ValueError):
        orc.moe_ffn(d, w.E + 1, w.I, w.Is, 0, w.E, w.topk)  # experts E != router E
    with pytest.raises(ValueError):
        orc.moe_ffn(d, w.E, w.I, w.Is, 3, 3, w.topk)  # empty band
    with pytest.raises(ValueError):
        orc.moe_ffn(d, w.E, w.I, w.Is, 0, w.E + 1, w.topk)
    with pytest.raises(ValueError):
        orc.moe_ffn(d, w.E, w.I, w.Is, 0, w.E, w.E + 1)
    with pytest.raises(ValueError):
        orc.router_logits(d["x"][:, :128], d["router_w"][:, :128], None)


def test_zipf_workload_popularity():
    # The prefill workload's router bias is drawn so that expert popularity
    # follows Zipf(1.1): measure the realised histogram with the oracle router.
    w = synth.WORKLOADS["prefill"]
    r = synth.make_router(w, "cpu")
    ids, _ = orc.topk(orc.router_logits(r["x"], r["router_w"], r["bias"]), w.topk)
    c = np.sort(torch.bincount(ids.flatten().long(), minlength=w.E).numpy())[::-1]
    ranks = np.arange(1, w.E + 1)
    slope = np.polyfit(np.log(ranks[1:128]), np.log(np.maximum(c[1:128], 1)), 1)[0]
    assert -1.25 <= slope <= -0.95, slope
    assert c.max() <= w.T and c.sum() == w.T * w.topk
