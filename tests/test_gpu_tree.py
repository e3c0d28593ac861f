"""GPU: the canonical-tree combine and the sum of band partials.

[P4] "GLM-5.3-Flash on CUDA over three ranks (--tp 3) ... #310", maintainer
reply: every sum follows one fixed tree of slices however the slices fall over
ranks, so every rank holds the same bits; [P2] "GLM-5.3-Flash on CUDA:
attention on one GPU, routed experts on the Sparks (proposal) #214", "Per MoE
layer": the partials are summed in rank order.

The tree combine is checked bit for bit against the oracle's fp32 tree applied
to the GPU's own leaves (its exported per-pick outputs and weights), within
tolerance against the oracle's layer, and by the property it exists for: the
outputs of any split into tree nodes, added by moe_ffn_reduce along the tree,
equal the full band's bits.
"""

import numpy as np
import pytest
import torch

import mixture_experts_ffn_06_amd as moe
import synth
from gpu_common import OracleSide, compare, gpu_inputs, log
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
MID = synth.Workload("mid", T=300, H=512, E=16, topk=4, I=192, Is=128)
ODD = synth.Workload("odd", T=90, H=768, E=40, topk=6, I=128, Is=128)


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int32)


def _call(w, d, lo, hi, combine="tree", shared=True, y_shared=None, y_picks=None, exports=None):
    y = moe.moe_ffn(d["x"], d["router_w"], d["bias"], d["experts"], d["shared"] if shared else None,
                    lo, hi, w.topk, exports=exports, combine=combine, y_shared=y_shared,
                    y_picks=y_picks)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("wname,fmt", [("mid", "bf16"), ("odd", "bf16"), ("odd", "w4"), ("odd", "affine4"),
                                      ("odd", "nvfp4")])
def test_tree_combine_bit_exact_from_gpu_leaves(wname, fmt):
    w = {"mid": MID, "odd": ODD}[wname].with_(fmt=fmt)
    d = gpu_inputs(w)
    d["bias"] = (-0.3 * torch.arange(w.E, dtype=torch.float32)).cuda()
    T, H, k = w.T, w.H, w.topk
    for lo, hi in ((0, w.E), (0, 4), (3, 11), (8, 16), (w.E - 1, w.E)):
        log(f"case {wname}/{fmt} band [{lo},{hi})")
        ex = {}
        ysh = torch.empty((T, H), dtype=torch.float32, device="cuda")
        ypk = torch.empty((T * k, H), dtype=torch.float32, device="cuda")
        y = _call(w, d, lo, hi, y_shared=ysh, y_picks=ypk, exports=ex)
        ids = ex["topk_ids"].cpu()
        wts = ex["topk_w"].cpu()
        pos = ex["pos"].cpu().view(T, k)
        ypk = ypk.cpu()
        nlo, lev = orc.tree_node(w.E, lo, hi)
        bad = 0
        for t in range(T):
            js = [j for j in range(k) if int(pos[t, j]) >= 0]
            leaf_ids = [int(ids[t, j]) for j in js]
            if js:
                vals = torch.stack([(wts[t, j] * ypk[int(pos[t, j])]).float() for j in js])
            else:
                vals = torch.zeros((0, H))
            want = orc.tree_value(leaf_ids, vals, nlo, lev)
            if not torch.equal(_bits(want), _bits(y[t])):
                bad += 1
        assert bad == 0, f"{bad} rows differ from the oracle tree on the GPU's leaves"
        # the shared expert went to y_shared: adding it back gives the call
        # that adds it itself, bit for bit
        y_add = _call(w, d, lo, hi)
        assert torch.equal(_bits(y + ysh), _bits(y_add))


def test_shared_apart_pick_order_bit_exact():
    w = MID
    d = gpu_inputs(w)
    ysh = torch.empty((w.T, w.H), dtype=torch.float32, device="cuda")
    y = _call(w, d, 0, w.E, combine="pick", y_shared=ysh)
    y_add = _call(w, d, 0, w.E, combine="pick")
    assert torch.equal(_bits(y + ysh), _bits(y_add))


@pytest.mark.parametrize("fmt", ["bf16", "w4", "affine4", "nvfp4"])
def test_tree_combine_against_the_oracle_layer(fmt):
    w = MID.with_(fmt=fmt, I=256 if fmt == "affine4" else MID.I)  # MLX affine needs I % 128 == 0
    d = gpu_inputs(w)
    d["bias"] = (-0.5 * torch.arange(w.E, dtype=torch.float32)).cuda()
    side = OracleSide(w, d)
    for lo, hi in ((0, w.E), (4, 8), (2, 13)):
        y = _call(w, d, lo, hi)
        compare(y, side.layer(list(range(w.T)), lo, hi, combine="tree"), f"tree {fmt} [{lo},{hi})")


def _random_node_split(rng, nlo, lev, E, out, force_above=99):
    if nlo >= E:
        return
    if lev == 0 or (lev <= force_above and rng.random() < 0.4):
        out.append((nlo, min(nlo + (1 << lev), E)))
        return
    _random_node_split(rng, nlo, lev - 1, E, out, force_above)
    _random_node_split(rng, nlo + (1 << (lev - 1)), lev - 1, E, out, force_above)


def _split_runs(w, d, bands):
    """Tree-mode calls for every band (the shared expert written apart by
    the first), added back by moe_ffn_reduce along the tree."""
    parts = []
    ysh = torch.empty((w.T, w.H), dtype=torch.float32, device="cuda")
    for i, (lo, hi) in enumerate(bands):
        parts.append(_call(w, d, lo, hi, shared=(i == 0), y_shared=ysh if i == 0 else None))
    y = moe.reduce(parts, "tree", bands=bands, E=w.E, y_shared=ysh)
    torch.cuda.synchronize()
    return y


def test_any_tree_split_equals_the_full_band_bit_exact():
    w = W["bands"]
    d = gpu_inputs(w)
    full = _call(w, d, 0, w.E)
    rng = np.random.default_rng(11)
    splits = {"bands of 32": list(synth.bands(w))}
    s = []
    _random_node_split(rng, 0, 8, w.E, s, force_above=5)  # at least 8 parts
    splits["random nodes"] = s
    # an arbitrary contiguous split, each band cut into its tree nodes
    pieces = []
    for lo, hi in ((0, 37), (37, 100), (100, 101), (101, 256)):
        pieces += moe.tree_pieces(lo, hi, w.E)
    splits["arbitrary bands as nodes"] = pieces
    for name, bands in splits.items():
        log(f"split {name}: {len(bands)} parts")
        y = _split_runs(w, d, bands)
        assert torch.equal(_bits(y), _bits(full)), name
    # the plain band-order sum of the same 32-expert partials is only close
    acc = None
    for i, (lo, hi) in enumerate(synth.bands(w)):
        p = _call(w, d, lo, hi, shared=(i == 0))
        acc = p if acc is None else acc + p
    drift = float((acc - full).abs().max())
    log(f"band-order sum of tree partials: max|d| = {drift:.3g}")
    assert drift <= (w.topk + 2) * 2.0 ** -23 * 4 * float(full.abs().max())


def test_tree_split_adversarial_band():
    w = W["bands_adversarial"]
    d = gpu_inputs(w)
    full = _call(w, d, 0, w.E)
    y = _split_runs(w, d, list(synth.bands(w)))
    assert torch.equal(_bits(y), _bits(full))


def test_tree_split_non_power_of_two_experts():
    w = ODD  # E = 40: the tree has 64 leaves, 40..63 always +0.0
    d = gpu_inputs(w)
    full = _call(w, d, 0, w.E)
    for bands in ([(0, 32), (32, 40)], moe.tree_pieces(0, 13, 40) + moe.tree_pieces(13, 40, 40)):
        y = _split_runs(w, d, bands)
        assert torch.equal(_bits(y), _bits(full)), bands


@pytest.mark.parametrize("E", [8, 130, 256])
def test_reduce_tree_matches_the_oracle_merge(E):
    rng = np.random.default_rng(E)
    T, H = 3, 512
    for trial in range(5):
        bands = []
        lev = max(1, (E - 1).bit_length())
        _random_node_split(rng, 0, lev, E, bands)
        bands = bands[:64]
        if bands[-1][1] != E:
            continue
        g = torch.Generator().manual_seed(trial)
        mag = 10.0 ** torch.randint(-5, 6, (len(bands), T, H), generator=g).float()
        parts = [(torch.randn(T, H, generator=g) * mag[i]).contiguous() for i in range(len(bands))]
        sh = torch.randn(T, H, generator=g)
        res = torch.randn(T, H, generator=g).to(torch.bfloat16)
        y = moe.reduce([p.cuda() for p in parts], "tree", bands=bands, E=E, y_shared=sh.cuda(),
                       residual=res.cuda())
        want = orc.tree_merge([p.flatten() for p in parts], bands, E, shared=sh.flatten())
        want = (want.reshape(T, H) + res.float()).contiguous()
        assert torch.equal(_bits(y), _bits(want)), (E, trial, bands)


@pytest.mark.parametrize("nparts", [1, 2, 5, 8])
def test_reduce_rank_order_matches_the_oracle(nparts):
    # partials of very different scales (fp32 addition is not associative on
    # them), the shared output and a residual: bit-exact against the oracle's
    # rank-order merge
    g = torch.Generator().manual_seed(3 + nparts)
    T, H = 5, 768
    parts = [(torch.randn(T, H, generator=g) * 10.0 ** (3 * (i % 4))).cuda() for i in range(nparts)]
    sh = torch.randn(T, H, generator=g).cuda()
    res = torch.randn(T, H, generator=g).to(torch.bfloat16).cuda()
    y = moe.reduce(parts, "rank", y_shared=sh, residual=res)
    want = orc.rank_merge([p.cpu() for p in parts], shared=sh.cpu(), residual=res.cpu())
    assert torch.equal(_bits(y.cpu()), _bits(want))
    y2 = moe.reduce(parts, "rank")
    assert torch.equal(_bits(y2.cpu()), _bits(orc.rank_merge([p.cpu() for p in parts])))


def test_reduce_rejects_bad_parts():
    z = torch.zeros(2, 256, device="cuda")
    for bands, code in (([(0, 3), (3, 8)], -4), ([(0, 4), (5, 8)], -4), ([(4, 8), (0, 4)], -4),
                        ([(2, 4), (4, 6)], -4)):
        with pytest.raises(moe.MoeError) as e:
            moe.reduce([z, z], "tree", bands=bands, E=8)
        assert e.value.code == code
    with pytest.raises(moe.MoeError) as e:
        moe.reduce([z] * 65, "rank")
    assert e.value.code == -2
    lib = moe.load_library()
    import ctypes
    arr = (ctypes.c_void_p * 1)(z.data_ptr())
    rc = lib.moe_ffn_reduce(ctypes.cast(arr, ctypes.c_void_p), 1, None, None, 8, 7, None, None, 2, 256,
                            z.data_ptr(), None)
    assert rc == -11
