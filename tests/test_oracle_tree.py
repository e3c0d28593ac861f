"""Pins for the oracle's canonical tree over expert ids.

[P4] "GLM-5.3-Flash on CUDA over three ranks (--tp 3) ... #310" (maintainer
reply): every sum follows one fixed tree of slices however the slices fall
over ranks, so all ranks hold the same bits.  The tree is the complete binary
tree over expert ids 0..E'-1 (E' the least power of two >= E); leaf e holds a
row's weighted output for a pick of expert e and +0.0 otherwise; an inner node
is left + right in fp32.  The oracle evaluates it recursively over node
ranges; the pins here check it against a dense numpy reduction written level
by level, against brute force for the node lookup, and against the property
the tree exists for: any split of the ids into tree nodes sums back to the
same bits.
"""

import numpy as np
import pytest
import torch

from oracle import oracle as orc


def _bits(a):
    return np.asarray(a, dtype=np.float32).view(np.int32)


def _dense_node(E, ids, vals, node_lo, level):
    """All E' leaves stored, +0.0 where no pick, reduced level by level with
    numpy float32 adds (IEEE round-to-nearest-even)."""
    Ep = 1
    while Ep < E:
        Ep *= 2
    n = vals.shape[1]
    arr = np.zeros((Ep, n), dtype=np.float32)
    for i, e in enumerate(ids):
        arr[e] = vals[i]
    sub = arr[node_lo:node_lo + (1 << level)]
    while sub.shape[0] > 1:
        sub = sub[0::2] + sub[1::2]
    return sub[0]


def _rand_vals(rng, m, n):
    """Values whose sums depend on association: mixed magnitudes, signs and
    some negative zeros."""
    mag = np.float32(10.0) ** rng.integers(-6, 7, size=(m, n)).astype(np.float32)
    v = (rng.standard_normal((m, n)).astype(np.float32) * mag).astype(np.float32)
    v[rng.random((m, n)) < 0.05] = np.float32(-0.0)
    return v


@pytest.mark.parametrize("E", [1, 2, 8, 130, 256, 1000, 1024])
def test_tree_value_matches_dense_level_reduction(E):
    rng = np.random.default_rng(E)
    for trial in range(40):
        m = int(rng.integers(0, min(E, 16) + 1))
        ids = rng.choice(E, size=m, replace=False).astype(np.int32)
        vals = _rand_vals(rng, m, 24)
        lo = int(rng.integers(0, E))
        hi = int(rng.integers(lo + 1, E + 1))
        nlo, lev = orc.tree_node(E, lo, hi)
        # leaves outside the band are +0.0: keep only the band's picks
        keep = [(i, e) for i, e in enumerate(ids) if lo <= e < hi]
        kid = np.array([e for _, e in keep], dtype=np.int32)
        kv = vals[[i for i, _ in keep]] if keep else np.zeros((0, 24), np.float32)
        got = orc.tree_value(kid, torch.from_numpy(kv), nlo, lev).numpy()
        want = _dense_node(E, kid, kv, nlo, lev)
        assert (_bits(got) == _bits(want)).all(), (E, trial, lo, hi)


def test_tree_node_brute_force():
    for E in (1, 5, 8, 130, 256):
        for lo in range(E):
            for hi in range(lo + 1, E + 1):
                nlo, lev = orc.tree_node(E, lo, hi)
                # the smallest aligned power-of-two range containing [lo, hi)
                best = None
                for L in range(0, 12):
                    a = (lo >> L) << L
                    if a + (1 << L) >= hi:
                        best = (a, L)
                        break
                assert (nlo, lev) == best, (E, lo, hi)


def test_tree_node_known_values():
    assert orc.tree_node(256, 0, 256) == (0, 8)
    assert orc.tree_node(256, 32, 64) == (32, 5)
    assert orc.tree_node(256, 30, 34) == (0, 6)   # straddles 32: the node [0, 64)
    assert orc.tree_node(130, 128, 130) == (128, 1)
    assert orc.tree_node(130, 0, 130) == (0, 8)
    assert orc.tree_node(8, 5, 6) == (5, 0)


def _random_node_split(rng, nlo, lev, E, out):
    """Cut the node [nlo, nlo + 2^lev) clipped to [0, E) into tree nodes."""
    if nlo >= E:
        return
    if lev == 0 or rng.random() < 0.35:
        hi = min(nlo + (1 << lev), E)
        # the band of a part is its node clipped to [0, E); shrink the node
        # to the smallest one containing the band, as a band call does
        out.append((nlo, hi))
        return
    _random_node_split(rng, nlo, lev - 1, E, out)
    _random_node_split(rng, nlo + (1 << (lev - 1)), lev - 1, E, out)


def _band_value(E, ids, vals, lo, hi):
    keep = [i for i, e in enumerate(ids) if lo <= e < hi]
    nlo, lev = orc.tree_node(E, lo, hi)
    kid = ids[keep]
    kv = vals[keep] if keep else np.zeros((0, vals.shape[1]), np.float32)
    return orc.tree_value(kid, torch.from_numpy(kv), nlo, lev)


@pytest.mark.parametrize("E", [8, 130, 256, 1024])
def test_any_node_split_merges_to_the_full_tree_bit_exact(E):
    rng = np.random.default_rng(100 + E)
    Ep = 1
    while Ep < E:
        Ep *= 2
    root_lev = Ep.bit_length() - 1
    for trial in range(30):
        m = int(rng.integers(1, min(E, 16) + 1))
        ids = rng.choice(E, size=m, replace=False).astype(np.int32)
        vals = _rand_vals(rng, m, 32)
        full = _band_value(E, ids, vals, 0, E)
        bands = []
        _random_node_split(rng, 0, root_lev, E, bands)
        parts = [_band_value(E, ids, vals, lo, hi) for lo, hi in bands]
        merged = orc.tree_merge(parts, bands, E)
        assert (_bits(merged.numpy()) == _bits(full.numpy())).all(), (E, trial, bands)


def test_plain_band_order_sum_differs_from_the_tree():
    """The property is not automatic: a left-to-right sum of the same
    partials loses it on values chosen to expose association."""
    E = 8
    ids = np.array([0, 2, 4, 6], dtype=np.int32)
    vals = np.array([[1e8], [1.0], [-1e8], [1.0]], dtype=np.float32)
    bands = [(0, 2), (2, 4), (4, 6), (6, 8)]
    parts = [_band_value(E, ids, vals, lo, hi) for lo, hi in bands]
    full = _band_value(E, ids, vals, 0, E).item()
    # tree: (1e8 + 1) + (-1e8 + 1) = 1e8 + (-1e8) = 0 (each inner sum rounds)
    assert orc.tree_merge(parts, bands, E).item() == full == 0.0
    fold = np.float32(0.0)
    for p in parts:
        fold = np.float32(fold + np.float32(p.item()))
    assert fold == 1.0  # ((1e8 + 1) - 1e8) + 1


def test_merge_adds_shared_last():
    E = 16
    rng = np.random.default_rng(7)
    ids = np.array([1, 9], dtype=np.int32)
    vals = _rand_vals(rng, 2, 8)
    parts = [_band_value(E, ids, vals, 0, 8), _band_value(E, ids, vals, 8, 16)]
    sh = torch.from_numpy(rng.standard_normal(8).astype(np.float32))
    got = orc.tree_merge(parts, [(0, 8), (8, 16)], E, shared=sh).numpy()
    want = (_dense_node(E, ids, vals, 0, 4) + sh.numpy()).astype(np.float32)
    assert (_bits(got) == _bits(want)).all()


def test_signed_zero_follows_the_dense_tree():
    E = 8
    mz = np.array([[-0.0]], dtype=np.float32)
    # a leaf node keeps -0.0; any larger node adds +0.0 siblings -> +0.0
    assert _bits(orc.tree_value([3], torch.from_numpy(mz), 3, 0).numpy())[0] == _bits(np.float32(-0.0))
    assert _bits(orc.tree_value([3], torch.from_numpy(mz), 2, 1).numpy())[0] == 0
    # two -0.0 siblings stay -0.0; under a larger node they become +0.0
    two = np.array([[-0.0], [-0.0]], dtype=np.float32)
    assert _bits(orc.tree_value([2, 3], torch.from_numpy(two), 2, 1).numpy())[0] == _bits(np.float32(-0.0))
    assert _bits(orc.tree_value([2, 3], torch.from_numpy(two), 0, 3).numpy())[0] == 0
    # no leaf at all: +0.0
    assert _bits(orc.tree_value([], torch.zeros(0, 1), 0, 3).numpy())[0] == 0


def test_merge_rejects_bands_that_are_not_nodes():
    z = torch.zeros(4)
    with pytest.raises(ValueError):
        orc.tree_merge([z, z], [(0, 3), (3, 8)], 8)      # [0, 3) is no node
    with pytest.raises(ValueError):
        orc.tree_merge([z, z], [(0, 4), (5, 8)], 8)      # gap
    with pytest.raises(ValueError):
        orc.tree_merge([z, z], [(4, 8), (0, 4)], 8)      # out of order
    with pytest.raises(ValueError):
        orc.tree_merge([z, z], [(2, 4), (4, 6)], 8)      # union [2, 6) is no node
    # E not a power of two: the last band may end at E
    assert orc.tree_merge([z, z], [(0, 128), (128, 130)], 130).shape == (4,)


# --------------------------------------------------------------------------
# The layer in tree mode (fp64 after the selection, like the pick-order mode).
# --------------------------------------------------------------------------

def _tiny(**kw):
    import synth
    w = synth.WORKLOADS["tiny"].with_(**kw)
    return w, synth.make_inputs(w, "cpu")


def test_layer_tree_single_pick_equals_pick_order():
    # one pick: the tree adds only +0.0 siblings to w * y
    w, d = _tiny(topk=1, T=5)
    for lo, hi in ((0, 8), (0, 4), (2, 3)):
        a, _, _ = orc.moe_ffn(d, w.E, w.I, w.Is, lo, hi, 1, combine="pick")
        b, _, _ = orc.moe_ffn(d, w.E, w.I, w.Is, lo, hi, 1, combine="tree")
        assert torch.equal(a, b)


def test_layer_tree_is_a_reassociation_of_pick_order():
    w, d = _tiny(T=6, topk=4)
    a, _, wt = orc.moe_ffn(d, w.E, w.I, w.Is, 0, w.E, w.topk, combine="pick")
    b, _, _ = orc.moe_ffn(d, w.E, w.I, w.Is, 0, w.E, w.topk, combine="tree")
    scale = float(a.abs().max())
    assert float((a - b).abs().max()) <= 16 * 2.0 ** -52 * scale


def test_layer_tree_node_bands_add_up_in_the_tree():
    # fp64 partials of the tree-mode layer over node bands, added along the
    # tree by hand, equal the full band's tree value (no shared expert)
    w, d = _tiny(T=5, topk=3)
    d = dict(d)
    d["shared"] = None
    full, _, _ = orc.moe_ffn(d, w.E, w.I, w.Is, 0, 8, w.topk, combine="tree")
    p = {b: orc.moe_ffn(d, w.E, w.I, w.Is, b[0], b[1], w.topk, combine="tree")[0]
         for b in ((0, 2), (2, 4), (4, 8))}
    assert torch.equal((p[(0, 2)] + p[(2, 4)]) + p[(4, 8)], full)
