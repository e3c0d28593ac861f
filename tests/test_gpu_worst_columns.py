"""Worst-column errors of the expert FFN, per projection class.

[P5] "GLM-5.3-Flash and full GLM-5.3 on the native CUDA engine (tracker)
#593", "The gate": an FP64 reference for every projection class whose
reduction order changes, reported with worst-column errors.

Each class is one call whose routed groups all take the same path: a zero
router with a bias that sends every row to the same k experts, so each group
holds all T rows and T picks the path (1..8 rows: GEMV; 9..32, 33..64,
65..128 rows: one MFMA tile of that height; more: 256-row tiles, the last
partial).  The per-pick expert outputs y_picks (before weighting) of sampled
picks are compared with the oracle's fp64 expert FFN of the same row.  For
every output column c: err[c] = max over the sampled picks of |y - ref|;
the worst column is the one with the largest err[c] relative to the class's
max|ref|.  The bar is the layer's: worst err <= 2e-2 * max|ref| (and cosine
>= 0.9999 over the class); the measured worst columns are printed.
"""

import pytest
import torch

import mixture_experts_ffn_06_amd as moe
import synth
from gpu_common import COS_MIN, REL_MAX, log, sample_rows
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

# full-size expert shapes, few experts (only the k picked ones are read)
BASE = synth.Workload("classes", T=1, H=6144, E=8, topk=4, I=2048, Is=0)
CLASSES = [("gemv", 5), ("mfma32", 20), ("mfma64", 50), ("mfma128", 100), ("mfma256", 300)]


@pytest.fixture(scope="module", params=["bf16", "w4", "affine4", "nvfp4"])
def experts(request):
    w = BASE.with_(fmt=request.param)
    return w, synth.make_experts(w, "cuda")


@pytest.mark.parametrize("cls,T", CLASSES)
def test_worst_column_per_class(experts, cls, T):
    w0, ex_gpu = experts
    w = w0.with_(T=T)
    d = synth.make_router(w, "cuda")
    d["router_w"].zero_()
    bias = torch.zeros(w.E)
    picks = (5, 1, 6, 2)
    for j, e in enumerate(picks):
        bias[e] = 10.0 - j
    y_picks = torch.empty((T * w.topk, w.H), device="cuda")
    ex = {}
    moe.moe_ffn(d["x"], d["router_w"], bias.cuda(), ex_gpu, None, 0, w.E, w.topk, exports=ex,
                y_picks=y_picks)
    torch.cuda.synchronize()
    assert ex["counts"].cpu().tolist() == [T if e in picks else 0 for e in range(w.E)]
    perm = ex["perm"].cpu()
    ids = ex["topk_ids"].cpu()
    cpu_ex = {"fmt": ex_gpu["fmt"]}
    for name, t in ex_gpu.items():
        if isinstance(t, torch.Tensor):
            cpu_ex[name] = torch.zeros(t.shape, dtype=t.dtype)
            for e in picks:
                cpu_ex[name][e].copy_(t[e])
    oe = orc.Experts(cpu_ex, w.E, w.H, w.I)
    x = d["x"].cpu()
    rows = sample_rows(T * w.topk, 12, seed=T)
    got, ref = [], []
    for r in rows:
        t, j = divmod(int(perm[r]), w.topk)
        ref.append(orc.expert_ffn(x[t].double(), oe, int(ids[t, j])))
        got.append(y_picks[r].cpu().double())
    got, ref = torch.stack(got), torch.stack(ref)
    scale = float(ref.abs().max())
    err_col = (got - ref).abs().max(dim=0).values
    c = int(err_col.argmax())
    worst = float(err_col[c])
    cos = float((got.flatten() @ ref.flatten()) / (got.norm() * ref.norm()))
    mean_rel = float(err_col.mean() / scale)
    log(f"worst column {w.fmt} {cls} (T={T}, {len(rows)} picks): column {c} max|d|={worst:.3g} "
        f"= {worst / scale:.3g} x max|ref| ({scale:.3g}); mean column {mean_rel:.3g}; cos={cos:.8f}")
    assert worst <= REL_MAX * scale
    assert cos >= COS_MIN
