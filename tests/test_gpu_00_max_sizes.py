"""GPU parity at the header's maximum sizes: the HIP library (through its C
ABI) against the CPU oracle on sampled rows.

It sits in a file of its own that sorts before the other GPU test files, so it
runs first: freeing its 26 GB workspace is followed by several seconds of lower
HBM throughput on this GPU (a decode layer measured 3% slower in the next
process), and running it first leaves the rest of the suite between it and
any later timing.
"""

import pytest
import torch

import synth
from gpu_common import compare, gpu_inputs, log, run_gpu, sample_rows
from oracle import oracle as orc

pytestmark = pytest.mark.gpu


def test_maximum_sizes_sampled():
    # The header's limits at once: 2^20 rows, 1024 experts, top-16 (H and I
    # small so the 26 GB workspace fits).  Routing of sampled rows against the
    # oracle; every dispatch array against the oracle's dispatch of the GPU's
    # ids; outputs of a few rows against the oracle's layer.
    w = synth.Workload("max", T=1 << 20, H=256, E=1024, topk=16, I=64, Is=64)
    log(f"case {w}")
    d = gpu_inputs(w)
    y, ex = run_gpu(w, d)
    rows = torch.tensor(sorted(set(sample_rows(w.T, 512, seed=5)) | {0, w.T - 1}), dtype=torch.long)
    x = d["x"].cpu()
    wr = d["router_w"].cpu()
    ids, wts = orc.topk(orc.router_logits(x[rows], wr, None), w.topk)
    ids_g = ex["topk_ids"].cpu()
    assert torch.equal(ids_g[rows], ids), "top-k ids differ from the oracle"
    assert float((ex["topk_w"].cpu()[rows].double() - wts).abs().max()) <= 2e-6
    counts, offsets, perm, pos = orc.dispatch(ids_g, 0, w.E)
    assert torch.equal(ex["counts"].cpu()[: w.E], counts)
    assert torch.equal(ex["offsets"].cpu()[: w.E + 1], offsets)
    assert torch.equal(ex["perm"].cpu()[: perm.numel()], perm)
    assert torch.equal(ex["pos"].cpu(), pos)
    log(f"group sizes: min {int(counts.min())} max {int(counts.max())}")
    orows = rows[:8]
    experts = {"fmt": d["experts"]["fmt"]}
    need = sorted({int(e) for e in ids_g[orows].flatten().tolist()})
    for name, t in d["experts"].items():
        if isinstance(t, torch.Tensor):
            experts[name] = torch.empty(t.shape, dtype=t.dtype)
            for e in need:
                experts[name][e].copy_(t[e])
    inputs = {"x": x, "router_w": wr, "bias": None, "experts": experts,
              "shared": {k: v.cpu() for k, v in d["shared"].items()}}
    ref, _, _ = orc.moe_ffn(inputs, w.E, w.I, w.Is, 0, w.E, w.topk, rows=orows.to(torch.int32))
    compare(y[orows.cuda()], ref, "maximum sizes, sampled rows")
