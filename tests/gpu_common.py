"""Helpers for the GPU parity tests: run the HIP library through its C ABI and
the CPU oracle on the same seeded inputs, and compare.

The oracle never sees anything the GPU computed: its inputs are CPU copies of
the seeded input tensors, and the experts it needs are chosen from the
oracle's own routing.
"""

from __future__ import annotations

import math
import sys
import time

import torch

import mixture_experts_ffn_06_amd as moe
import synth
from oracle import oracle as orc

# the benchmark spec tolerance on fp32 outputs against the oracle
REL_MAX = 2e-2
COS_MIN = 0.9999


def log(msg: str):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def gpu_inputs(w: synth.Workload) -> dict:
    return synth.make_inputs(w, "cuda")


def run_gpu(w: synth.Workload, d: dict, lo=None, hi=None, shared=True, topk=None, exports=True):
    lo = w.band_lo if lo is None else lo
    hi = w.band_hi if hi is None else hi
    topk = w.topk if topk is None else topk
    ex = {} if exports else None
    y = moe.moe_ffn(d["x"], d["router_w"], d["bias"], d["experts"], d["shared"] if shared else None,
                    lo, hi, topk, exports=ex)
    torch.cuda.synchronize()
    return y, ex


class OracleSide:
    """CPU copies of one workload's inputs for the oracle."""

    def __init__(self, w: synth.Workload, d: dict, topk=None):
        self.w = w
        self.k = w.topk if topk is None else topk
        self.x = d["x"].cpu()
        self.wr = d["router_w"].cpu()
        self.bias = None if d["bias"] is None else d["bias"].cpu()
        self.logits = orc.router_logits(self.x, self.wr, self.bias)
        self.ids, self.wts = orc.topk(self.logits, self.k)
        self._gpu_experts = d["experts"]
        self._gpu_shared = d["shared"]
        self._experts = {"fmt": d["experts"]["fmt"]}
        for name, t in d["experts"].items():
            if isinstance(t, torch.Tensor):
                self._experts[name] = torch.empty(t.shape, dtype=t.dtype)  # pages stay untouched
        self._have = set()
        self.shared = None
        if d["shared"] is not None:
            self.shared = {k: v.cpu() for k, v in d["shared"].items()}

    def _fetch(self, experts):
        for e in sorted(set(experts) - self._have):
            for name, t in self._gpu_experts.items():
                if isinstance(t, torch.Tensor):
                    self._experts[name][e].copy_(t[e])
            self._have.add(e)

    def layer(self, rows, lo, hi, shared=True, combine="pick"):
        rows = torch.as_tensor(rows, dtype=torch.int32)
        need = {int(e) for e in self.ids[rows.long()].flatten().tolist() if lo <= e < hi}
        self._fetch(need)
        inputs = {"x": self.x, "router_w": self.wr, "bias": self.bias, "experts": self._experts,
                  "shared": self.shared if shared else None}
        w = self.w
        out, ids, wts = orc.moe_ffn(inputs, w.E, w.I, w.Is, lo, hi, self.k, rows=rows,
                                    combine=combine)
        return out


def compare(y_gpu: torch.Tensor, ref: torch.Tensor, what: str = ""):
    """max|delta| <= REL_MAX * max|ref| and cosine >= COS_MIN (per tensor)."""
    g = y_gpu.detach().double().cpu()
    r = ref.double()
    scale = float(r.abs().max())
    err = float((g - r).abs().max())
    cos = float((g.flatten() @ r.flatten()) / (g.norm() * r.norm() + 1e-300)) if scale > 0 else 1.0
    log(f"{what}: max|ref|={scale:.4g} max|d|={err:.3g} rel={err / max(scale, 1e-300):.3g} cos={cos:.8f}")
    if scale == 0:
        assert err == 0, what
        return
    assert err <= REL_MAX * scale, f"{what}: max|d| {err} > {REL_MAX} * {scale}"
    assert cos >= COS_MIN, f"{what}: cosine {cos}"


def check_routing(ex: dict, side: OracleSide, lo: int, hi: int):
    """ids and every dispatch array bit-exact; weights to fp32 accuracy."""
    ids_g = ex["topk_ids"].cpu()
    assert torch.equal(ids_g, side.ids), "top-k ids differ from the oracle"
    wg = ex["topk_w"].cpu().double()
    assert float((wg - side.wts).abs().max()) <= 2e-6, "top-k weights"
    counts, offsets, perm, pos = orc.dispatch(side.ids, lo, hi)
    n = perm.numel()
    assert torch.equal(ex["counts"].cpu()[: hi - lo], counts)
    assert torch.equal(ex["offsets"].cpu()[: hi - lo + 1], offsets)
    assert torch.equal(ex["perm"].cpu()[:n], perm)
    assert torch.equal(ex["pos"].cpu(), pos)


def sample_rows(T: int, n: int, seed: int = 0):
    if T <= n:
        return list(range(T))
    g = torch.Generator().manual_seed(seed)
    rest = torch.randperm(T - 2, generator=g)[: n - 2] + 1
    return sorted({0, T - 1, *rest.tolist()})


__all__ = ["gpu_inputs", "run_gpu", "OracleSide", "compare", "check_routing", "sample_rows", "log",
           "math"]
