"""The layer inside a HIP graph: one moe_ffn call captured on a stream, the
graph replayed several times with the program's own eager work and
synchronisations between the replays, every replay checked bit for bit
against the eager call on the same inputs (the kernels are deterministic and
the call enqueues no allocation, copy, memset or host synchronisation).

Covers the decode-sized path (GEMV groups), the 4-bit path at one row, and a
batch with every MFMA tile list and the multi-block dispatch.
"""

import pytest
import torch

import mixture_experts_ffn_06_amd as moe
import synth
from gpu_common import gpu_inputs, log

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
MID = synth.Workload("mid", T=300, H=512, E=16, topk=4, I=192, Is=128)


def _capture_and_replay(w, d, replays=3, **opts):
    dev = d["x"].device
    out = torch.empty((w.T, w.H), dtype=torch.float32, device=dev)
    ws = torch.empty((moe.workspace_bytes(w.T, w.H, w.E, w.I, w.Is, w.topk, 0 if w.fmt == "bf16" else 1),),
                     dtype=torch.uint8, device=dev)

    def call():
        moe.moe_ffn(d["x"], d["router_w"], d["bias"], d["experts"], d["shared"], w.band_lo, w.band_hi,
                    w.topk, out=out, workspace=ws, **opts)

    call()
    torch.cuda.synchronize()
    ref = out.clone()
    # warm-up on a side stream, as capture requires, then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for i in range(replays):
        out.fill_(float("nan"))  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i} differs from the eager call"
    log(f"{w.name}: {replays} replays equal the eager call")


@pytest.mark.parametrize("wname", ["decode", "w4_t1", "affine4_t1", "nvfp4_t1"])
def test_graph_replay_full_size(wname):
    w = W[wname]
    _capture_and_replay(w, gpu_inputs(w))


@pytest.mark.parametrize("fmt", ["bf16", "w4", "affine4", "nvfp4"])
def test_graph_replay_mfma_lists_and_multiblock_dispatch(fmt):
    w = MID.with_(fmt=fmt, I=256 if fmt == "affine4" else MID.I)  # MLX affine needs I % 128 == 0
    d = gpu_inputs(w)
    d["bias"] = (-0.35 * torch.arange(w.E, dtype=torch.float32)).cuda()  # groups of 0 to > 256 rows
    _capture_and_replay(w, d)


def test_graph_replay_tree_combine_norm_residual():
    w = MID
    d = gpu_inputs(w)
    gamma = (1.0 + 0.05 * torch.randn(w.H, generator=torch.Generator().manual_seed(3))).to(torch.bfloat16).cuda()
    _capture_and_replay(w, d, combine="tree", norm=gamma, residual=True)
