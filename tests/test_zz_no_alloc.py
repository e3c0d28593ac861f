"""moe_ffn_static (scratch in the library's static per-GPU array, no
allocation in the call) against moe_ffn (caller's workspace): the same
kernels, so outputs and every routing export must agree bit for bit.  Two
calls in a row, the second with fewer rows, so the second reuses the array
the first left full; in every weight format, on the GEMV and MFMA paths.
"""

import pytest
import torch

import mixture_experts_ffn_06_amd as moe
import synth
from gpu_common import log

pytestmark = pytest.mark.gpu

BIG = synth.Workload("noalloc", T=100, H=2048, E=64, topk=8, I=512, Is=256)
EXPORTS = ("topk_ids", "topk_w", "counts", "offsets", "pos")
FMT_CODE = {"bf16": moe.MOE_BF16, "w4": moe.MOE_W4A16, "affine4": moe.MOE_AFFINE4, "nvfp4": moe.MOE_NVFP4}


def _run(fn, w, d, T, **kw):
    x = d["x"][:T]
    ex = {}
    y = fn(x, d["router_w"], d["bias"], d["experts"], d["shared"], 0, w.E, w.topk, exports=ex, **kw)
    torch.cuda.synchronize()
    return y, ex


@pytest.mark.parametrize("fmt", ["bf16", "w4", "affine4", "nvfp4"])
def test_static_matches_workspace_entry_two_calls(fmt):
    w = BIG.with_(fmt=fmt)
    d = synth.make_inputs(w, "cuda")
    # a falling bias makes groups of every size: MFMA tiles and GEMV groups
    d["bias"] = (-0.05 * torch.arange(w.E, dtype=torch.float32)).cuda()
    for T in (w.T, 5):
        log(f"moe_ffn_static vs moe_ffn: fmt={fmt} T={T}")
        need = moe.workspace_bytes(T, w.H, w.E, w.I, w.Is, w.topk, FMT_CODE[fmt])
        assert need <= moe.MOE_STATIC_SCRATCH_BYTES
        y_ref, ex_ref = _run(moe.moe_ffn, w, d, T)
        y_st, ex_st = _run(moe.moe_ffn_static, w, d, T)
        assert torch.equal(y_st, y_ref), f"T={T}: outputs differ"
        for k in EXPORTS:
            assert torch.equal(ex_st[k], ex_ref[k]), f"T={T}: {k} differs"
        n = int(ex_ref["offsets"][-1])
        assert torch.equal(ex_st["perm"][:n], ex_ref["perm"][:n])
        # run to run through the static array
        y_again, _ = _run(moe.moe_ffn_static, w, d, T)
        assert torch.equal(y_again, y_ref)


def test_static_rejects_sizes_beyond_the_array():
    # T = 4096 rows at these sizes need far more than the array: rejected
    # before anything is enqueued, and the output is left untouched
    w = synth.Workload("noalloc_big", T=4096, H=2048, E=64, topk=8, I=512, Is=256)
    assert moe.workspace_bytes(w.T, w.H, w.E, w.I, w.Is, w.topk) > moe.MOE_STATIC_SCRATCH_BYTES
    d = synth.make_inputs(w, "cuda")
    out = torch.full((w.T, w.H), 7.0, device="cuda")
    with pytest.raises(moe.MoeError) as err:
        moe.moe_ffn_static(d["x"], d["router_w"], d["bias"], d["experts"], d["shared"], 0, w.E,
                           w.topk, out=out)
    assert err.value.code == -13
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
