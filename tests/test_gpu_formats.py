"""GPU parity of the MLX affine and NVFP4 expert formats: the HIP library
(through its C ABI) against the CPU oracle on the same seeded inputs, to the
layer's bar (ids and dispatch bit for bit; max|delta| <= 2e-2 * max|ref|,
cosine >= 0.9999).

Pages: [P5] "GLM-5.3-Flash and full GLM-5.3 on the native CUDA engine
(tracker) #593", "The pieces, in order" (quantised expert checkpoints read in
their stored form, dequantised in the kernels); [P4] "GLM-5.3-Flash on CUDA
over three ranks (--tp 3) ... #310" (whole-unit column slices per rank, added
in rank order).  MLX affine: weight = s * q + b per 64 inputs; NVFP4: weight =
e2m1(q) * e4m3(s) per 16 inputs times a per-matrix fp32 scale.
"""

import pytest
import torch

import mixture_experts_ffn_06_amd as moe
import synth
from gpu_common import OracleSide, check_routing, compare, gpu_inputs, log, run_gpu, sample_rows
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
FORMATS = ["affine4", "nvfp4"]

# Small enough for the oracle on every row, several tiles and ragged tails on
# both expert paths (a falling bias spreads the group sizes from 0 past two
# MFMA row tiles); I a multiple of 128 as MLX affine needs, not of 256.
SMALL = {
    "tiny": synth.Workload("tiny", T=4, H=256, E=8, topk=2, I=128, Is=128),
    "mid": synth.Workload("mid", T=300, H=512, E=16, topk=4, I=384, Is=128),
    "wide": synth.Workload("wide", T=70, H=1280, E=40, topk=6, I=640, Is=192),
}
BIAS_STEP = {"tiny": 0.0, "mid": 0.5, "wide": 0.15}


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("wname", ["tiny", "mid", "wide"])
def test_small_workloads_every_row(wname, fmt):
    w = SMALL[wname].with_(fmt=fmt)
    log(f"case {w}")
    d = gpu_inputs(w)
    if BIAS_STEP[wname]:
        d["bias"] = (-BIAS_STEP[wname] * torch.arange(w.E, dtype=torch.float32)).cuda()
    side = OracleSide(w, d)
    y, ex = _run(w, d)
    check_routing(ex, side, 0, w.E)
    log(f"group sizes {sorted(ex['counts'].cpu().tolist(), reverse=True)}")
    compare(y, side.layer(list(range(w.T)), 0, w.E), f"{wname}/{fmt}")


def _run(w, d, lo=None, hi=None, shared=True):
    return run_gpu(w, d, lo, hi, shared=shared)


@pytest.mark.parametrize("wname,nrows", [("affine4_t1", 1), ("affine4_t2048", 6), ("nvfp4_t1", 1),
                                         ("nvfp4_t2048", 6)])
def test_full_size(wname, nrows):
    w = W[wname]
    log(f"case {w}")
    d = gpu_inputs(w)
    side = OracleSide(w, d)
    y, ex = _run(w, d)
    check_routing(ex, side, 0, w.E)
    rows = sample_rows(w.T, nrows, seed=6)
    compare(y[rows], side.layer(rows, 0, w.E), wname)
    y2, _ = _run(w, d)
    assert torch.equal(y, y2), "run-to-run bits differ"


@pytest.mark.parametrize("fmt", FORMATS)
def test_gate_up_stride_regression(fmt):
    # Zero gate rows (affine: codes 0 with bias 0; NVFP4: code 0 is +0) give
    # silu(0) * up = 0: the routed part must vanish exactly, which reading the
    # up rows or another expert's rows at a stride of I would break.
    w = SMALL["mid"].with_(fmt=fmt)
    d = gpu_inputs(w)
    ex_ = d["experts"]
    ex_["q_gate_up"][:, : w.I, :] = 0
    if fmt == "affine4":
        ex_["z_gate_up"][:, : w.I, :] = 0
    y, _ = _run(w, d)
    side = OracleSide(w, d)
    compare(y, side.layer(list(range(w.T)), 0, w.E), f"stride regression {fmt}")
    y_routed, _ = _run(w, d, shared=False)
    assert float(y_routed.abs().max()) == 0.0


def test_nvfp4_matrix_scales_apply_per_expert_and_matrix():
    # Doubling one expert's down-matrix scale doubles that expert's pick
    # outputs exactly (a power of two on the finished sums) and leaves every
    # other pick's bits alone; a changed gate-matrix scale, which passes
    # through silu, is checked against the oracle.
    w = SMALL["mid"].with_(fmt="nvfp4")
    d = gpu_inputs(w)
    d["bias"] = (-0.5 * torch.arange(w.E, dtype=torch.float32)).cuda()
    yp0 = torch.empty((w.T * w.topk, w.H), device="cuda")
    ex0 = {}
    moe.moe_ffn(d["x"], d["router_w"], d["bias"], d["experts"], None, 0, w.E, w.topk, exports=ex0,
                y_picks=yp0)
    e_star = 1
    d["experts"]["g_down"][e_star] *= 2.0
    yp1 = torch.empty_like(yp0)
    ex1 = {}
    moe.moe_ffn(d["x"], d["router_w"], d["bias"], d["experts"], None, 0, w.E, w.topk, exports=ex1,
                y_picks=yp1)
    torch.cuda.synchronize()
    off = ex0["offsets"].cpu()
    lo, hi = int(off[e_star]), int(off[e_star + 1])
    assert hi > lo
    assert torch.equal(yp1[lo:hi], 2.0 * yp0[lo:hi])
    assert torch.equal(yp1[:lo], yp0[:lo]) and torch.equal(yp1[hi:], yp0[hi:])
    # and the whole layer with a changed gate scale against the oracle
    d["experts"]["g_gate_up"][e_star, 0] *= 3.0
    side = OracleSide(w, d)
    y, ex = _run(w, d)
    compare(y, side.layer(list(range(w.T)), 0, w.E), "nvfp4 changed matrix scales")


def _cpu_copy(experts):
    return {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in experts.items()}


TPW = synth.Workload("tpw", T=120, H=512, E=16, topk=4, I=384, Is=384)
CUTS = {"affine4": ((0, 128), (128, 384), (256, 384)), "nvfp4": ((0, 64), (64, 320), (128, 192))}


@pytest.mark.parametrize("fmt", FORMATS)
def test_tp_slices_hold_the_named_columns(fmt):
    w = TPW.with_(fmt=fmt)
    d = gpu_inputs(w)
    cpu = _cpu_copy(d["experts"])
    for i_lo, i_hi in CUTS[fmt]:
        s = moe.tp_slice_experts(d["experts"], i_lo, i_hi)
        torch.cuda.synchronize()
        want = orc.tp_slice(cpu, i_lo, i_hi)
        assert set(k for k, v in want.items() if isinstance(v, torch.Tensor)) == \
            set(k for k, v in s.items() if isinstance(v, torch.Tensor))
        for name, t in want.items():
            if isinstance(t, torch.Tensor):
                assert torch.equal(s[name].cpu(), t), (fmt, name, i_lo, i_hi)


def test_affine_tp_slice_rejects_half_units():
    w = TPW.with_(fmt="affine4")
    d = gpu_inputs(w)
    with pytest.raises(moe.MoeError):
        moe.tp_slice_experts(d["experts"], 64, 192)


@pytest.mark.parametrize("fmt,unit,ranks", [("affine4", 128, 3), ("affine4", 128, 2), ("nvfp4", 64, 5),
                                            ("nvfp4", 128, 3)])
def test_tp_layer_adds_up_to_the_whole_layer(fmt, unit, ranks):
    w = TPW.with_(fmt=fmt)
    d = gpu_inputs(w)
    d["bias"] = (-0.4 * torch.arange(w.E, dtype=torch.float32)).cuda()
    shares = moe.tp_shares(w.I, unit, ranks)
    sshares = moe.tp_shares(w.Is, 64, ranks)
    parts = []
    lo = slo = 0
    for r in range(ranks):
        ex = moe.tp_slice_experts(d["experts"], lo, lo + shares[r])
        sh = moe.tp_slice_shared(d["shared"], slo, slo + sshares[r])
        parts.append(moe.moe_ffn(d["x"], d["router_w"], d["bias"], ex, sh, 0, w.E, w.topk))
        torch.cuda.synchronize()
        lo += shares[r]
        slo += sshares[r]
    y = moe.reduce(parts, "rank")
    torch.cuda.synchronize()
    log(f"{fmt} unit {unit} ranks {ranks}: shares {shares}")
    side = OracleSide(w, d)
    compare(y, side.layer(list(range(w.T)), 0, w.E), f"tp {fmt} {unit}x{ranks}")
