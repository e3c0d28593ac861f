"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
the same seeded inputs.  Top-k ids and every dispatch array must match bit for
bit; outputs must satisfy max|delta| <= 2e-2 * max|ref| and cosine >= 0.9999.

Pages: [P1] "GLM-5.2 multi-GPU: expert-parallel sharding + the resident-fit
benchmark" (gates table: band of one rank == monolith, sum of bands vs
monolith, all picks on one rank, fail-closed); [P2] "GLM-5.3-Flash on CUDA:
attention on one GPU, routed experts on the Sparks (proposal) #214" (identical
replies run to run); [P5] "GLM-5.3-Flash and full GLM-5.3 on the native CUDA
engine (tracker) #593" (the swiglu stride bug: fused rows are 2w wide).
"""

import pytest
import torch

import synth
from gpu_common import OracleSide, check_routing, compare, gpu_inputs, log, run_gpu, sample_rows

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS

# Workloads small enough for the oracle on every row, spanning several tiles
# and ragged tails on both expert paths (group sizes from 0 to > 2 MFMA row
# tiles thanks to a falling bias), with odd sizes: H not a multiple of 512,
# I not a multiple of 128, E not a multiple of 64.
MID = synth.Workload("mid", T=300, H=512, E=16, topk=4, I=192, Is=128)
WIDE = synth.Workload("wide", T=70, H=1280, E=40, topk=6, I=320, Is=192)


def _falling_bias(d, E, step):
    d["bias"] = (-step * torch.arange(E, dtype=torch.float32)).cuda()
    return d


@pytest.mark.parametrize("fmt", ["bf16", "w4"])
@pytest.mark.parametrize("wname", ["tiny", "mid", "wide"])
def test_small_workloads_every_row(wname, fmt):
    w = {"tiny": W["tiny"], "mid": MID, "wide": WIDE}[wname].with_(fmt=fmt)
    log(f"case {w}")
    d = gpu_inputs(w)
    if wname == "mid":
        _falling_bias(d, w.E, 0.5)
    if wname == "wide":
        _falling_bias(d, w.E, 0.15)
    side = OracleSide(w, d)
    y, ex = run_gpu(w, d)
    check_routing(ex, side, 0, w.E)
    counts = ex["counts"].cpu()
    log(f"group sizes {sorted(counts.tolist(), reverse=True)}")
    compare(y, side.layer(list(range(w.T)), 0, w.E), f"{wname}/{fmt}")


def test_tiny_every_band():
    w = W["tiny"]
    d = gpu_inputs(w)
    side = OracleSide(w, d)
    for lo in range(w.E):
        for hi in range(lo + 1, w.E + 1):
            for shared in (True, False):
                y, ex = run_gpu(w, d, lo, hi, shared=shared)
                check_routing(ex, side, lo, hi)
                ref = side.layer(list(range(w.T)), lo, hi, shared=shared)
                if float(ref.abs().max()) == 0:
                    assert float(y.abs().max()) == 0
                else:
                    compare(y, ref, f"tiny band [{lo},{hi}) shared={shared}")


def test_mid_bands_sum_and_determinism():
    w = MID
    d = _falling_bias(gpu_inputs(w), w.E, 0.5)
    full, _ = run_gpu(w, d)
    again, _ = run_gpu(w, d)
    assert torch.equal(full, again), "run-to-run bits differ"
    cuts = [0, 1, 3, 4, 9, 16]
    acc = None
    for b, (lo, hi) in enumerate(zip(cuts[:-1], cuts[1:])):
        p, _ = run_gpu(w, d, lo, hi, shared=(b == 0))
        acc = p.clone() if acc is None else acc + p
    # reassociation only: (k + 2) fp32 roundings of terms bounded by max|out|
    scale = float(full.abs().max())
    assert float((acc - full).abs().max()) <= (w.topk + 2) * 2.0 ** -23 * 4 * scale


def test_decode_full_size():
    w = W["decode"]
    log(f"case {w}")
    d = gpu_inputs(w)
    side = OracleSide(w, d)
    y, ex = run_gpu(w, d)
    check_routing(ex, side, 0, w.E)
    log(f"distinct experts touched {int((ex['counts'] > 0).sum())}")
    compare(y, side.layer(list(range(w.T)), 0, w.E), "decode")
    y2, _ = run_gpu(w, d)
    assert torch.equal(y, y2)


@pytest.fixture(scope="module")
def decode_wide_batch():
    # decode-sized experts with 65 rows of input; the cases below take the
    # first T rows
    w = W["decode"].with_(T=65)
    return w, gpu_inputs(w)


@pytest.mark.parametrize("T", [1, 2, 3, 5, 8, 9, 64, 65])
def test_router_launch_shapes_full_width(decode_wide_batch, T):
    """Each router launch shape (one or two rows per wave with every step's
    loads in flight, eight rows per wave, 8 x 8 tiles) at the full width
    H = 6144, E = 256: ids and the dispatch bit-exact, weights to fp32."""
    w0, d0 = decode_wide_batch
    w = w0.with_(T=T)
    d = dict(d0, x=d0["x"][:T].contiguous())
    log(f"case T={T}")
    side = OracleSide(w, d)
    y, ex = run_gpu(w, d)
    check_routing(ex, side, 0, w.E)
    if T <= 3:
        compare(y, side.layer(list(range(T)), 0, w.E), f"T={T}")


def test_prefill_full_size_sampled():
    w = W["prefill"]
    log(f"case {w}")
    d = gpu_inputs(w)
    side = OracleSide(w, d)
    y, ex = run_gpu(w, d)
    check_routing(ex, side, 0, w.E)
    c = ex["counts"].cpu()
    log(f"groups > 8 rows: {int((c > 8).sum())}, largest {int(c.max())}, smallest {int(c.min())}")
    rows = sample_rows(w.T, 10, seed=3)
    compare(y[rows], side.layer(rows, 0, w.E), "prefill sampled rows")
    y2, _ = run_gpu(w, d)
    assert torch.equal(y, y2)


def test_shared_probe_full_size_sampled():
    """The compute-bound probe: every pick outside the band [8, 256), so the
    layer is the shared expert's 4096 rows alone (one 256-row group per
    column tile on every CU)."""
    w = W["shared_probe"]
    log(f"case {w}")
    d = gpu_inputs(w)
    side = OracleSide(w, d)
    y, ex = run_gpu(w, d)
    check_routing(ex, side, w.band_lo, w.band_hi)
    assert int(ex["counts"][: w.band_hi - w.band_lo].sum()) == 0
    rows = sample_rows(w.T, 10, seed=4)
    compare(y[rows], side.layer(rows, w.band_lo, w.band_hi), "shared probe sampled rows")


def test_bands_full_size():
    w = W["bands"]
    log(f"case {w}")
    d = gpu_inputs(w)
    side = OracleSide(w, d)
    full, ex = run_gpu(w, d)
    check_routing(ex, side, 0, w.E)
    acc = None
    for b, (lo, hi) in enumerate(synth.bands(w)):
        p, exb = run_gpu(w, d, lo, hi, shared=(b == 0))
        check_routing(exb, side, lo, hi)
        acc = p.clone() if acc is None else acc + p
    scale = float(full.abs().max())
    drift = float((acc - full).abs().max())
    log(f"bands: max|sum - full| = {drift:.3g} (max|full| {scale:.3g})")
    assert drift <= (w.topk + 2) * 2.0 ** -23 * 4 * scale
    rows = sample_rows(w.T, 6, seed=4)
    compare(full[rows], side.layer(rows, 0, w.E), "bands full-band sampled rows")


def test_bands_adversarial_exact():
    # All picks land in band [0, 32): the other bands add exact zeros and band
    # 0 computes the same groups as the full band -> max|delta| = 0.
    w = W["bands_adversarial"]
    d = gpu_inputs(w)
    full, ex = run_gpu(w, d)
    assert int(ex["counts"][32:].sum()) == 0
    acc = None
    for b, (lo, hi) in enumerate(synth.bands(w)):
        p, _ = run_gpu(w, d, lo, hi, shared=(b == 0))
        if b > 0:
            assert float(p.abs().max()) == 0.0
        acc = p.clone() if acc is None else acc + p
    assert float((acc - full).abs().max()) == 0.0
    side = OracleSide(w, d)
    check_routing(ex, side, 0, w.E)
    rows = sample_rows(w.T, 4, seed=5)
    compare(full[rows], side.layer(rows, 0, w.E), "adversarial sampled rows")


@pytest.mark.parametrize("wname,nrows", [("w4_t1", 1), ("w4_t2048", 6)])
def test_w4_full_size(wname, nrows):
    w = W[wname]
    log(f"case {w}")
    d = gpu_inputs(w)
    side = OracleSide(w, d)
    y, ex = run_gpu(w, d)
    check_routing(ex, side, 0, w.E)
    rows = sample_rows(w.T, nrows, seed=6)
    compare(y[rows], side.layer(rows, 0, w.E), wname)


@pytest.mark.parametrize("topk", [1, 8])
def test_all_picks_on_one_expert_set(topk):
    # +10 on the first topk experts: every row picks exactly those, so each
    # group holds all T rows (one group of T rows when topk = 1).
    w = MID.with_(topk=topk, E=16, bias="one_expert")
    d = gpu_inputs(w)
    d["bias"] = synth.make_bias(w).cuda()
    side = OracleSide(w, d)
    y, ex = run_gpu(w, d)
    check_routing(ex, side, 0, w.E)
    assert ex["counts"].cpu().tolist()[:topk] == [w.T] * topk
    compare(y, side.layer(list(range(w.T)), 0, w.E), f"one-expert topk={topk}")


def test_zero_router_uniform_weights():
    # Zero router weights: every logit is +0, so ids are 0..k-1 and every
    # weight is exactly 1/k.
    w = MID.with_(topk=4)
    d = gpu_inputs(w)
    d["router_w"] = torch.zeros_like(d["router_w"])
    y, ex = run_gpu(w, d)
    assert (ex["topk_ids"].cpu() == torch.arange(4, dtype=torch.int32)).all()
    assert (ex["topk_w"].cpu() == 0.25).all()


def test_negative_zero_logits():
    # Products that underflow to -0.0 give -0.0 partial sums; logits are +0.0,
    # so the tie-break picks 0..k-1 as in the oracle.
    w = W["tiny"]
    d = gpu_inputs(w)
    d["x"] = torch.full_like(d["x"], -1e-30)
    d["router_w"] = torch.full_like(d["router_w"], 1e-30)
    side = OracleSide(w, d)
    y, ex = run_gpu(w, d)
    check_routing(ex, side, 0, w.E)


@pytest.mark.parametrize("fmt", ["bf16", "w4"])
def test_gate_up_stride_regression(fmt):
    # The fused gate/up rows of an expert are 2I wide (gate rows first).  Zero
    # gate rows give silu(0) * up = 0, so the routed part vanishes and the
    # output is the shared expert alone; reading the up rows, or another
    # expert's rows, at a stride of I would make it nonzero.
    w = MID.with_(fmt=fmt)
    d = gpu_inputs(w)
    ex_ = d["experts"]
    if fmt == "bf16":
        ex_["w_gate_up"][:, : w.I, :] = 0
    else:
        # codes equal to an integer zero point: gate weights exactly 0
        ex_["q_gate_up"][:, : w.I, :] = 0x88
        ex_["z_gate_up"][:, : w.I, :] = 8.0
    y, _ = run_gpu(w, d)
    side = OracleSide(w, d)
    compare(y, side.layer(list(range(w.T)), 0, w.E), f"stride regression {fmt}")
    # and the routed part alone is exactly zero
    y_routed, _ = run_gpu(w, d, shared=False)
    assert float(y_routed.abs().max()) == 0.0


def test_empty_band_gives_zero_or_shared():
    w = W["bands_adversarial"].with_(T=64)
    d = gpu_inputs(w)
    y, ex = run_gpu(w, d, 64, 96, shared=False)
    assert int(ex["offsets"][-1]) == 0
    assert float(y.abs().max()) == 0.0
    assert (ex["pos"].cpu() == -1).all()


@pytest.mark.parametrize("fmt", ["bf16", "w4"])
@pytest.mark.parametrize("H,Is", [(1024, 192), (1024, 640), (3584, 640), (4096, 640)])
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 6, 7, 8])
def test_shared_gateup_beside_the_dispatch(T, H, Is, fmt):
    # With at most 8 rows and H a multiple of 512 the shared expert's gate/up
    # runs in the blocks of the top-k/dispatch launch beyond the first, one
    # row-count specialisation per T; Is = 192 leaves most blocks one column
    # pair, Is = 640 gives some waves two.  H = 3584 and 4096 stage the rows
    # in more than one load block (4096: whole blocks; 3584: a partial last
    # one).  Whole layer against the oracle.
    w = synth.Workload("sh_fused", T=T, H=H, E=32, topk=4, I=128, Is=Is, fmt=fmt)
    log(f"case {w}")
    d = gpu_inputs(w)
    side = OracleSide(w, d)
    y, ex = run_gpu(w, d)
    check_routing(ex, side, 0, w.E)
    compare(y, side.layer(list(range(w.T)), 0, w.E), f"shared beside the dispatch T={T} H={H} Is={Is}/{fmt}")


@pytest.mark.parametrize("fmt", ["bf16", "w4"])
@pytest.mark.parametrize("T", [16, 17])
def test_small_batch_topk_dispatch_boundary(T, fmt):
    # Up to 16 rows the top-k and the dispatch run in one block, with the
    # picks of every row (up to 16 x 16) kept in LDS; 17 rows take the
    # separate kernels.  topk = 16 fills that buffer.
    w = synth.Workload("boundary", T=T, H=256, E=64, topk=16, I=128, Is=64, fmt=fmt)
    log(f"case {w}")
    d = gpu_inputs(w)
    side = OracleSide(w, d)
    y, ex = run_gpu(w, d)
    check_routing(ex, side, 0, w.E)
    compare(y, side.layer(list(range(w.T)), 0, w.E), f"boundary T={T}/{fmt}")
    # a band in the middle: picks outside it are marked -1 in pos
    y, ex = run_gpu(w, d, 16, 40, shared=False)
    check_routing(ex, side, 16, 40)
    compare(y, side.layer(list(range(w.T)), 16, 40, shared=False), f"boundary T={T}/{fmt} band")
