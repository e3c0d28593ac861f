"""GPU: the 4-bit MFMA launch with wide column tiles, every row against the
oracle.

Routed 4-bit experts whose K is a multiple of 512 and whose widths are whole
tiles (I % 128 == 0 for gate/up, H % 256 == 0 for down) run every group of
more than 8 rows in one launch of items 256 weight rows wide: first the items
of up to 128 rows (groups of more than 64), then those of up to 64 (9..64
rows) ([P5] "GLM-5.3-Flash and full GLM-5.3
on the native CUDA engine (tracker) #593", "The pieces, in order": quantised
expert checkpoints dequantised in the kernels; the W4A16 workload's
(q - z) * s per 32 inputs, MLX affine's s * q + b per 64, NVFP4's e2m1 *
e4m3 per 16 times a matrix scale).  A falling router bias spreads the group
sizes over every tile list: groups of more than 256 rows, 129..256, 65..128,
33..64, 9..32 and the GEMV path's <= 8.
"""

import pytest
import torch

import synth
from gpu_common import OracleSide, check_routing, compare, gpu_inputs, log, run_gpu

pytestmark = pytest.mark.gpu

FORMATS = ["w4", "affine4", "nvfp4"]
WIDE4 = synth.Workload("wide4", T=600, H=1024, E=16, topk=4, I=512, Is=256)


@pytest.mark.parametrize("fmt", FORMATS)
def test_every_row_all_tile_lists(fmt):
    w = WIDE4.with_(fmt=fmt)
    log(f"case {w}")
    d = gpu_inputs(w)
    d["bias"] = (-0.4 * torch.arange(w.E, dtype=torch.float32)).cuda()
    y, ex = run_gpu(w, d)
    counts = sorted(ex["counts"].cpu().tolist(), reverse=True)
    log(f"group sizes {counts}")
    assert counts[0] > 256 and any(64 < c <= 128 for c in counts) and any(8 < c <= 32 for c in counts)
    side = OracleSide(w, d)
    check_routing(ex, side, 0, w.E)
    compare(y, side.layer(list(range(w.T)), 0, w.E), f"wide tiles {fmt}")
    y2, _ = run_gpu(w, d)
    assert torch.equal(y, y2), "run-to-run bits differ"


@pytest.mark.parametrize("fmt", FORMATS)
def test_band_and_no_shared(fmt):
    # a band that cuts the largest groups off, no shared expert: only routed
    # 4-bit groups reach the launch
    w = WIDE4.with_(fmt=fmt, T=300)
    d = gpu_inputs(w)
    d["bias"] = (-0.4 * torch.arange(w.E, dtype=torch.float32)).cuda()
    y, ex = run_gpu(w, d, 2, 13, shared=False)
    side = OracleSide(w, d)
    check_routing(ex, side, 2, 13)
    compare(y, side.layer(list(range(w.T)), 2, 13, shared=False), f"wide tiles band {fmt}")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("T", [20, 40, 100, 200])
def test_one_tile_list_alone(fmt, T):
    # A zero router (every logit +0.0, ties to the lower id) sends every row
    # to experts 0..3: four groups of T rows, so only one tile list of the
    # launch has items (T = 20: 9..32 rows, 40: 33..64, 100: 65..128, 200:
    # two 128-row items per group), and the other list is empty.
    w = WIDE4.with_(fmt=fmt, T=T)
    log(f"case {w}")
    d = gpu_inputs(w)
    d["router_w"].zero_()
    d["bias"] = torch.zeros(w.E, dtype=torch.float32, device="cuda")
    y, ex = run_gpu(w, d)
    assert sorted(ex["counts"].cpu().tolist(), reverse=True)[:5] == [T, T, T, T, 0]
    side = OracleSide(w, d)
    check_routing(ex, side, 0, w.E)
    compare(y, side.layer(list(range(w.T)), 0, w.E), f"one tile list {fmt} T={T}")
