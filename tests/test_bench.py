"""The benchmark's host logic, on the CPU: the one-GPU refusal, the roofline
bookkeeping (algorithmic bytes and flops of the dominant launch, the bound
it picks) and the lookup of the committed HBM byte counters.
"""

import os
import subprocess
import sys

import pytest
import torch

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

W = synth.WORKLOADS
GB = 1e9


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _stages(gu_gemv=0.5, gu_mfma=3.0):
    return {"gu_gemv": gu_gemv, "gu_mfma": gu_mfma}


def test_decode_roofline_counts_the_routed_gemv_bytes_only():
    w = W["decode"]
    counts = torch.zeros(w.E, dtype=torch.int32)
    counts[:60] = 1  # 60 touched experts of one row each
    counts[0] = 4
    r = bench.roofline_for(w, counts, _stages(gu_gemv=0.5), counted=False)
    routed = int(counts.sum())
    # the shared expert's gate/up runs in the top-k/dispatch launch at T <= 8
    wbytes = 60 * 2 * w.I * w.H * 2
    act = routed * w.H * 2 + routed * w.I * 2
    assert r["algorithmic_bytes"] == wbytes + act
    assert r["algorithmic_flops"] == 2.0 * routed * 2 * w.I * w.H
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["kernel"].startswith("gateup_gemv_kernel<0,")
    assert r["achieved"] == pytest.approx((wbytes + act) / 0.5e-3 / GB, rel=1e-3)
    assert r["frac"] == pytest.approx(r["achieved"] / bench.HBM_PEAK_GBS, abs=1e-4)
    assert r["traffic"] is None  # counted=False: not the counters' configuration


def test_prefill_roofline_leaves_the_gemv_groups_out():
    w = W["prefill"]
    counts = torch.full((w.E,), 128, dtype=torch.int32)
    counts[:10] = 4  # ten groups on the GEMV path
    r = bench.roofline_for(w, counts, _stages(gu_mfma=3.0), counted=False)
    routed_m = int(counts.sum()) - 40
    wbytes = 246 * 2 * w.I * w.H * 2 + 2 * w.Is * w.H * 2
    act = (routed_m + w.T) * w.H * 2 + routed_m * w.I * 2 + w.T * w.Is * 2
    assert r["touched_experts"] == 246
    assert r["algorithmic_bytes"] == wbytes + act
    assert "expert_mfma" in r["kernel"]


def test_shared_probe_is_compute_bound():
    w = W["shared_probe"]
    counts = torch.zeros(w.band_hi - w.band_lo, dtype=torch.int32)
    r = bench.roofline_for(w, counts, _stages(gu_mfma=0.165), counted=False)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["algorithmic_flops"] == 2.0 * w.T * 2 * w.Is * w.H
    assert r["achieved"] == pytest.approx(r["algorithmic_flops"] / 0.165e-3 / 1e12, rel=1e-3)


def test_traffic_lookup(tmp_path, monkeypatch):
    h = bench._source_hash(bench.KERNEL_SOURCES["gemv"])
    f = tmp_path / "traffic.txt"
    f.write_text("header line\n"
                 f"traffic decode moe::gateup_gemv_kernel<0,12> 3000 {h}\n"
                 f"traffic decode moe::down_gemv_kernel<0> 1000 {h}\n"
                 "traffic decode moe::old_kernel 5 0123456789abcdef\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("decode", ["moe::gateup_gemv_kernel<0,12>"]) == 3000
    assert bench.measured_traffic("decode", ["moe::gateup_gemv_kernel<0,12>",
                                             "moe::down_gemv_kernel<0>"]) == 4000
    # a kernel without a line, or counters taken on other sources: no traffic
    assert bench.measured_traffic("prefill", ["moe::gateup_gemv_kernel<0,12>"]) is None
    assert bench.measured_traffic("decode", ["moe::old_kernel"]) is None


def test_committed_counters_parse():
    # every machine-readable line of the committed summary is well formed
    n = 0
    with open(bench.TRAFFIC_FILE) as fh:
        for line in fh:
            f = line.split()
            if f and f[0] == "traffic":
                assert len(f) == 5 and f[1] in W and f[2].startswith("moe::")
                assert int(f[3]) > 0 and len(f[4]) == 16
                n += 1
    assert n >= 20


@pytest.mark.parametrize("name", ["decode", "prefill", "shared_probe", "bands", "bands_adversarial",
                                  "w4_t1", "w4_t2048", "affine4_t1", "affine4_t2048", "nvfp4_t1",
                                  "nvfp4_t2048"])
def test_committed_counters_cover_the_reported_launches(name):
    # The default run reports counter traffic for the dominant launches of
    # every workload; the committed counters must name those launches and
    # carry the hash of the current kernel sources.  A renamed kernel, or a
    # kernel source changed without new counter runs, fails here instead of
    # turning the reported traffic into null.
    w = W[name]
    counts = torch.zeros(w.E, dtype=torch.long)
    counts[: w.topk] = w.T  # the launch names do not depend on the routing
    r = bench.roofline_for(w, counts, _stages(), counted=True)
    assert r["traffic"] is not None, f"{name}: no committed counters for {r['kernel']}"
