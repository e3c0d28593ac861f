"""Benchmark of one routed MoE FFN layer on one MI355X.

A step is one call of the whole layer (router, top-k, dispatch, gate/up +
SwiGLU, down, combine + shared expert) over one batch of synthetic rows whose
inputs and weights are already resident in HBM.  Before every step a 1 GiB
scratch read evicts the L2 and the MALL (256 MB), so every step reads its
weights from HBM; the layer's own time per step is measured with HIP events on
the launch stream (the eviction is outside them).  A read leaves the caches
clean, as the weight reads of a model's other layers would; a 1 GiB write
(--flush write) instead leaves them full of dirty lines whose write-back lands
in the next kernel's time (about 10% of a decode-sized layer).

Prints one JSON line: rows/s, us per layer, the dominant kernel's roofline
fraction (measured live with the same events) and the oracle timed on the
host cores on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE FFN rows/s + µs/layer; decode % HBM roofline, prefill % bf16 MFMA peak"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


class Hip:
    """hipEvent helpers through ctypes (events recorded by the library)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def events(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.lib.hipEventSynchronize(ctypes.c_void_p(b)) == 0
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return float(ms.value)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_moe_kernels_all_workloads.txt")
KERNEL_SOURCES = {
    "gemv": ["mixture_experts_ffn_06_amd/csrc/gemv.hip", "mixture_experts_ffn_06_amd/csrc/common.h"],
    "pipe": ["mixture_experts_ffn_06_amd/csrc/mfma_pipe.hip", "mixture_experts_ffn_06_amd/csrc/common.h"],
}


def _source_hash(files):
    import hashlib

    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernels):
    """HBM bytes per launch of `kernels` (summed) from the committed counter
    summary: FETCH_SIZE and WRITE_SIZE, each scaled by what it reads for a plain
    copy of known size.  None when a kernel has no line for this workload or
    its sources changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    table = {}
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            f = line.split()
            if len(f) == 5 and f[0] == "traffic":
                table[(f[1], f[2])] = (int(f[3]), f[4])
    total = 0
    for k in kernels:
        hit = table.get((workload, k))
        if hit is None:
            return None
        fam = "gemv" if "gemv" in k else "pipe"
        if hit[1] != _source_hash(KERNEL_SOURCES[fam]):
            return None
        total += hit[0]
    return total


# the library's format codes, and the dtype label of each format's path
# (bf16 activations, weights decoded from the stored form)
FMT_CODE = {"bf16": 0, "w4": 1, "affine4": 2, "nvfp4": 3}
FMT_DTYPE = {"bf16": "bf16", "w4": "w4a16", "affine4": "affine4a16", "nvfp4": "nvfp4a16"}


def _expert_gu_bytes(w):
    """Stored bytes of one expert's fused gate/up matrix (2I rows of H inputs)."""
    rows = 2 * w.I
    if w.fmt == "bf16":
        return rows * w.H * 2
    codes = rows * (w.H // 2)
    if w.fmt == "w4":
        return codes + rows * (w.H // 32) * 2 * 2  # bf16 scale and zero per 32 inputs
    if w.fmt == "affine4":
        return codes + rows * (w.H // 64) * 2 * 2  # bf16 scale and bias per 64 inputs
    return codes + rows * (w.H // 16) + 2 * 4  # E4M3 scale per 16 inputs, two fp32 matrix scales


def roofline_for(w, counts, stage_ms, counted=True):
    """Dominant kernel and its algorithmic bytes and flops per launch.

    The gate/up projection dominates every workload.  Its algorithmic bytes:
    each touched expert's fused gate/up weights once (2*I*H bf16 values, or
    4-bit codes plus a bf16 scale and zero per 32 inputs), the shared
    expert's, the routed and shared rows of x it reads and the bf16
    intermediate it writes.  Its flops: 2*(2I)*H per routed row and
    2*(2Is)*H per shared row.  Decode-sized batches (every group on the GEMV
    path) take the GEMV launch, without the shared expert when the top-k /
    dispatch launch computes its gate/up (T <= 8, H a multiple of 512, its
    rows within 128 KiB); larger ones the MFMA launches (one per tile
    height), whose time is summed.  The bound is whichever of HBM bytes at
    8 TB/s and flops at the bf16 dense MFMA peak takes longer; the MFMA
    fraction is reported beside it for every workload.  counted: the committed
    counters were taken on this configuration (not with another routing or a
    tensor-parallel slice), so their traffic applies."""
    n_touched = int((counts > 0).sum())
    routed = int(counts.sum())
    sh_rows = w.T if w.Is else 0
    wbytes = n_touched * _expert_gu_bytes(w) + (2 * w.Is * w.H * 2 if w.Is else 0)
    act = (routed + sh_rows) * w.H * 2 + routed * w.I * 2 + sh_rows * w.Is * 2
    nbytes = wbytes + act
    flops = 2.0 * routed * 2 * w.I * w.H + 2.0 * sh_rows * 2 * w.Is * w.H
    if w.T <= 8:
        # (one-row 4-bit calls take the one-row kernel, whose bf16 path loads 4
        # lane steps at a time; H = 6144 otherwise takes 12)
        one = w.T == 1 and w.fmt != "bf16"
        cb = min(4 if one else 12, max(4, -(-((w.H + 511) // 512) // 4) * 4))
        kernel = f"gateup_gemv_kernel<{FMT_CODE[w.fmt]},{cb},{1 if one else 8}>"
        ms = stage_ms["gu_gemv"]
        traffic = measured_traffic(w.name, [f"moe::{kernel}"])
        if w.Is and w.H % 512 == 0 and w.T * w.H * 2 <= 128 * 1024:
            # the shared expert's gate/up ran in the top-k/dispatch launch
            wbytes = n_touched * _expert_gu_bytes(w)
            act = routed * w.H * 2 + routed * w.I * 2
            nbytes = wbytes + act
            flops = 2.0 * routed * 2 * w.I * w.H
    else:
        # 4-bit: the wide-tile launch (groups of more than 64 rows, then of
        # 9..64) when H % 512 == 0 and I % 128 == 0, else the 128-, 64- and
        # 32-row launches
        wide = w.H % 512 == 0 and w.I % 128 == 0
        fc = FMT_CODE[w.fmt]
        w4_names = ([f"expert_mfma_w4w_kernel<{fc},true>"] if wide
                    else [f"expert_mfma_w4_kernel<{fc},true,{bm}>" for bm in (128, 64, 32)])
        kernel = ("expert_mfma_pipe_kernel<true,256> + expert_mfma_small_kernel<true>" if w.fmt == "bf16"
                  else " + ".join(w4_names) + " + shared-expert bf16 launch")
        ms = stage_ms["gu_mfma"]
        if w.fmt == "bf16":
            traffic = measured_traffic(
                w.name, ["moe::expert_mfma_pipe_kernel<true,256>", "moe::expert_mfma_small_kernel<true>"])
        else:
            # the 4-bit launches, plus the one bf16 launch that holds the shared
            # expert's rows (256-row tiles above 128 rows, else the small-tile launch)
            sh = "expert_mfma_pipe_kernel<true,256>" if w.T > 128 else "expert_mfma_small_kernel<true>"
            traffic = measured_traffic(w.name, [f"moe::{k}" for k in w4_names] + [f"moe::{sh}"])
        # rows on the GEMV path (groups of 1..8 rows) are not in this launch
        small = counts[(counts > 0) & (counts <= 8)]
        n_touched -= int(small.numel())
        routed_m = routed - int(small.sum())
        wbytes = n_touched * _expert_gu_bytes(w) + (2 * w.Is * w.H * 2 if w.Is else 0)
        act = (routed_m + sh_rows) * w.H * 2 + routed_m * w.I * 2 + sh_rows * w.Is * 2
        nbytes = wbytes + act
        flops = 2.0 * routed_m * 2 * w.I * w.H + 2.0 * sh_rows * 2 * w.Is * w.H
    if not counted:
        traffic = None
    sec = ms * 1e-3
    gbs = nbytes / sec / 1e9
    tfs = flops / sec / 1e12
    t_bytes = nbytes / (HBM_PEAK_GBS * 1e9)
    t_flops = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    mfma = {"achieved": round(tfs, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tfs / MFMA_BF16_PEAK_TFLOPS, 4)}
    if t_bytes >= t_flops:
        out = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        out = {"bound": "mfma", **mfma}
    out.update({"traffic": traffic, "kernel": kernel, "kernel_us": round(ms * 1e3, 2),
                "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
                "touched_experts": n_touched, "mfma": mfma,
                "floor_us": round(max(t_bytes, t_flops) * 1e6, 2)})
    return out


def cpu_baseline(w, d, ex, rows_budget, min_seconds=10.0, modes=None):
    """The oracle, as it stands, on a bounded sample of rows of the workload."""
    import torch

    from oracle import oracle as orc

    rows = list(range(min(w.T, rows_budget)))
    need = sorted({int(e) for e in ex["topk_ids"][: len(rows)].flatten().tolist()})
    experts = {"fmt": d["experts"]["fmt"]}
    for name, t in d["experts"].items():
        if isinstance(t, torch.Tensor):
            experts[name] = torch.empty(t.shape, dtype=t.dtype)
            for e in need:
                experts[name][e].copy_(t[e])
    inputs = {"x": d["x"].cpu(), "router_w": d["router_w"].cpu(),
              "bias": None if d["bias"] is None else d["bias"].cpu(), "experts": experts,
              "shared": None if d["shared"] is None else {k: v.cpu() for k, v in d["shared"].items()}}
    ex_o = orc.Experts(experts, w.E, w.H, w.I)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    rows_t = torch.tensor(rows, dtype=torch.int32)
    # the sample is run again until about min_seconds of host time are spent
    reps, t0 = 0, time.perf_counter()
    while True:
        orc.moe_ffn(inputs, w.E, w.I, w.Is, w.band_lo, w.band_hi, w.topk, rows=rows_t, experts=ex_o,
                    **(modes or {}))
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    # the oracle's widest step runs one expert FFN per (row, in-band pick)
    # and per (row, shared expert), spread over the OpenMP threads
    ids = ex["topk_ids"][: len(rows)].cpu()
    tasks = int(((ids >= w.band_lo) & (ids < w.band_hi)).sum()) + (len(rows) if w.Is else 0)
    return {"value": round(reps * len(rows) / dt, 3), "unit": "rows/s", "cores": min(threads, tasks),
            "threads_available": threads, "os_cpu_count": os.cpu_count(), "cpu_model": cpu_model,
            "kind": "oracle",
            "sample": f"rows 0..{len(rows) - 1} of the {w.name} workload, run {reps} times "
                      f"(fp64 oracle: routing per row, then {tasks} expert FFNs, one per "
                      f"(row, pick) and per (row, shared expert), OpenMP over them), {dt:.2f} s"}


def layer_work(w, counts):
    """Algorithmic HBM bytes and flops of one whole layer call: each touched
    in-band expert's weights once, the shared expert's, the router weight
    (and bias), the rows read and the fp32 output written; flops 2*3*H*I per
    in-band pick and 2*3*H*Is per shared row (the fp32 router's 2*T*E*H
    apart)."""
    from synth import expert_bytes, shared_bytes

    n_touched = int((counts > 0).sum())
    routed = int(counts.sum())
    nbytes = (n_touched * expert_bytes(w) + shared_bytes(w) + w.E * w.H * 4 + w.T * w.H * 2 +
              w.T * w.H * 4)
    flops = 6.0 * w.H * w.I * routed + (6.0 * w.H * w.Is * w.T if w.Is else 0.0)
    return nbytes, flops


def layer_roofline(w, counts, ms):
    nbytes, flops = layer_work(w, counts)
    sec = ms * 1e-3
    t_floor = max(nbytes / (HBM_PEAK_GBS * 1e9), flops / (MFMA_BF16_PEAK_TFLOPS * 1e12))
    return {"algorithmic_bytes": nbytes, "algorithmic_flops": flops,
            "GB_per_s": round(nbytes / sec / 1e9, 1), "hbm_frac": round(nbytes / sec / 1e9 / HBM_PEAK_GBS, 4),
            "TFLOP_per_s": round(flops / sec / 1e12, 1),
            "mfma_frac": round(flops / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "floor_us": round(t_floor * 1e6, 2), "frac_of_floor": round(t_floor / sec, 4)}


class Runner:
    """Times whole-layer calls of one workload on the current stream: an
    eviction read before every call, HIP events on the launch stream around
    the call itself, and a separate set of calls with the library's stage
    events for the per-stage breakdown."""

    def __init__(self, args, hip, flush):
        self.args, self.hip, self.flush = args, hip, flush

    def evict(self):
        import torch  # noqa: F401

        if self.args.flush == "read":
            self.flush.sum()  # reads 1 GiB, writes one scalar
        elif self.args.flush == "write":
            self.flush.fill_(1)

    def run(self, w, d, opts, steps, warmup, band=None, ws=None, out=None, exports=True):
        import torch

        import mixture_experts_ffn_06_amd as moe

        lo, hi = band if band is not None else (w.band_lo, w.band_hi)
        dev = d["x"].device
        stream = torch.cuda.current_stream(dev)
        if out is None:
            out = torch.empty((w.T, w.H), dtype=torch.float32, device=dev)
        if ws is None:
            ws = torch.empty((moe.workspace_bytes(w.T, w.H, w.E, w.I, w.Is, w.topk,
                                                  FMT_CODE[w.fmt]),),
                             dtype=torch.uint8, device=dev)
        ex = {} if exports else None

        def call(**kw):
            moe.moe_ffn(d["x"], d["router_w"], d["bias"], d["experts"], d["shared"], lo, hi, w.topk,
                        out=out, workspace=ws, **opts, **kw)

        self.evict()
        call(exports=ex)  # also exports the routing, for the roofline bookkeeping
        for _ in range(warmup):
            self.evict()
            call()
        torch.cuda.synchronize()
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            self.evict()
            starts[i].record(stream)
            call()
            ends[i].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        layer_ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
        nstage = min(steps, 10)
        ev = [self.hip.events(moe.MOE_NUM_EVENTS) for _ in range(nstage)]
        for i in range(nstage):
            self.evict()
            call(events=ev[i])
        torch.cuda.synchronize()
        names = moe.EVENT_SLOTS
        stage = {n: 0.0 for n in names[:-1]}
        for i in range(nstage):
            for s_ in range(len(names) - 1):
                stage[names[s_]] += self.hip.elapsed_ms(ev[i][s_], ev[i][s_ + 1]) / nstage
        return {"ms": sum(layer_ms) / len(layer_ms), "ms_min": min(layer_ms), "wall": wall,
                "stage": stage, "ex": ex, "out": out, "ws": ws}


def summary(w, r, counted=True):
    """The compact per-workload object: time, rows/s, the whole layer against
    its roofline, and the gate/up launches (the dominant kernel)."""
    counts = r["ex"]["counts"].cpu()
    roof = roofline_for(w, counts, r["stage"], counted=counted)
    return {"us_per_layer": round(r["ms"] * 1e3, 2), "rows_per_s": round(w.T / (r["ms"] * 1e-3), 1),
            "config": {"T": w.T, "H": w.H, "E": w.E, "topk": w.topk, "I": w.I, "Is": w.Is,
                       "fmt": w.fmt, "band": [w.band_lo, w.band_hi], "bias": w.bias},
            "stage_us": {k: round(v * 1e3, 2) for k, v in r["stage"].items()},
            "layer": layer_roofline(w, counts, r["ms"]),
            "gate_up": {k: roof[k] for k in ("kernel", "kernel_us", "bound", "achieved", "unit", "frac",
                                             "traffic", "algorithmic_bytes", "algorithmic_flops")}
            | {"mfma_frac": roof["mfma"]["frac"]}}


def extra_workloads(runner, d_bf16, dev, args):
    """Every other workload of the set at its full size, timed in the same
    process after the headline: prefill (its own object), the expert bands
    (one after another, then the exchange step), the adversarial band case,
    the compute-bound shared-expert probe, and the 4-bit experts at 1 and
    2048 rows.  The bf16 workloads share the decode workload's experts (same
    seeds and shapes); the 4-bit ones are drawn after those are freed."""
    import torch

    import mixture_experts_ffn_06_amd as moe
    import synth

    W = synth.WORKLOADS
    steps, warmup = max(3, args.steps // 2), 2
    res = {}

    def inputs(w):
        base = W["decode"]
        assert (w.E, w.H, w.I, w.Is, w.fmt, w.seed) == (base.E, base.H, base.I, base.Is, base.fmt, base.seed)
        d = synth.make_router(w, dev)
        d["experts"], d["shared"] = d_bf16["experts"], d_bf16["shared"]
        return d

    # prefill, the probe
    for name in ("prefill", "shared_probe"):
        w = W[name]
        print(f"bench: {name}", file=sys.stderr, flush=True)
        r = runner.run(w, inputs(w), {}, steps, warmup)
        res[name] = summary(w, r)
        del r
        torch.cuda.empty_cache()

    # bands: the full band, then the 8 bands one after another and their sum
    for name in ("bands", "bands_adversarial"):
        w = W[name]
        print(f"bench: {name}", file=sys.stderr, flush=True)
        d = inputs(w)
        r = runner.run(w, d, {}, steps, warmup)
        o = summary(w, r)
        per_band = []
        parts = []
        for b, (lo, hi) in enumerate(synth.bands(w)):
            dd = dict(d)
            if b > 0:
                dd["shared"] = None  # the shared expert is band 0's
            rb = runner.run(w, dd, {}, steps, warmup, band=(lo, hi), ws=r["ws"], exports=False)
            per_band.append(round(rb["ms"] * 1e3, 2))
            parts.append(rb["out"])
        # the exchange step on one GPU: the 8 partials added in rank order
        red_ms = []
        for i in range(steps + 2):
            runner.evict()
            a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            moe.reduce(parts, "rank")
            b_.record()
            torch.cuda.synchronize()
            if i >= 2:
                red_ms.append(a.elapsed_time(b_))
        o["band_us"] = per_band
        o["bands_sum_us"] = round(sum(per_band), 2)
        o["reduce_rank_order_us"] = round(sum(red_ms) / len(red_ms) * 1e3, 2)
        res[name] = o
        del r, parts, d
        torch.cuda.empty_cache()

    # 4-bit experts, one format at a time (the bf16 ones are freed first)
    d_bf16.clear()
    torch.cuda.empty_cache()
    for fam in ("w4", "affine4", "nvfp4"):
        w4 = None
        for name in (f"{fam}_t1", f"{fam}_t2048"):
            w = W[name]
            print(f"bench: {name}", file=sys.stderr, flush=True)
            d = synth.make_router(w, dev)
            if w4 is None:
                w4 = {"experts": synth.make_experts(w, dev), "shared": synth.make_shared(w, dev)}
            d.update(w4)
            r = runner.run(w, d, {}, steps if w.T > 1 else args.steps, warmup)
            res[name] = summary(w, r)
            del r, d
            torch.cuda.empty_cache()
        del w4
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode")
    ap.add_argument("--flush", choices=["read", "write", "none"], default="read",
                    help="how L2 and MALL are evicted before each step (1 GiB scratch read or write)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="time only --workload (by default the decode headline is followed by "
                         "every other workload at full size, each in an object of the same line)")
    ap.add_argument("--cpu-rows", type=int, default=8)
    ap.add_argument("--combine", choices=["pick", "tree"], default="pick",
                    help="order of the routed sum: pick order or the canonical tree over expert ids")
    ap.add_argument("--reduce-parts", type=int, default=0, metavar="N",
                    help="also time moe_ffn_reduce adding N band partials of the output along "
                         "the tree (N a power of two dividing E)")
    ap.add_argument("--router", choices=["softmax", "sigmoid"], default="softmax",
                    help="softmax router (bias on the logits) or sigmoid + selection bias")
    ap.add_argument("--norm", action="store_true",
                    help="RMSNorm the rows before routing (weight ~ 1 + N(0, 0.05), eps 1e-5) "
                         "and add the raw rows after the combine")
    ap.add_argument("--tp", type=int, default=1, metavar="N",
                    help="time one tensor-parallel rank's share: the experts' intermediate "
                         "columns split over N ranks (whole units, remainder on the lowest ranks)")
    ap.add_argument("--tp-rank", type=int, default=0)
    ap.add_argument("--tp-unit", type=int, default=64)
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the layer captured once in a HIP graph (the eviction "
                         "stays outside the graph) instead of eager calls")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain elementwise copy of MIB MiB five times (a known byte "
                         "count for calibrating HBM byte counters), then exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(the layer's expert bands are run one after another on one GPU).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.ones((n,), dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)  # reads and writes n*4 bytes
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4,
                          "launches": 5}), flush=True)
        return

    import mixture_experts_ffn_06_amd as moe
    import synth

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_gen = time.perf_counter()
    d = synth.make_inputs(w, dev)
    tp_info = None
    if args.tp > 1:
        # this rank's slice of every expert (and of the shared expert), laid
        # out by the library; the layer then runs at the rank's real shape
        shares = moe.tp_shares(w.I, args.tp_unit, args.tp)
        sshares = moe.tp_shares(w.Is, args.tp_unit, args.tp)
        r = args.tp_rank
        lo, slo = sum(shares[:r]), sum(sshares[:r])
        d["experts"] = moe.tp_slice_experts(d["experts"], lo, lo + shares[r])
        d["shared"] = moe.tp_slice_shared(d["shared"], slo, slo + sshares[r])
        tp_info = {"ranks": args.tp, "rank": r, "unit": args.tp_unit, "I": shares[r],
                   "Is": sshares[r]}
        w = w.with_(I=shares[r], Is=sshares[r])
        torch.cuda.empty_cache()
    torch.cuda.synchronize()
    print(f"inputs ready in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    gamma = None
    if args.norm:
        gg = torch.Generator().manual_seed(1000 * 0 + 7)
        gamma = (1.0 + 0.05 * torch.randn(w.H, generator=gg)).to(torch.bfloat16).to(dev)
    opts = dict(combine=args.combine, router=args.router, norm=gamma, residual=args.norm)

    hip = Hip()
    stream = torch.cuda.current_stream(dev)
    flush = torch.ones((1 << 28,), dtype=torch.int32, device=dev)  # 1 GiB
    runner = Runner(args, hip, flush)

    if args.graph:
        # replays of one call captured in a HIP graph (the eviction stays
        # outside the graph), on the same stream as eager calls would run
        out = torch.empty((w.T, w.H), dtype=torch.float32, device=dev)
        ws = torch.empty((moe.workspace_bytes(w.T, w.H, w.E, w.I, w.Is, w.topk,
                                              FMT_CODE[w.fmt]),), dtype=torch.uint8, device=dev)

        def call():
            moe.moe_ffn(d["x"], d["router_w"], d["bias"], d["experts"], d["shared"], w.band_lo,
                        w.band_hi, w.topk, out=out, workspace=ws, **opts)
        cap = torch.cuda.Stream(dev)
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            call()
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call()
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            runner.evict()
            graph.replay()
        torch.cuda.synchronize()
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        t0 = time.perf_counter()
        for i in range(args.steps):
            runner.evict()
            starts[i].record(stream)
            graph.replay()
            ends[i].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        layer_ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
        # the routing and stage breakdown come from eager calls
        r = runner.run(w, d, opts, min(args.steps, 10), 1, ws=ws, out=out)
        r.update({"ms": sum(layer_ms) / len(layer_ms), "ms_min": min(layer_ms), "wall": wall})
    else:
        r = runner.run(w, d, opts, args.steps, args.warmup)
    ms, ex, out = r["ms"], r["ex"], r["out"]
    counts = ex["counts"].cpu()
    # the counters were taken with the default routing on the whole layer
    roof = roofline_for(w, counts, r["stage"], counted=args.tp == 1 and args.router == "softmax")

    reduce_info = None
    if args.reduce_parts:
        # the exchange step: N band partials (copies of this output) added
        # along the canonical tree, then the shared output and the residual
        n = args.reduce_parts
        span = w.E // n
        parts = [out.clone() for _ in range(n)]
        bands = [(i * span, (i + 1) * span) for i in range(n)]
        red = torch.empty_like(out)
        r_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.steps)]
        for i in range(args.steps + 2):
            runner.evict()
            if i >= 2:
                r_ev[i - 2][0].record(stream)
            moe.reduce(parts, "tree", bands=bands, E=w.E, y_shared=out, residual=d["x"], out=red)
            if i >= 2:
                r_ev[i - 2][1].record(stream)
        torch.cuda.synchronize()
        r_ms = sum(a.elapsed_time(b) for a, b in r_ev) / len(r_ev)
        nbytes = (n + 2) * w.T * w.H * 4 + w.T * w.H * 2
        reduce_info = {"parts": n, "us": round(r_ms * 1e3, 2), "bytes": nbytes,
                       "GB_per_s": round(nbytes / (r_ms * 1e-3) / 1e9, 1)}

    line = {
        "metric": METRIC,
        "value": round(w.T / (ms * 1e-3), 2),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_min": round(r["ms_min"], 4),
        "us_per_layer": round(ms * 1e3, 2),
        "wall_ms_per_step_incl_eviction": round(r["wall"] / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": FMT_DTYPE[w.fmt],
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "H": w.H, "E": w.E, "topk": w.topk, "I": w.I,
                   "Is": w.Is, "fmt": w.fmt, "band": [w.band_lo, w.band_hi],
                   "combine": args.combine, "tp": tp_info, "router": args.router,
                   "launch": "hip graph replay" if args.graph else "eager",
                   "norm": "rmsnorm eps 1e-5 + residual" if args.norm else None,
                   "l2_mall_eviction": {"read": "1 GiB read", "write": "1 GiB write",
                                        "none": None}[args.flush]},
        "stage_us": {k: round(v * 1e3, 2) for k, v in r["stage"].items()},
        "roofline": roof,
        "layer": layer_roofline(w, counts, ms),
    }
    if reduce_info is not None:
        line["reduce"] = reduce_info
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(
            w, d, ex, args.cpu_rows,
            modes=dict(combine=args.combine, router=args.router,
                       norm=None if gamma is None else gamma.cpu(), residual=args.norm))
    plain = (args.workload == "decode" and args.tp == 1 and args.router == "softmax" and
             not args.norm and args.combine == "pick" and not args.graph and not args.reduce_parts)
    if plain and not args.no_extra:
        del r, out
        extra = extra_workloads(runner, d, dev, args)
        line["prefill"] = extra.pop("prefill")
        line["workloads"] = extra
    print(json.dumps(line, separators=(",", ":")), flush=True)


if __name__ == "__main__":
    main()
