"""Instruction order that the shared expert's gate/up staging relies on, read
from the gfx950 assembly of dispatch.hip (CPU only: hipcc cross-compiles).

The rows go to LDS by direct global->LDS loads, then each wave issues its
first column's 2 x 6 weight loads, waits with vmcnt(12) (loads return in
issue order, so only the weights may still be in flight) and meets the others
at a plain s_barrier.  That is only right if every row load issues before the
twelve weight loads and nothing else counted by vmcnt sits between them, and
if no LDS read of the rows comes before the barrier.  Every instantiation
(one per row count, in each top-k/dispatch kernel) is checked.
"""

import os
import re
import shutil
import subprocess

import pytest

from mixture_experts_ffn_06_amd import build as hb

VM_OPS = re.compile(r"^\s*(global_|buffer_|flat_|scratch_)\w*")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(hb.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "dispatch.s"
    flags = [f for f in hb.FLAGS if f != "-fPIC"]
    cmd = [hb.HIPCC, *flags, "-x", "hip", "--cuda-device-only", "-S",
           os.path.join(hb.CSRC, "dispatch.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    lines = [ln.split(";")[0].rstrip() for ln in out.read_text().splitlines()]
    return [ln for ln in lines if ln.strip()]


def test_row_loads_then_weights_then_wait_then_barrier(asm):
    sites = [i for i, ln in enumerate(asm) if ln.strip() == "s_waitcnt vmcnt(12)"]
    # 8 row counts x 2 top-k/dispatch kernels
    assert len(sites) >= 16, f"{len(sites)} staging waits found"
    for i in sites:
        # the barrier follows the wait (labels and scalar moves may sit between)
        nxt = next(j for j in range(i + 1, len(asm)) if "s_barrier" in asm[j] or "ds_read" in asm[j]
                   or VM_OPS.match(asm[j]))
        assert "s_barrier" in asm[nxt], f"line {i}: {asm[nxt]!r} before the barrier"
        # back from the wait to the last row load
        k = max(j for j in range(i) if "global_load_lds" in asm[j])
        span = asm[k + 1:i]
        vm = [ln.strip() for ln in span if VM_OPS.match(ln)]
        assert len(vm) == 12 and all(v.startswith("global_load_dwordx4") for v in vm), \
            f"between the last row load and the wait at line {i}: {vm}"
        assert not any("ds_read" in ln for ln in span), f"LDS read before the barrier at line {i}"
