"""The C ABI on the CPU (no GPU needed): the library loads, exports every
symbol the header declares, the ctypes layouts match the header, and every
argument check fails closed before any HIP call.

[P1] "GLM-5.2 multi-GPU: expert-parallel sharding + the resident-fit
benchmark", gates table: fail-closed rejections (plan.Dim != NumExperts,
ranks > experts).
"""

import ctypes
import os
import re
import subprocess

import pytest

import mixture_experts_ffn_06_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ffn.h")


def test_library_exports_every_declared_symbol():
    text = open(HEADER).read()
    declared = set(re.findall(r"^\S.*?\b(moe_\w+)\s*\(", text, flags=re.M))
    assert declared == {"moe_ffn", "moe_ffn_static", "moe_ffn_workspace_bytes", "moe_ffn_strerror", "moe_ffn_reduce",
                        "moe_tp_shares", "moe_tp_slice_experts", "moe_tp_slice_shared"}
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert declared <= exported
    lib = moe.load_library()
    for name in declared:
        assert hasattr(lib, name)


def _c_struct_layout(src_body: str):
    """Compile a tiny C program against the header and print sizeof/offsetof."""
    import tempfile

    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "probe.c")
        exe = os.path.join(d, "probe")
        with open(c, "w") as f:
            f.write('#include <stdio.h>\n#include <stddef.h>\n#include "moe_ffn.h"\nint main(void){\n')
            f.write(src_body)
            f.write("return 0;}\n")
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), "-o", exe, c], check=True)
        return subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()


@pytest.mark.parametrize("cname,pyname", [
    ("moe_x", "MoeX"), ("moe_router", "MoeRouter"), ("moe_experts", "MoeExperts"),
    ("moe_shared", "MoeShared"), ("moe_out", "MoeOut"),
])
def test_struct_layouts_match_header(cname, pyname):
    py = getattr(moe, pyname)
    body = f'printf("%zu ", sizeof({cname}));\n'
    for fname, _ in py._fields_:
        body += f'printf("%zu ", offsetof({cname}, {fname}));\n'
    vals = [int(v) for v in _c_struct_layout(body)]
    assert vals[0] == ctypes.sizeof(py)
    assert vals[1:] == [getattr(py, f).offset for f, _ in py._fields_]


def test_constants_match_header():
    text = open(HEADER).read()

    def define(name):
        m = re.search(rf"#define {name} \(?(-?\d+)", text)
        return int(m.group(1))

    for code, name in moe.ERRORS.items():
        assert define(name) == code
    assert define("MOE_NUM_EVENTS") == moe.MOE_NUM_EVENTS
    assert define("MOE_MAX_TOPK") == moe.MOE_MAX_TOPK
    assert define("MOE_MAX_E") == moe.MOE_MAX_E
    assert define("MOE_BF16") == moe.MOE_BF16 and define("MOE_W4A16") == moe.MOE_W4A16
    assert define("MOE_AFFINE4") == moe.MOE_AFFINE4 and define("MOE_NVFP4") == moe.MOE_NVFP4
    m = re.search(r"#define MOE_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert int(m.group(1)) << int(m.group(2)) == moe.MOE_STATIC_SCRATCH_BYTES


def test_strerror_every_code():
    for code in moe.ERRORS:
        assert moe.strerror(code) and moe.strerror(code) != "unknown error code"
    assert moe.strerror(-99) == "unknown error code"


def test_workspace_bytes():
    small = moe.workspace_bytes(4, 256, 8, 128, 128, 2)
    assert small > 0
    big = moe.workspace_bytes(4096, 6144, 256, 2048, 2048, 8)
    # at least the fp32 expert outputs of every pick and shared row
    assert big >= (4096 * 8 + 4096) * 6144 * 4
    assert moe.workspace_bytes(0, 256, 8, 128, 128, 2) == 0
    assert moe.workspace_bytes(4, 250, 8, 128, 128, 2) == 0
    assert moe.workspace_bytes(4, 256, 8, 100, 128, 2) == 0
    assert moe.workspace_bytes(4, 256, 8, 128, 128, 9) == 0
    assert moe.workspace_bytes(4, 256, 8, 128, 128, 2, 7) == 0


# Fake, aligned, never-dereferenced device addresses: every call below must be
# rejected by the argument checks, which run before any HIP call.
A = 1 << 20


def _call(T=4, H=256, E=8, I=128, Is=128, topk=2, lo=0, hi=8, fmt=0, group=32, rE=None, rH=None,
          eH=None, sH=None, shared=True, ws_bytes=None, null=None, misalign=None):
    ptr = {name: A * (i + 1) for i, name in enumerate(
        ["x", "wr", "bias", "wgu", "wd", "qgu", "sgu", "zgu", "qd", "sd", "zd", "swgu", "swd",
         "y", "ws", "ggu", "gd"])}
    if null:
        ptr[null] = None
    if misalign:
        ptr[misalign] += 8
    dx = moe.MoeX(ptr["x"], T, H)
    dr = moe.MoeRouter(ptr["wr"], ptr["bias"], E if rE is None else rE, H if rH is None else rH)
    de = moe.MoeExperts(E, H if eH is None else eH, I, fmt, group, ptr["wgu"], ptr["wd"], ptr["qgu"],
                        ptr["sgu"], ptr["zgu"], ptr["qd"], ptr["sd"], ptr["zd"], ptr["ggu"], ptr["gd"])
    ds = moe.MoeShared(Is, H if sH is None else sH, ptr["swgu"], ptr["swd"]) if shared else None
    need = moe.workspace_bytes(T, H, E, I, Is if shared else 0, max(1, min(topk, 16)), fmt if fmt in (0, 1, 2, 3) else 0)
    do = moe.MoeOut(ptr["y"], None, None, None, None, None, None, ptr["ws"],
                    need if ws_bytes is None else ws_bytes, None)
    lib = moe.load_library()
    return lib.moe_ffn(ctypes.byref(dx), ctypes.byref(dr), ctypes.byref(de),
                       ctypes.byref(ds) if ds else None, lo, hi, topk, ctypes.byref(do), None)


@pytest.mark.parametrize("kw,code", [
    (dict(null="x"), moe.MOE_E_NULL if hasattr(moe, "MOE_E_NULL") else -1),
    (dict(null="wr"), -1),
    (dict(null="y"), -1),
    (dict(null="wgu"), -1),
    (dict(null="wd"), -1),
    (dict(null="swgu"), -1),
    (dict(fmt=1, null="zd"), -1),
    (dict(H=250), -2),
    (dict(rH=512), -2),
    (dict(eH=512), -2),
    (dict(sH=512), -2),
    (dict(I=100), -2),
    (dict(Is=96), -2),
    (dict(T=0), -2),
    (dict(E=2000, hi=2000), -2),
    (dict(rE=9), -3),  # the router's expert count differs from the experts'
    (dict(lo=-1), -4),
    (dict(hi=9), -4),
    (dict(lo=3, hi=3), -4),
    (dict(lo=5, hi=4), -4),
    (dict(topk=0), -5),
    (dict(topk=9), -5),  # more picks than experts
    (dict(topk=17, E=32, hi=32), -5),
    (dict(fmt=2), -6),  # MLX affine with 32-input groups
    (dict(fmt=1, group=64), -6),
    (dict(fmt=3, group=32), -6),
    (dict(fmt=4), -6),
    (dict(fmt=2, group=64, I=192), -2),  # MLX affine needs I % 128 == 0
    (dict(fmt=2, group=64, null="zd"), -1),  # the biases
    (dict(fmt=3, group=16, null="ggu"), -1),  # the matrix scales
    (dict(fmt=3, group=16, null="gd"), -1),
    (dict(fmt=3, group=16, null="sd"), -1),
    (dict(fmt=3, group=16, misalign="ggu"), -8),
    (dict(ws_bytes=1024), -7),
    (dict(null="ws"), -7),
    (dict(misalign="x"), -8),
    (dict(misalign="wgu"), -8),
    (dict(misalign="y"), -8),
    (dict(misalign="ws"), -8),
])
def test_fail_closed(kw, code):
    assert _call(**kw) == code


def test_unused_format_pointers_ignored():
    # bf16 experts: the 4-bit pointers may be anything (here: misaligned).
    assert _call(misalign="qgu", ws_bytes=1024) == -7
    assert _call(fmt=1, misalign="wgu", ws_bytes=1024) == -7
    # NVFP4 has no zeros; W4A16 and MLX affine no matrix scales
    assert _call(fmt=3, group=16, null="zgu", ws_bytes=1024) == -7
    assert _call(fmt=2, group=64, null="ggu", ws_bytes=1024) == -7


def test_python_binding_raises(monkeypatch):
    import torch

    x = torch.zeros((4, 250), dtype=torch.bfloat16)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_ffn(x, torch.zeros(8, 250), None,
                    {"fmt": "bf16", "w_gate_up": torch.zeros(8, 256, 250, dtype=torch.bfloat16),
                     "w_down": torch.zeros(8, 250, 128, dtype=torch.bfloat16)},
                    None, 0, 8, 2, workspace=torch.zeros(16, dtype=torch.uint8))
    assert e.value.code == -2


def test_tp_shares_match_the_page_examples():
    # host-only entry point: the shares the page prints (tests/golden/tp_shares.json)
    import json
    cases = json.load(open(os.path.join(ROOT, "tests", "golden", "tp_shares.json")))["cases"]
    for c in cases:
        assert moe.tp_shares(c["dim"], c["unit"], c["ranks"]) == c["shares"], c["what"]
    for args in ((2000, 64, 3), (64, 64, 2), (0, 64, 1), (128, 64, 0)):
        with pytest.raises(moe.MoeError) as e:
            moe.tp_shares(*args)
        assert e.value.code == -2
