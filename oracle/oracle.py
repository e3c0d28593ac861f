"""Python access to the plain CPU oracle (moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark use this module; the product path never imports it.  It
shares no code with the HIP library.

All arguments are CPU torch tensors (bf16 tensors are passed by their bits).
Results come back as CPU tensors: logits fp32, weights and outputs fp64,
indices int32.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fp contraction: explicit fmaf only)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", "-Wall",
             "-o", tmp, _SRC, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


class _Experts(ctypes.Structure):
    _fields_ = [
        ("fmt", ctypes.c_int32),
        ("E", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("I", ctypes.c_int32),
        ("w_gate_up", ctypes.c_void_p),
        ("w_down", ctypes.c_void_p),
        ("q_gate_up", ctypes.c_void_p),
        ("s_gate_up", ctypes.c_void_p),
        ("z_gate_up", ctypes.c_void_p),
        ("q_down", ctypes.c_void_p),
        ("s_down", ctypes.c_void_p),
        ("z_down", ctypes.c_void_p),
        ("g_gate_up", ctypes.c_void_p),
        ("g_down", ctypes.c_void_p),
    ]


# weight formats of the oracle (its own numbering)
_FMT = {"bf16": 0, "w4": 1, "affine4": 2, "nvfp4": 3}


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P, I32 = ctypes.c_void_p, ctypes.c_int32
        lib.oracle_dot_r.restype = ctypes.c_float
        lib.oracle_dot_r.argtypes = [P, P, I32]
        lib.oracle_router_logits.restype = I32
        lib.oracle_router_logits.argtypes = [P, I32, I32, P, P, I32, P]
        lib.oracle_topk.restype = I32
        lib.oracle_topk.argtypes = [P, I32, I32, I32, P, P]
        lib.oracle_dispatch.restype = I32
        lib.oracle_dispatch.argtypes = [P, I32, I32, I32, I32, P, P, P, P]
        lib.oracle_expert_ffn.restype = I32
        lib.oracle_expert_ffn.argtypes = [P, ctypes.POINTER(_Experts), I32, P]
        lib.oracle_expert_matrix.restype = I32
        lib.oracle_expert_matrix.argtypes = [ctypes.POINTER(_Experts), I32, I32, P]
        lib.oracle_fp4_e2m1.restype = ctypes.c_double
        lib.oracle_fp4_e2m1.argtypes = [I32]
        lib.oracle_fp8_e4m3.restype = ctypes.c_double
        lib.oracle_fp8_e4m3.argtypes = [I32]
        layer = [P, I32, I32, P, P, I32, ctypes.POINTER(_Experts), P, P, I32]
        lib.oracle_moe_ffn.restype = I32
        lib.oracle_moe_ffn.argtypes = layer + [I32, I32, I32, I32, I32, P, ctypes.c_float, I32,
                                               P, I32, P, P, P]
        lib.oracle_rmsnorm.restype = I32
        lib.oracle_rmsnorm.argtypes = [P, I32, I32, P, ctypes.c_float, P, P]
        lib.oracle_exp_c.restype = ctypes.c_float
        lib.oracle_exp_c.argtypes = [ctypes.c_float]
        lib.oracle_sigmoid_c.restype = ctypes.c_float
        lib.oracle_sigmoid_c.argtypes = [ctypes.c_float]
        lib.oracle_topk_sigmoid.restype = I32
        lib.oracle_topk_sigmoid.argtypes = [P, P, I32, I32, I32, P, P]
        lib.oracle_tree_node.restype = I32
        lib.oracle_tree_node.argtypes = [I32, I32, I32, ctypes.POINTER(I32), ctypes.POINTER(I32)]
        lib.oracle_tree_value.restype = I32
        lib.oracle_tree_value.argtypes = [P, P, I32, I32, I32, ctypes.c_size_t, P]
        lib.oracle_tp_shares.restype = I32
        lib.oracle_tp_shares.argtypes = [I32, I32, I32, P]
        lib.oracle_tree_merge.restype = I32
        lib.oracle_tree_merge.argtypes = [I32, I32, P, P, P, P, ctypes.c_size_t, P]
        lib.oracle_rank_merge.restype = I32
        lib.oracle_rank_merge.argtypes = [I32, P, P, P, ctypes.c_size_t, P]
        lib.oracle_moe_ffn_monolith.restype = I32
        lib.oracle_moe_ffn_monolith.argtypes = layer + [I32, P, I32, P]
        _lib = lib
    return _lib


def _cpu(t: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if t is None:
        return None
    return t.detach().to("cpu").contiguous()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(rc: int, what: str):
    if rc < 0:
        raise ValueError(f"oracle: {what} rejected its arguments")
    return rc


class Experts:
    """Holds CPU copies of routed expert weights and the ctypes descriptor."""

    def __init__(self, experts: dict, E: int, H: int, I: int):
        self.keep = {k: _cpu(v) for k, v in experts.items() if isinstance(v, torch.Tensor)}
        fmt = experts["fmt"]
        gsz = {"w4": 32, "affine4": 64, "nvfp4": 16}.get(fmt, 0)
        if fmt == "bf16":
            want = {"w_gate_up": (2 * I, H), "w_down": (H, I)}
        else:
            want = {"q_gate_up": (2 * I, H // 2), "s_gate_up": (2 * I, H // gsz),
                    "q_down": (H, I // 2), "s_down": (H, I // gsz)}
            if fmt == "nvfp4":
                want.update({"g_gate_up": (2,), "g_down": ()})
            else:
                want.update({"z_gate_up": (2 * I, H // gsz), "z_down": (H, I // gsz)})
        for name, shape in want.items():
            t = self.keep.get(name)
            if t is not None and (tuple(t.shape[1:]) != shape or t.shape[0] < E):
                raise ValueError(f"oracle: {name} has shape {tuple(t.shape)}, want [{E}, {shape}]")
        if fmt == "nvfp4":
            for name in ("s_gate_up", "s_down"):
                if self.keep.get(name) is not None and self.keep[name].dtype != torch.uint8:
                    raise ValueError(f"oracle: nvfp4 {name} must be uint8 (E4M3 bytes)")
            for name in ("g_gate_up", "g_down"):
                if self.keep.get(name) is not None and self.keep[name].dtype != torch.float32:
                    raise ValueError(f"oracle: nvfp4 {name} must be fp32")
        d = _Experts()
        d.fmt = _FMT[fmt]
        d.E, d.H, d.I = E, H, I
        for name in ("w_gate_up", "w_down", "q_gate_up", "s_gate_up", "z_gate_up",
                     "q_down", "s_down", "z_down", "g_gate_up", "g_down"):
            t = self.keep.get(name)
            setattr(d, name, None if t is None else t.data_ptr())
        self.desc = d


def dot_r(x: torch.Tensor, w: torch.Tensor) -> float:
    """The fixed-order fp32 router dot of two fp32 vectors (length % 256 == 0)."""
    x, w = _cpu(x).float(), _cpu(w).float()
    return float(_load().oracle_dot_r(_ptr(x), _ptr(w), x.numel()))


def router_logits(x: torch.Tensor, router_w: torch.Tensor, bias: Optional[torch.Tensor]) -> torch.Tensor:
    x, wr, b = _cpu(x), _cpu(router_w).float(), _cpu(bias)
    T, H = x.shape
    E = wr.shape[0]
    out = torch.empty((T, E), dtype=torch.float32)
    _check(_load().oracle_router_logits(_ptr(x), T, H, _ptr(wr), _ptr(b), E, _ptr(out)), "router")
    return out


def topk(logits: torch.Tensor, k: int):
    lg = _cpu(logits).float()
    T, E = lg.shape
    ids = torch.empty((T, k), dtype=torch.int32)
    w = torch.empty((T, k), dtype=torch.float64)
    _check(_load().oracle_topk(_ptr(lg), T, E, k, _ptr(ids), _ptr(w)), "topk")
    return ids, w


def exp_c(x: float) -> float:
    """The fixed fp32 exp of the sigmoid router (range reduction by ln 2,
    degree-6 Taylor polynomial, exact scaling)."""
    return float(_load().oracle_exp_c(float(x)))


def sigmoid_c(x: float) -> float:
    """The fixed fp32 sigmoid 1 / (1 + exp_c(-x))."""
    return float(_load().oracle_sigmoid_c(float(x)))


def topk_sigmoid(logits: torch.Tensor, bias: Optional[torch.Tensor], k: int):
    """Sigmoid router: picks by (sigmoid(l) + bias desc, id asc), weights the
    raw scores.  logits are unbiased."""
    lg = _cpu(logits).float()
    b = None if bias is None else _cpu(bias).float()
    T, E = lg.shape
    ids = torch.empty((T, k), dtype=torch.int32)
    w = torch.empty((T, k), dtype=torch.float64)
    _check(_load().oracle_topk_sigmoid(_ptr(lg), _ptr(b), T, E, k, _ptr(ids), _ptr(w)),
           "topk_sigmoid")
    return ids, w


def rmsnorm(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-5):
    """Normed bf16 rows (every step one fp32 rounding, the sum of squares in
    R-order) and the per-row inverse RMS."""
    xb = _cpu(x).to(torch.bfloat16).contiguous()
    g = _cpu(gamma).to(torch.bfloat16).contiguous()
    T, H = xb.shape
    out = torch.empty((T, H), dtype=torch.bfloat16)
    inv = torch.empty(T, dtype=torch.float32)
    _check(_load().oracle_rmsnorm(_ptr(xb), T, H, _ptr(g), eps, _ptr(out), _ptr(inv)), "rmsnorm")
    return out, inv


def dispatch(ids: torch.Tensor, lo: int, hi: int):
    """Returns (counts [nb], offsets [nb+1], perm [N_in], pos [T*k])."""
    ids = _cpu(ids).to(torch.int32)
    T, k = ids.shape
    nb = hi - lo
    counts = torch.empty(nb, dtype=torch.int32)
    offsets = torch.empty(nb + 1, dtype=torch.int32)
    perm = torch.empty(max(T * k, 1), dtype=torch.int32)
    pos = torch.empty(max(T * k, 1), dtype=torch.int32)
    n = _check(_load().oracle_dispatch(_ptr(ids), T, k, lo, hi, _ptr(counts), _ptr(offsets),
                                       _ptr(perm), _ptr(pos)), "dispatch")
    return counts, offsets, perm[:n].clone(), pos[: T * k].clone()


def expert_ffn(x_row: torch.Tensor, experts: Experts, e: int) -> torch.Tensor:
    """One expert's SwiGLU FFN on one fp64 row."""
    xd = _cpu(x_row).to(torch.float64)
    y = torch.empty(experts.desc.H, dtype=torch.float64)
    _check(_load().oracle_expert_ffn(_ptr(xd), ctypes.byref(experts.desc), e, _ptr(y)), "expert_ffn")
    return y


def expert_matrix(experts: Experts, e: int, which: int) -> torch.Tensor:
    """Dequantised fp64 weights of expert e: which=0 gate/up [2I,H], 1 down [H,I]."""
    d = experts.desc
    shape = (2 * d.I, d.H) if which == 0 else (d.H, d.I)
    out = torch.empty(shape, dtype=torch.float64)
    _check(_load().oracle_expert_matrix(ctypes.byref(d), e, which, _ptr(out)), "expert_matrix")
    return out


def fp4_e2m1(code: int) -> float:
    """Value of a 4-bit FP4 E2M1 code (the oracle's decode)."""
    return float(_load().oracle_fp4_e2m1(int(code)))


def fp8_e4m3(byte: int) -> float:
    """Value of an FP8 E4M3 byte (the oracle's decode; NaN for the NaN codes)."""
    return float(_load().oracle_fp8_e4m3(int(byte)))


def tp_shares(dim: int, unit: int, ranks: int):
    """Tensor-parallel shares of dim: whole units, remainder on the lowest ranks."""
    out = torch.empty(max(ranks, 1), dtype=torch.int32)
    _check(_load().oracle_tp_shares(dim, unit, ranks, _ptr(out)), "tp_shares")
    return out[:ranks].tolist()


def tp_slice(experts: dict, i_lo: int, i_hi: int) -> dict:
    """The intermediate columns [i_lo, i_hi) of every expert (gate rows, up
    rows, down-projection inputs), as a smaller expert set.  Plain indexing of
    the stored arrays: bf16 [E,2I,H] / [E,H,I], or 4-bit codes with one
    (scale, zero) per 32 inputs."""
    fmt = experts["fmt"]
    if fmt == "bf16":
        gu = experts["w_gate_up"]
        I = gu.shape[-2] // 2
        rows = list(range(i_lo, i_hi)) + list(range(I + i_lo, I + i_hi))
        out = {"fmt": fmt, "w_gate_up": gu[..., rows, :].contiguous(),
               "w_down": experts["w_down"][..., i_lo:i_hi].contiguous()}
        return out
    q = experts["q_gate_up"]
    I = q.shape[-2] // 2
    rows = list(range(i_lo, i_hi)) + list(range(I + i_lo, I + i_hi))
    gsz = {"w4": 32, "affine4": 64, "nvfp4": 16}[fmt]
    out = {"fmt": fmt,
           "q_gate_up": q[..., rows, :].contiguous(),
           "s_gate_up": experts["s_gate_up"][..., rows, :].contiguous(),
           "q_down": experts["q_down"][..., i_lo // 2:i_hi // 2].contiguous(),
           "s_down": experts["s_down"][..., i_lo // gsz:i_hi // gsz].contiguous()}
    if fmt == "nvfp4":
        # the per-matrix scales are the whole matrix's: a slice keeps them
        out["g_gate_up"] = experts["g_gate_up"].clone()
        out["g_down"] = experts["g_down"].clone()
    else:
        out["z_gate_up"] = experts["z_gate_up"][..., rows, :].contiguous()
        out["z_down"] = experts["z_down"][..., i_lo // gsz:i_hi // gsz].contiguous()
    return out


def tree_node(E: int, lo: int, hi: int):
    """(first leaf, level) of the smallest canonical-tree node containing [lo, hi)."""
    nlo, lev = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(_load().oracle_tree_node(E, lo, hi, ctypes.byref(nlo), ctypes.byref(lev)), "tree_node")
    return nlo.value, lev.value


def tree_value(ids, vals: torch.Tensor, node_lo: int, level: int) -> torch.Tensor:
    """fp32 value of a canonical-tree node: leaf ids[i] holds the fp32 row
    vals[i] (vals [m, n]), every other leaf +0.0.  Returns [n]."""
    idt = torch.as_tensor(ids, dtype=torch.int32).contiguous()
    v = _cpu(vals).float().contiguous()
    m = idt.numel()
    n = v.shape[1] if m else (v.numel() if v.dim() == 1 else v.shape[-1])
    out = torch.empty(n, dtype=torch.float32)
    _check(_load().oracle_tree_value(_ptr(idt), _ptr(v), m, node_lo, level, n, _ptr(out)),
           "tree_value")
    return out


def tree_merge(parts, bands, E: int, shared: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Sum of fp32 band partials along the canonical tree (+ shared last)."""
    ps = [_cpu(p).float().contiguous() for p in parts]
    n = ps[0].numel()
    lo = torch.tensor([b[0] for b in bands], dtype=torch.int32)
    hi = torch.tensor([b[1] for b in bands], dtype=torch.int32)
    arr = (ctypes.c_void_p * len(ps))(*[p.data_ptr() for p in ps])
    sh = None if shared is None else _cpu(shared).float().contiguous()
    out = torch.empty(n, dtype=torch.float32)
    _check(_load().oracle_tree_merge(E, len(ps), _ptr(lo), _ptr(hi), ctypes.cast(arr, ctypes.c_void_p),
                                     _ptr(sh), n, _ptr(out)), "tree_merge")
    return out.reshape(ps[0].shape)


def rank_merge(parts, shared: Optional[torch.Tensor] = None,
               residual: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp32 rank partials added in rank order (a left fold), then + shared,
    then + the bf16 residual."""
    ps = [_cpu(p).float().contiguous() for p in parts]
    n = ps[0].numel()
    arr = (ctypes.c_void_p * len(ps))(*[p.data_ptr() for p in ps])
    sh = None if shared is None else _cpu(shared).float().contiguous()
    res = None if residual is None else _cpu(residual).to(torch.bfloat16).contiguous().view(torch.int16)
    out = torch.empty(n, dtype=torch.float32)
    _check(_load().oracle_rank_merge(len(ps), ctypes.cast(arr, ctypes.c_void_p), _ptr(sh), _ptr(res), n,
                                     _ptr(out)), "rank_merge")
    return out.reshape(ps[0].shape)


def moe_ffn(inputs: dict, E: int, I: int, Is: int, lo: int, hi: int, k: int,
            rows: Optional[torch.Tensor] = None, experts: Optional[Experts] = None,
            combine: str = "pick", router: str = "softmax",
            norm: Optional[torch.Tensor] = None, eps: float = 1e-5, residual: bool = False):
    """The layer for the band [lo, hi) on the listed rows (all rows if None).
    combine: "pick" (pick order) or "tree" (canonical tree over expert ids).
    router: "softmax" (bias on the logits) or "sigmoid" (bias steers the
    selection only, weights are the raw scores).  norm: bf16 [H] RMSNorm
    weight (the layer then runs on the normed rows); residual: add the raw
    rows last.
    Returns (out fp64 [nrows, H], ids int32 [nrows, k], w fp64 [nrows, k])."""
    if combine not in ("pick", "tree"):
        raise ValueError(f"oracle: combine {combine!r}")
    if router not in ("softmax", "sigmoid"):
        raise ValueError(f"oracle: router {router!r}")
    x, wr, b = _cpu(inputs["x"]), _cpu(inputs["router_w"]).float(), _cpu(inputs["bias"])
    T, H = x.shape
    ex = experts if experts is not None else Experts(inputs["experts"], E, H, I)
    sh = inputs.get("shared")
    sgu = _cpu(sh["w_gate_up"]) if sh else None
    sd = _cpu(sh["w_down"]) if sh else None
    r = None if rows is None else _cpu(rows).to(torch.int32)
    gm = None if norm is None else _cpu(norm).to(torch.bfloat16).contiguous()
    nrows = T if r is None else r.numel()
    out = torch.empty((nrows, H), dtype=torch.float64)
    ids = torch.empty((nrows, k), dtype=torch.int32)
    w = torch.empty((nrows, k), dtype=torch.float64)
    # The router's expert count comes from the router weight itself; the
    # experts' from their descriptor -- the oracle rejects a mismatch.
    Er = wr.shape[0]
    if b is not None and b.numel() != Er:
        raise ValueError("oracle: bias length != router experts")
    _check(_load().oracle_moe_ffn(_ptr(x), T, H, _ptr(wr), _ptr(b), Er, ctypes.byref(ex.desc),
                                  _ptr(sgu), _ptr(sd), Is if sh else 0, lo, hi, k,
                                  0 if combine == "pick" else 1, 0 if router == "softmax" else 1,
                                  _ptr(gm), eps, 1 if residual else 0, _ptr(r), nrows,
                                  _ptr(out), _ptr(ids), _ptr(w)), "moe_ffn")
    return out, ids, w


def moe_ffn_monolith(inputs: dict, E: int, I: int, Is: int, k: int,
                     rows: Optional[torch.Tensor] = None, experts: Optional[Experts] = None):
    """The routed layer with no band logic (every pick contributes)."""
    x, wr, b = _cpu(inputs["x"]), _cpu(inputs["router_w"]).float(), _cpu(inputs["bias"])
    T, H = x.shape
    ex = experts if experts is not None else Experts(inputs["experts"], E, H, I)
    sh = inputs.get("shared")
    sgu = _cpu(sh["w_gate_up"]) if sh else None
    sd = _cpu(sh["w_down"]) if sh else None
    r = None if rows is None else _cpu(rows).to(torch.int32)
    nrows = T if r is None else r.numel()
    out = torch.empty((nrows, H), dtype=torch.float64)
    Er = wr.shape[0]
    if b is not None and b.numel() != Er:
        raise ValueError("oracle: bias length != router experts")
    _check(_load().oracle_moe_ffn_monolith(_ptr(x), T, H, _ptr(wr), _ptr(b), Er, ctypes.byref(ex.desc),
                                           _ptr(sgu), _ptr(sd), Is if sh else 0, k, _ptr(r), nrows,
                                           _ptr(out)), "moe_ffn_monolith")
    return out
