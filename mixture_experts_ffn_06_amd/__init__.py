"""Python binding of libmoeffn.so: one routed mixture-of-experts FFN layer,
restricted to an expert band, on an MI355X (gfx950).

Argument marshalling only: every step of the layer runs in the HIP kernels of
libmoeffn.so.  torch supplies device memory and the stream.  The binding fails
loudly when the library is not built; there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoeffn.so")

MOE_BF16 = 0
MOE_W4A16 = 1
MOE_AFFINE4 = 2
MOE_NVFP4 = 3
_FORMATS = {"bf16": MOE_BF16, "w4": MOE_W4A16, "affine4": MOE_AFFINE4, "nvfp4": MOE_NVFP4}
_GROUP = {MOE_BF16: 0, MOE_W4A16: 32, MOE_AFFINE4: 64, MOE_NVFP4: 16}
MOE_MAX_TOPK = 16
MOE_MAX_E = 1024
MOE_NUM_EVENTS = 9
EVENT_SLOTS = ("router", "topk", "dispatch", "gu_gemv", "gu_mfma", "dn_gemv", "dn_mfma",
               "combine", "end")

ERRORS = {
    0: "MOE_OK", -1: "MOE_E_NULL", -2: "MOE_E_SHAPE", -3: "MOE_E_DIM", -4: "MOE_E_BAND",
    -5: "MOE_E_TOPK", -6: "MOE_E_FORMAT", -7: "MOE_E_WORKSPACE", -8: "MOE_E_ALIGN",
    -9: "MOE_E_HIP", -10: "MOE_E_DEVICE", -11: "MOE_E_COMBINE", -12: "MOE_E_ROUTER",
    -13: "MOE_E_SCRATCH",
}
MOE_STATIC_SCRATCH_BYTES = 32 << 20
MOE_ROUTER_SOFTMAX = 0
MOE_ROUTER_SIGMOID = 1
_ROUTER = {"softmax": MOE_ROUTER_SOFTMAX, "sigmoid": MOE_ROUTER_SIGMOID}
MOE_COMBINE_PICK = 0
MOE_COMBINE_TREE = 1
MOE_REDUCE_RANK = 0
MOE_REDUCE_TREE = 1
MOE_MAX_PARTS = 64
_COMBINE = {"pick": MOE_COMBINE_PICK, "tree": MOE_COMBINE_TREE}
_REDUCE = {"rank": MOE_REDUCE_RANK, "tree": MOE_REDUCE_TREE}


class MoeError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERRORS.get(code, code)}: {message}")
        self.code = code
        self.name = ERRORS.get(code, str(code))


class MoeX(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("norm_w", ctypes.c_void_p), ("eps", ctypes.c_float)]


class MoeRouter(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("E", ctypes.c_int32),
                ("H", ctypes.c_int32), ("mode", ctypes.c_int32)]


class MoeExperts(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("fmt", ctypes.c_int32), ("group", ctypes.c_int32),
                ("w_gate_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("q_gate_up", ctypes.c_void_p), ("s_gate_up", ctypes.c_void_p),
                ("z_gate_up", ctypes.c_void_p), ("q_down", ctypes.c_void_p),
                ("s_down", ctypes.c_void_p), ("z_down", ctypes.c_void_p),
                ("g_gate_up", ctypes.c_void_p), ("g_down", ctypes.c_void_p)]


class MoeShared(ctypes.Structure):
    _fields_ = [("Is", ctypes.c_int32), ("H", ctypes.c_int32), ("w_gate_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p)]


class MoeOut(ctypes.Structure):
    _fields_ = [("y", ctypes.c_void_p), ("topk_ids", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
                ("counts", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
                ("perm", ctypes.c_void_p), ("pos", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("stage_events", ctypes.c_void_p), ("y_shared", ctypes.c_void_p),
                ("y_picks", ctypes.c_void_p), ("combine", ctypes.c_int32),
                ("residual", ctypes.c_int32), ("xn", ctypes.c_void_p)]


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libmoeffn.so; raises when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoeError(-9, f"{LIB_PATH} is not built; run `python -m mixture_experts_ffn_06_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P, I32 = ctypes.c_void_p, ctypes.c_int32
        lib.moe_ffn.restype = I32
        lib.moe_ffn.argtypes = [ctypes.POINTER(MoeX), ctypes.POINTER(MoeRouter),
                                ctypes.POINTER(MoeExperts), ctypes.POINTER(MoeShared), I32, I32,
                                I32, ctypes.POINTER(MoeOut), P]
        lib.moe_ffn_static.restype = I32
        lib.moe_ffn_static.argtypes = lib.moe_ffn.argtypes
        lib.moe_ffn_workspace_bytes.restype = ctypes.c_size_t
        lib.moe_ffn_workspace_bytes.argtypes = [I32] * 7
        lib.moe_ffn_strerror.restype = ctypes.c_char_p
        lib.moe_ffn_strerror.argtypes = [I32]
        lib.moe_tp_shares.restype = I32
        lib.moe_tp_shares.argtypes = [I32, I32, I32, P]
        lib.moe_tp_slice_experts.restype = I32
        lib.moe_tp_slice_experts.argtypes = [ctypes.POINTER(MoeExperts), I32, I32,
                                             ctypes.POINTER(MoeExperts), P]
        lib.moe_tp_slice_shared.restype = I32
        lib.moe_tp_slice_shared.argtypes = [ctypes.POINTER(MoeShared), I32, I32,
                                            ctypes.POINTER(MoeShared), P]
        lib.moe_ffn_reduce.restype = I32
        lib.moe_ffn_reduce.argtypes = [P, I32, P, P, I32, I32, P, P, I32, I32, P, P]
        _lib = lib
    return _lib


def strerror(code: int) -> str:
    return load_library().moe_ffn_strerror(code).decode()


def workspace_bytes(T: int, H: int, E: int, I: int, Is: int, topk: int, fmt: int = MOE_BF16) -> int:
    return int(load_library().moe_ffn_workspace_bytes(T, H, E, I, Is, topk, fmt))


def _p(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _fmt_code(experts: dict) -> int:
    return _FORMATS[experts["fmt"]]


def make_descriptors(x, router_w, bias, experts, shared, E=None, I=None, router="softmax",
                     norm=None, eps=1e-5):
    """ctypes descriptors for the tensors (no copies, no checks: the library checks)."""
    T, H = x.shape
    fmt = _fmt_code(experts)
    if E is None:
        E = (experts["w_gate_up"] if fmt == MOE_BF16 else experts["q_gate_up"]).shape[0]
    if I is None:
        I = (experts["w_gate_up"] if fmt == MOE_BF16 else experts["q_gate_up"]).shape[1] // 2
    dx = MoeX(_p(x), T, H, _p(norm), eps)
    dr = MoeRouter(_p(router_w), _p(bias), router_w.shape[0], router_w.shape[1],
                   _ROUTER[router] if router in _ROUTER else int(router))
    de = MoeExperts(E, H, I, fmt, _GROUP[fmt],
                    _p(experts.get("w_gate_up")), _p(experts.get("w_down")),
                    _p(experts.get("q_gate_up")), _p(experts.get("s_gate_up")),
                    _p(experts.get("z_gate_up")), _p(experts.get("q_down")),
                    _p(experts.get("s_down")), _p(experts.get("z_down")),
                    _p(experts.get("g_gate_up")), _p(experts.get("g_down")))
    ds = None
    if shared is not None:
        ds = MoeShared(shared["w_down"].shape[1], shared["w_gate_up"].shape[1],
                       _p(shared["w_gate_up"]), _p(shared["w_down"]))
    return dx, dr, de, ds


def moe_ffn(x: torch.Tensor, router_w: torch.Tensor, bias: Optional[torch.Tensor], experts: dict,
            shared: Optional[dict], band_lo: int, band_hi: int, topk: int,
            out: Optional[torch.Tensor] = None, exports: Optional[dict] = None,
            workspace: Optional[torch.Tensor] = None, stream=None, events=None,
            combine: str = "pick", y_shared: Optional[torch.Tensor] = None,
            y_picks: Optional[torch.Tensor] = None, router: str = "softmax",
            norm: Optional[torch.Tensor] = None, eps: float = 1e-5, residual: bool = False,
            xn: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Run the layer for the expert band [band_lo, band_hi).

    x bf16 [T,H]; router_w fp32 [E,H]; bias fp32 [E] or None; experts / shared
    as produced by the synth module (dicts of device tensors).  Returns the fp32
    [T,H] partial residual (`out` if given).  `exports`, if a dict, receives
    topk_ids, topk_w, counts, offsets, perm, pos.  `events` is a list of
    MOE_NUM_EVENTS raw hipEvent_t handles recorded at the stage boundaries.
    combine: "pick" (pick order) or "tree" (canonical tree over expert ids).
    y_shared: fp32 [T,H] receiving the shared expert's output instead of
    adding it; y_picks: fp32 [T*topk,H] receiving the per-pick expert outputs
    in perm order.  router: "softmax" (bias on the logits) or "sigmoid" (bias
    steers the selection only, raw-score weights).  norm: bf16 [H] RMSNorm
    weight (the layer runs on the normed rows, eps as given); residual: add
    the raw rows last; xn: bf16 [T,H] receiving the normed rows.
    """
    return _layer(False, x, router_w, bias, experts, shared, band_lo, band_hi, topk, out, exports,
                  workspace, stream, events, combine, y_shared, y_picks, router, norm, eps, residual,
                  xn)


def moe_ffn_static(x: torch.Tensor, router_w: torch.Tensor, bias: Optional[torch.Tensor],
                   experts: dict, shared: Optional[dict], band_lo: int, band_hi: int, topk: int,
                   out: Optional[torch.Tensor] = None, exports: Optional[dict] = None, stream=None,
                   events=None, combine: str = "pick", y_shared: Optional[torch.Tensor] = None,
                   y_picks: Optional[torch.Tensor] = None, router: str = "softmax",
                   norm: Optional[torch.Tensor] = None, eps: float = 1e-5, residual: bool = False,
                   xn: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_ffn with its scratch in the library's static per-GPU array
    (MOE_STATIC_SCRATCH_BYTES): the library call allocates nothing.  Calls
    that overlap on one GPU share that array and race.  Arguments as moe_ffn,
    without a workspace; `out` and the exports are still the caller's (this
    wrapper allocates them with torch when they are not given)."""
    return _layer(True, x, router_w, bias, experts, shared, band_lo, band_hi, topk, out, exports,
                  None, stream, events, combine, y_shared, y_picks, router, norm, eps, residual, xn)


def _layer(static, x, router_w, bias, experts, shared, band_lo, band_hi, topk, out, exports,
           workspace, stream, events, combine, y_shared, y_picks, router, norm, eps, residual, xn):
    if combine not in _COMBINE:
        raise MoeError(-11, f"combine must be one of {sorted(_COMBINE)}")
    lib = load_library()
    T, H = x.shape
    dx, dr, de, ds = make_descriptors(x, router_w, bias, experts, shared, router=router, norm=norm,
                                      eps=eps)
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=dev)
    ex = {}
    if exports is not None:
        nb = band_hi - band_lo
        ex = {
            "topk_ids": torch.empty((T, topk), dtype=torch.int32, device=dev),
            "topk_w": torch.empty((T, topk), dtype=torch.float32, device=dev),
            "counts": torch.empty((max(nb, 1),), dtype=torch.int32, device=dev),
            "offsets": torch.empty((max(nb, 0) + 1,), dtype=torch.int32, device=dev),
            "perm": torch.empty((T * topk,), dtype=torch.int32, device=dev),
            "pos": torch.empty((T * topk,), dtype=torch.int32, device=dev),
        }
    if workspace is None and not static:
        nbytes = lib.moe_ffn_workspace_bytes(T, H, de.E, de.I, ds.Is if ds else 0, topk, de.fmt)
        workspace = torch.empty((max(int(nbytes), 1),), dtype=torch.uint8, device=dev)
    ev_arr = None
    if events is not None:
        ev_arr = (ctypes.c_void_p * MOE_NUM_EVENTS)(*events)
    dout = MoeOut(_p(out), _p(ex.get("topk_ids")), _p(ex.get("topk_w")), _p(ex.get("counts")),
                  _p(ex.get("offsets")), _p(ex.get("perm")), _p(ex.get("pos")),
                  _p(workspace), 0 if workspace is None else workspace.numel(),
                  ctypes.cast(ev_arr, ctypes.c_void_p) if ev_arr is not None else None,
                  _p(y_shared), _p(y_picks), _COMBINE[combine], 1 if residual else 0, _p(xn))
    if stream is None:
        st = torch.cuda.current_stream(dev).cuda_stream if dev.type == "cuda" else 0
    else:
        st = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    entry = lib.moe_ffn_static if static else lib.moe_ffn
    rc = entry(ctypes.byref(dx), ctypes.byref(dr), ctypes.byref(de),
               ctypes.byref(ds) if ds is not None else None, band_lo, band_hi, topk,
               ctypes.byref(dout), ctypes.c_void_p(st))
    if rc != 0:
        raise MoeError(rc, strerror(rc))
    if exports is not None:
        exports.update(ex)
    return out


def _stream_handle(dev, stream):
    if stream is None:
        return torch.cuda.current_stream(dev).cuda_stream if dev.type == "cuda" else 0
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def reduce(parts, order: str = "rank", bands=None, E: int = 0,
           y_shared: Optional[torch.Tensor] = None, residual: Optional[torch.Tensor] = None,
           out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Sum fp32 [T,H] band partials in rank order or along the canonical tree
    (bands: their [lo, hi) ranges, tree nodes), then + y_shared, + residual
    (bf16 [T,H])."""
    if order not in _REDUCE:
        raise MoeError(-11, f"order must be one of {sorted(_REDUCE)}")
    lib = load_library()
    T, H = parts[0].shape
    dev = parts[0].device
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=dev)
    n = len(parts)
    arr = (ctypes.c_void_p * max(n, 1))(*[p.data_ptr() for p in parts])
    lo = hi = None
    if bands is not None:
        lo = (ctypes.c_int32 * n)(*[int(b[0]) for b in bands])
        hi = (ctypes.c_int32 * n)(*[int(b[1]) for b in bands])
    rc = lib.moe_ffn_reduce(ctypes.cast(arr, ctypes.c_void_p), n,
                            ctypes.cast(lo, ctypes.c_void_p) if lo is not None else None,
                            ctypes.cast(hi, ctypes.c_void_p) if hi is not None else None,
                            E, _REDUCE[order], _p(y_shared), _p(residual), T, H, _p(out),
                            ctypes.c_void_p(_stream_handle(dev, stream)))
    if rc != 0:
        raise MoeError(rc, strerror(rc))
    return out


def tp_shares(dim: int, unit: int, ranks: int):
    """Tensor-parallel shares of dim: whole units, remainder on the lowest ranks."""
    arr = (ctypes.c_int32 * max(ranks, 1))()
    rc = load_library().moe_tp_shares(dim, unit, ranks, ctypes.cast(arr, ctypes.c_void_p))
    if rc != 0:
        raise MoeError(rc, strerror(rc))
    return list(arr)[:ranks]


_SLICE_GU = ("w_gate_up", "q_gate_up", "s_gate_up", "z_gate_up")


def tp_slice_experts(experts: dict, i_lo: int, i_hi: int, stream=None) -> dict:
    """A rank's slice of every routed expert (intermediate columns
    [i_lo, i_hi)), laid out by the library into new device tensors."""
    lib = load_library()
    fmt = _fmt_code(experts)
    ref = experts["w_gate_up"] if fmt == MOE_BF16 else experts["q_gate_up"]
    E, I2 = ref.shape[0], ref.shape[1]
    I = I2 // 2
    n = i_hi - i_lo
    out = {"fmt": experts["fmt"]}
    for name, t in experts.items():
        if not isinstance(t, torch.Tensor):
            continue
        shape = list(t.shape)
        if name in ("g_gate_up", "g_down"):
            pass  # NVFP4 matrix scales: kept whole
        elif name in _SLICE_GU:
            shape[1] = 2 * n
        else:  # down projection: inputs along the last dimension
            shape[2] = shape[2] * n // I
        out[name] = torch.empty(shape, dtype=t.dtype, device=t.device)
    H = (out.get("w_down") if fmt == MOE_BF16 else out["q_down"]).shape[1]
    src = make_descriptors(torch.empty((1, H)), torch.empty((E, H)), None, experts, None, E=E, I=I)[2]
    dst = make_descriptors(torch.empty((1, H)), torch.empty((E, H)), None, out, None, E=E, I=n)[2]
    rc = lib.moe_tp_slice_experts(ctypes.byref(src), i_lo, i_hi, ctypes.byref(dst),
                                  ctypes.c_void_p(_stream_handle(ref.device, stream)))
    if rc != 0:
        raise MoeError(rc, strerror(rc))
    return out


def tp_slice_shared(shared: dict, i_lo: int, i_hi: int, stream=None) -> dict:
    """A rank's slice of the shared expert (columns [i_lo, i_hi) of Is)."""
    lib = load_library()
    gu, dn = shared["w_gate_up"], shared["w_down"]
    H, Is, n = gu.shape[1], dn.shape[1], i_hi - i_lo
    out = {"w_gate_up": torch.empty((2 * n, H), dtype=gu.dtype, device=gu.device),
           "w_down": torch.empty((H, n), dtype=dn.dtype, device=dn.device)}
    src = MoeShared(Is, H, _p(gu), _p(dn))
    dst = MoeShared(n, H, _p(out["w_gate_up"]), _p(out["w_down"]))
    rc = lib.moe_tp_slice_shared(ctypes.byref(src), i_lo, i_hi, ctypes.byref(dst),
                                 ctypes.c_void_p(_stream_handle(gu.device, stream)))
    if rc != 0:
        raise MoeError(rc, strerror(rc))
    return out


def tree_pieces(lo: int, hi: int, E: int):
    """Cut the band [lo, hi) into canonical-tree nodes (clipped to [0, E)),
    largest first from the left: the bands whose tree-mode outputs
    moe_ffn_reduce adds back exactly.  Host logic only."""
    if not (0 <= lo < hi <= E):
        raise ValueError(f"band [{lo}, {hi}) outside [0, {E})")
    Ep = 1
    while Ep < E:
        Ep *= 2
    out = []
    a = lo
    while a < hi:
        size = 1
        # grow while the node stays aligned, inside the padded range, and its
        # in-range part stays inside the band
        while a % (2 * size) == 0 and a + 2 * size <= Ep and min(a + 2 * size, E) <= hi:
            size *= 2
        b = min(a + size, E)
        out.append((a, b))
        a = b
    return out


__all__ = ["MOE_AFFINE4", "MOE_NVFP4", "moe_ffn", "moe_ffn_static", "MOE_STATIC_SCRATCH_BYTES", "reduce", "tree_pieces", "tp_shares", "tp_slice_experts", "tp_slice_shared", "workspace_bytes", "strerror", "load_library", "MoeError", "LIB_PATH",
           "MOE_BF16", "MOE_W4A16", "MOE_NUM_EVENTS", "EVENT_SLOTS", "make_descriptors",
           "MoeX", "MoeRouter", "MoeExperts", "MoeShared", "MoeOut", "MOE_COMBINE_PICK",
           "MOE_COMBINE_TREE", "MOE_REDUCE_RANK", "MOE_REDUCE_TREE", "MOE_MAX_PARTS",
           "MOE_ROUTER_SOFTMAX", "MOE_ROUTER_SIGMOID"]
