"""Seeded synthetic inputs for the routed mixture-of-experts FFN layer.

This module is shared by the oracle side (tests, CPU baseline) and the GPU
side (tests, benchmark).  It holds random draws and the storage-format packing
of those draws only -- none of the layer's arithmetic (no routing, no
selection, no products).

The pages measure on real GLM-5.2 / GLM-5.3-Flash checkpoints that are not
available here; these synthetic workloads stand in for them with the shapes
and distributions listed in WORKLOADS.  Every tensor has its own generator,
seeded ``1000 * workload_seed + tensor_index`` (workload_seed is 0 for every
workload), so a tensor's values do not depend on which other tensors are made.
Large tensors are drawn on the device they live on, one expert at a time.
"""

from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import torch

# Tensor indices for the per-tensor seeds.
_IDX_X, _IDX_WR, _IDX_BIAS = 0, 1, 2
_IDX_WGU, _IDX_WD, _IDX_SGU, _IDX_SD = 3, 4, 5, 6
_IDX_QGU, _IDX_SGU4, _IDX_ZGU4, _IDX_QD, _IDX_SD4, _IDX_ZD4 = 7, 8, 9, 10, 11, 12
_IDX_GGU, _IDX_GD = 13, 14

# Scale on the log-Zipf router bias (see zipf_bias).  With this scale the
# realised expert popularity of the prefill workload (top-8 of 256 experts,
# router logits of standard deviation about 0.02 * sqrt(6144)) falls off with
# a log-log slope of about -1.1 over popularity ranks 2..128; the test suite
# measures the realised histogram with the oracle's router.
ZIPF_BETA = 0.80
ZIPF_S = 1.1


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    topk: int
    I: int
    Is: int  # 0 = no shared expert
    fmt: str = "bf16"  # "bf16" | "w4" | "affine4" | "nvfp4"
    bias: Optional[str] = None  # None | "zipf" | "band0" | "one_expert" | "first_k"
    band: tuple = (0, 0)  # (lo, hi); hi = 0 means the full band [0, E)
    seed: int = 0
    w_std: float = 0.02  # expert / shared weights ~ N(0, w_std)
    wr_std: float = 0.02  # router weights ~ N(0, wr_std)

    @property
    def band_lo(self) -> int:
        return self.band[0]

    @property
    def band_hi(self) -> int:
        return self.band[1] if self.band[1] > 0 else self.E

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads: tiny, decode, prefill (Zipf-skewed groups), expert bands
# on one GPU (plus the adversarial all-picks-in-band-0 case), and 4-bit
# group-affine experts at one row and at 2048 rows; plus a compute-bound
# probe of the shared expert alone at prefill size.
WORKLOADS = {
    "tiny": Workload("tiny", T=4, H=256, E=8, topk=2, I=128, Is=128),
    "decode": Workload("decode", T=8, H=6144, E=256, topk=8, I=2048, Is=2048),
    "prefill": Workload("prefill", T=4096, H=6144, E=256, topk=8, I=2048, Is=2048, bias="zipf"),
    "bands": Workload("bands", T=512, H=6144, E=256, topk=8, I=2048, Is=2048),
    "bands_adversarial": Workload(
        "bands_adversarial", T=512, H=6144, E=256, topk=8, I=2048, Is=2048, bias="band0"
    ),
    "w4_t1": Workload("w4_t1", T=1, H=6144, E=256, topk=8, I=2048, Is=2048, fmt="w4"),
    "w4_t2048": Workload("w4_t2048", T=2048, H=6144, E=256, topk=8, I=2048, Is=2048, fmt="w4"),
    # The other 4-bit checkpoint formats on the same shapes: MLX affine
    # (64-input groups, s * q + b) and NVFP4 (E2M1 codes, an E4M3 scale per 16
    # inputs and an fp32 scale per matrix).
    "affine4_t1": Workload("affine4_t1", T=1, H=6144, E=256, topk=8, I=2048, Is=2048, fmt="affine4"),
    "affine4_t2048": Workload("affine4_t2048", T=2048, H=6144, E=256, topk=8, I=2048, Is=2048, fmt="affine4"),
    "nvfp4_t1": Workload("nvfp4_t1", T=1, H=6144, E=256, topk=8, I=2048, Is=2048, fmt="nvfp4"),
    "nvfp4_t2048": Workload("nvfp4_t2048", T=2048, H=6144, E=256, topk=8, I=2048, Is=2048, fmt="nvfp4"),
    # Compute-bound probe: prefill sizes with every pick on experts 0..7 and
    # the band [8, 256), so no routed pick is in the band and the MFMA work
    # is the shared expert's 4096 rows alone.
    "shared_probe": Workload(
        "shared_probe", T=4096, H=6144, E=256, topk=8, I=2048, Is=2048, bias="first_k", band=(8, 256)
    ),
}

BAND_WIDTH = 32  # the expert-band workload runs bands [32b, 32b + 32)


def _gen(device, seed: int, index: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(1000 * seed + index)
    return g


def _normal_bf16(shape, std, device, g, chunk_dim0=False) -> torch.Tensor:
    """N(0, std) drawn in fp32 and rounded to bf16 (round-to-nearest-even)."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    if chunk_dim0:
        for i in range(shape[0]):
            tmp = torch.empty(shape[1:], dtype=torch.float32, device=device)
            tmp.normal_(0.0, std, generator=g)
            out[i].copy_(tmp)
    else:
        tmp = torch.empty(shape, dtype=torch.float32, device=device)
        tmp.normal_(0.0, std, generator=g)
        out.copy_(tmp)
    return out


def _uniform_bf16(shape, lo, hi, device, g, chunk_dim0=False) -> torch.Tensor:
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    if chunk_dim0:
        for i in range(shape[0]):
            tmp = torch.empty(shape[1:], dtype=torch.float32, device=device)
            tmp.uniform_(lo, hi, generator=g)
            out[i].copy_(tmp)
    else:
        tmp = torch.empty(shape, dtype=torch.float32, device=device)
        tmp.uniform_(lo, hi, generator=g)
        out.copy_(tmp)
    return out


def _codes_w4(shape, device, g) -> torch.Tensor:
    """Uniform 4-bit codes in [0, 15] for a [E, N, K] matrix, packed two per
    byte along K with the even k in the low nibble: result [E, N, K/2] uint8."""
    E, N, K = shape
    out = torch.empty((E, N, K // 2), dtype=torch.uint8, device=device)
    for e in range(E):
        q = torch.randint(0, 16, (N, K), generator=g, device=device, dtype=torch.int32)
        out[e].copy_((q[:, 0::2] | (q[:, 1::2] << 4)).to(torch.uint8))
    return out


def _affine_bias(scale: torch.Tensor, device, g) -> torch.Tensor:
    """MLX affine biases: -scale * u with u ~ U(7, 9) per group (the affine
    form of a zero point mid-range of the codes), rounded to bf16."""
    out = torch.empty(scale.shape, dtype=torch.bfloat16, device=device)
    for i in range(scale.shape[0]):
        u = torch.empty(scale.shape[1:], dtype=torch.float32, device=device)
        u.uniform_(7.0, 9.0, generator=g)
        out[i].copy_(-scale[i].float() * u)
    return out


def _e4m3_bytes(shape, lo, hi, device, g) -> torch.Tensor:
    """FP8 E4M3 bytes of values ~U(lo, hi) (rounded to nearest even), as uint8."""
    out = torch.empty(shape, dtype=torch.uint8, device=device)
    for i in range(shape[0]):
        u = torch.empty(shape[1:], dtype=torch.float32, device=device)
        u.uniform_(lo, hi, generator=g)
        out[i].copy_(u.to(torch.float8_e4m3fn).view(torch.uint8))
    return out


def zipf_bias(E: int, seed: int, s: float = ZIPF_S, beta: float = ZIPF_BETA) -> torch.Tensor:
    """Per-expert router offset b_e = beta * ln p_{pi(e)}, where p_r is Zipf(s)
    over popularity ranks r = 1..E and pi is a seeded permutation of the
    experts (so popularity is not tied to the expert id).  fp32, on the CPU."""
    g = _gen("cpu", seed, _IDX_BIAS)
    perm = torch.randperm(E, generator=g)
    r = torch.arange(1, E + 1, dtype=torch.float64)
    p = r.pow(-s)
    p = p / p.sum()
    b = torch.empty(E, dtype=torch.float64)
    b[torch.arange(E)] = beta * torch.log(p[perm])
    return b.to(torch.float32)


def make_bias(w: Workload) -> Optional[torch.Tensor]:
    if w.bias is None:
        return None
    if w.bias == "zipf":
        return zipf_bias(w.E, w.seed)
    if w.bias == "band0":
        # +10 on experts [0, 32): with top-8, every row picks 8 of those 32.
        b = torch.zeros(w.E, dtype=torch.float32)
        b[:BAND_WIDTH] = 10.0
        return b
    if w.bias == "first_k":
        # +1000 on the first topk experts: far beyond any logit of these
        # weights at any T, so every row picks exactly them
        b = torch.zeros(w.E, dtype=torch.float32)
        b[: w.topk] = 1000.0
        return b
    if w.bias == "one_expert":
        # +10 on the first topk experts: every row picks exactly them.
        b = torch.zeros(w.E, dtype=torch.float32)
        b[: w.topk] = 10.0
        return b
    raise ValueError(f"unknown bias kind {w.bias!r}")


def make_router(w: Workload, device="cpu") -> dict:
    """x [T,H] bf16 ~ N(0,1), router weight [E,H] fp32 ~ N(0, wr_std), and the
    optional per-expert bias [E] fp32."""
    x = _normal_bf16((w.T, w.H), 1.0, device, _gen(device, w.seed, _IDX_X))
    wr = torch.empty((w.E, w.H), dtype=torch.float32, device=device)
    wr.normal_(0.0, w.wr_std, generator=_gen(device, w.seed, _IDX_WR))
    b = make_bias(w)
    return {"x": x, "router_w": wr, "bias": None if b is None else b.to(device)}


def make_experts(w: Workload, device="cpu") -> dict:
    """Routed expert weights.  bf16: w_gate_up [E, 2I, H] (gate rows first),
    w_down [E, H, I].  w4: codes [E, N, K/2] uint8 plus bf16 scale ~U(.005,.02)
    and zero ~U(7,9) per 32-wide group along K."""
    E, H, I = w.E, w.H, w.I
    if w.fmt == "bf16":
        return {
            "fmt": "bf16",
            "w_gate_up": _normal_bf16((E, 2 * I, H), w.w_std, device, _gen(device, w.seed, _IDX_WGU), True),
            "w_down": _normal_bf16((E, H, I), w.w_std, device, _gen(device, w.seed, _IDX_WD), True),
        }
    if w.fmt == "w4":
        return {
            "fmt": "w4",
            "q_gate_up": _codes_w4((E, 2 * I, H), device, _gen(device, w.seed, _IDX_QGU)),
            "s_gate_up": _uniform_bf16((E, 2 * I, H // 32), 0.005, 0.02, device, _gen(device, w.seed, _IDX_SGU4), True),
            "z_gate_up": _uniform_bf16((E, 2 * I, H // 32), 7.0, 9.0, device, _gen(device, w.seed, _IDX_ZGU4), True),
            "q_down": _codes_w4((E, H, I), device, _gen(device, w.seed, _IDX_QD)),
            "s_down": _uniform_bf16((E, H, I // 32), 0.005, 0.02, device, _gen(device, w.seed, _IDX_SD4), True),
            "z_down": _uniform_bf16((E, H, I // 32), 7.0, 9.0, device, _gen(device, w.seed, _IDX_ZD4), True),
        }
    if w.fmt == "affine4":
        s_gu = _uniform_bf16((E, 2 * I, H // 64), 0.005, 0.02, device, _gen(device, w.seed, _IDX_SGU4), True)
        s_d = _uniform_bf16((E, H, I // 64), 0.005, 0.02, device, _gen(device, w.seed, _IDX_SD4), True)
        return {
            "fmt": "affine4",
            "q_gate_up": _codes_w4((E, 2 * I, H), device, _gen(device, w.seed, _IDX_QGU)),
            "s_gate_up": s_gu,
            "z_gate_up": _affine_bias(s_gu, device, _gen(device, w.seed, _IDX_ZGU4)),
            "q_down": _codes_w4((E, H, I), device, _gen(device, w.seed, _IDX_QD)),
            "s_down": s_d,
            "z_down": _affine_bias(s_d, device, _gen(device, w.seed, _IDX_ZD4)),
        }
    if w.fmt == "nvfp4":
        # block scales in E4M3's normal range, per-matrix scales ~U(1/512, 1/256):
        # weights up to 6 * 4 / 256 in magnitude
        g_gu = torch.empty((E, 2), dtype=torch.float32, device=device)
        g_gu.uniform_(1.0 / 512, 1.0 / 256, generator=_gen(device, w.seed, _IDX_GGU))
        g_d = torch.empty((E,), dtype=torch.float32, device=device)
        g_d.uniform_(1.0 / 512, 1.0 / 256, generator=_gen(device, w.seed, _IDX_GD))
        return {
            "fmt": "nvfp4",
            "q_gate_up": _codes_w4((E, 2 * I, H), device, _gen(device, w.seed, _IDX_QGU)),
            "s_gate_up": _e4m3_bytes((E, 2 * I, H // 16), 1.5, 4.0, device, _gen(device, w.seed, _IDX_SGU4)),
            "q_down": _codes_w4((E, H, I), device, _gen(device, w.seed, _IDX_QD)),
            "s_down": _e4m3_bytes((E, H, I // 16), 1.5, 4.0, device, _gen(device, w.seed, _IDX_SD4)),
            "g_gate_up": g_gu,
            "g_down": g_d,
        }
    raise ValueError(f"unknown format {w.fmt!r}")


def make_shared(w: Workload, device="cpu") -> Optional[dict]:
    """Shared expert (bf16, unrouted): w_gate_up [2Is, H], w_down [H, Is]."""
    if w.Is <= 0:
        return None
    return {
        "w_gate_up": _normal_bf16((2 * w.Is, w.H), w.w_std, device, _gen(device, w.seed, _IDX_SGU)),
        "w_down": _normal_bf16((w.H, w.Is), w.w_std, device, _gen(device, w.seed, _IDX_SD)),
    }


def make_inputs(w: Workload, device="cpu") -> dict:
    d = make_router(w, device)
    d["experts"] = make_experts(w, device)
    d["shared"] = make_shared(w, device)
    return d


def expert_bytes(w: Workload) -> int:
    """Bytes of one routed expert's weights as stored."""
    if w.fmt == "bf16":
        return 3 * w.H * w.I * 2
    codes = 3 * w.H * w.I // 2
    if w.fmt == "w4":
        return codes + 2 * (3 * w.H * w.I // 32) * 2  # bf16 scale and zero per 32
    if w.fmt == "affine4":
        return codes + 2 * (3 * w.H * w.I // 64) * 2  # bf16 scale and bias per 64
    return codes + 3 * w.H * w.I // 16 + 3 * 4  # E4M3 scale per 16, fp32 per matrix


def shared_bytes(w: Workload) -> int:
    return 3 * w.H * w.Is * 2 if w.Is > 0 else 0


def bands(w: Workload):
    """The expert bands [32b, 32b + 32) of the band workload, in band order."""
    return [(lo, min(lo + BAND_WIDTH, w.E)) for lo in range(0, w.E, BAND_WIDTH)]


__all__ = [
    "Workload",
    "WORKLOADS",
    "BAND_WIDTH",
    "ZIPF_BETA",
    "ZIPF_S",
    "make_inputs",
    "make_router",
    "make_experts",
    "make_shared",
    "make_bias",
    "zipf_bias",
    "expert_bytes",
    "shared_bytes",
    "bands",
]
