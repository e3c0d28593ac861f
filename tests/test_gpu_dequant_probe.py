"""Bit-exact probe of the in-kernel 4-bit dequantisation of the down
projection, on both expert paths.

[P5] "GLM-5.3-Flash and full GLM-5.3 on the native CUDA engine (tracker)
#593", "What exists now": glue kernels are fixed byte-exactly against host
references; "The pieces, in order": W4A16 checkpoints, weight = (code - zero)
* scale per 32-input group.

Constructed 4-bit gate/up rows make each expert's intermediate h one-hot:
with the rows x = e_{k_t} (one-hot inputs), gate row i0 decodes to 32 at every
input and up row i0 to 1/32, every other gate/up row to exactly 0 (codes equal
to an integer zero point).  So g = 32, silu(32) = 32 in fp32 (exp(-32) is far
below half an ulp of 1), h[i0] = 32 * (1/32) = 1 and h[i] = 0 elsewhere, all
exact in bf16.  The expert output y = W_down h is then column i0 of the
dequantised down matrix, exported through y_picks.  The down matrix keeps
random codes, scales ~U(.005, .02) and non-integer zeros ~U(7, 9), so
(code - zero) * scale needs up to 17 significant bits: exact in fp32.

Expected, from the oracle's exact (fp64) decode of the same stored bytes:
  groups of <= 8 rows (GEMV path): the fp32 value itself, bit for bit;
  larger groups (MFMA path, bf16 operands): round-to-nearest-even bf16 of it.

The other two 4-bit formats, built the same way:
  MLX affine (weight = s * q + b per 64 inputs, bf16 s and b): gate/up codes 0
  with bias 0 give weight 0, row i0 codes 1 with scales 32 and 1/32.  The down
  matrix keeps random codes, scales ~U(.005, .02) and biases -s * U(7, 9) in
  bf16, so s * q + b is exact in fp32; expected as for W4A16.
  NVFP4 (weight = e2m1(q) * e4m3(s) per 16 inputs * a per-matrix fp32 scale):
  gate/up codes 0 (+0) give weight 0, row i0 code 2 (1.0) with block scales
  0x60 (32) and 0x10 (1/32), matrix scales 1.  The down matrix keeps random
  codes (both signs), random finite E4M3 block scales and a random fp32 matrix
  scale per expert.  e2m1 * e4m3 has at most 6 significant bits, exact in bf16,
  and the matrix scale multiplies the finished sum on both paths, so the
  expected value is the fp32 rounding of the exact decode on both paths.
"""

import pytest
import torch

import mixture_experts_ffn_06_amd as moe
from gpu_common import log
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

H, E, K = 512, 16, 4
# intermediate widths: 256 takes the 128-weight-row MFMA tiles for the down
# projection, 512 the 512-weight-row tiles (K a multiple of 512)
WIDTHS = [256, 512]


def _pack(q):
    q = q.to(torch.int32)
    return (q[..., 0::2] | (q[..., 1::2] << 4)).to(torch.uint8)


def _router(T, g):
    # one-hot rows at random inputs; zero router with a bias that fixes each
    # row's picks (experts 3, 7, 11, 14 in that order)
    kt = torch.randint(0, H, (T,), generator=g)
    x = torch.zeros(T, H)
    x[torch.arange(T), kt] = 1.0
    bias = torch.zeros(E)
    for j, e in enumerate((3, 7, 11, 14)):
        bias[e] = 10.0 - j
    return x.to(torch.bfloat16), bias


def _inputs_affine(T, i0, seed, I):
    g = torch.Generator().manual_seed(seed)
    q_gu = torch.zeros((E, 2 * I, H), dtype=torch.int64)
    s_gu = torch.full((E, 2 * I, H // 64), 0.01)
    for e in range(E):
        q_gu[e, i0[e]] = 1
        q_gu[e, I + i0[e]] = 1
        s_gu[e, i0[e]] = 32.0
        s_gu[e, I + i0[e]] = 1.0 / 32.0
    b_gu = torch.zeros((E, 2 * I, H // 64))
    q_dn = torch.randint(0, 16, (E, H, I), generator=g)
    bf = torch.bfloat16
    s_dn = (torch.rand(E, H, I // 64, generator=g) * 0.015 + 0.005).to(bf)
    b_dn = (-s_dn.float() * (torch.rand(E, H, I // 64, generator=g) * 2 + 7)).to(bf)
    experts = {"fmt": "affine4", "q_gate_up": _pack(q_gu), "s_gate_up": s_gu.to(bf),
               "z_gate_up": b_gu.to(bf), "q_down": _pack(q_dn), "s_down": s_dn, "z_down": b_dn}
    return (*_router(T, g), experts)


def _inputs_nvfp4(T, i0, seed, I):
    g = torch.Generator().manual_seed(seed)
    q_gu = torch.zeros((E, 2 * I, H), dtype=torch.int64)
    s_gu = torch.full((E, 2 * I, H // 16), 0x38, dtype=torch.uint8)  # 1.0
    for e in range(E):
        q_gu[e, i0[e]] = 2  # e2m1 1.0
        q_gu[e, I + i0[e]] = 2
        s_gu[e, i0[e]] = 0x60  # 32
        s_gu[e, I + i0[e]] = 0x10  # 1/32
    q_dn = torch.randint(0, 16, (E, H, I), generator=g)
    s_dn = torch.randint(0, 0x7f, (E, H, I // 16), generator=g)  # finite E4M3, both halves of the range
    s_dn = (s_dn | (torch.randint(0, 2, s_dn.shape, generator=g) << 7)).to(torch.uint8)
    experts = {"fmt": "nvfp4", "q_gate_up": _pack(q_gu), "s_gate_up": s_gu, "q_down": _pack(q_dn),
               "s_down": s_dn, "g_gate_up": torch.ones(E, 2),
               "g_down": torch.rand(E, generator=g) * 0.75 + 0.25}
    return (*_router(T, g), experts)


def _inputs(T, i0, seed, I):
    g = torch.Generator().manual_seed(seed)
    # gate/up: zero point 8 everywhere, codes 8 (weight 0) except gate and up
    # row i0[e] of every expert: codes 9 with scales 32 and 1/32
    q_gu = torch.full((E, 2 * I, H), 8)
    s_gu = torch.full((E, 2 * I, H // 32), 0.01)
    for e in range(E):
        q_gu[e, i0[e]] = 9
        q_gu[e, I + i0[e]] = 9
        s_gu[e, i0[e]] = 32.0
        s_gu[e, I + i0[e]] = 1.0 / 32.0
    z_gu = torch.full((E, 2 * I, H // 32), 8.0)
    q_dn = torch.randint(0, 16, (E, H, I), generator=g)
    s_dn = torch.rand(E, H, I // 32, generator=g) * 0.015 + 0.005
    z_dn = torch.rand(E, H, I // 32, generator=g) * 2 + 7
    bf = torch.bfloat16
    experts = {"fmt": "w4", "q_gate_up": _pack(q_gu), "s_gate_up": s_gu.to(bf),
               "z_gate_up": z_gu.to(bf), "q_down": _pack(q_dn), "s_down": s_dn.to(bf),
               "z_down": z_dn.to(bf)}
    return (*_router(T, g), experts)


@pytest.mark.parametrize("I", WIDTHS)
@pytest.mark.parametrize("fmt", ["w4", "affine4", "nvfp4"])
@pytest.mark.parametrize("T", [1, 3, 8, 9, 20, 40, 100, 129, 300])
def test_down_dequant_bit_exact(T, fmt, I):
    i0 = [(37 * e + 11 * T) % I for e in range(E)]
    make = {"w4": _inputs, "affine4": _inputs_affine, "nvfp4": _inputs_nvfp4}[fmt]
    x, bias, experts = make(T, i0, seed=100 + T, I=I)
    dev = "cuda"
    xg = x.to(dev)
    exg = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in experts.items()}
    wr = torch.zeros(E, H, device=dev)
    y_picks = torch.full((T * K, H), float("nan"), device=dev)
    ex = {}
    moe.moe_ffn(xg, wr, bias.to(dev), exg, None, 0, E, K, exports=ex, y_picks=y_picks)
    torch.cuda.synchronize()
    ids = ex["topk_ids"].cpu()
    assert (ids == torch.tensor([3, 7, 11, 14], dtype=torch.int32)).all()
    perm = ex["perm"].cpu()
    yp = y_picks.cpu()
    oe = orc.Experts(experts, E, H, I)
    cols = {e: orc.expert_matrix(oe, e, 1)[:, i0[e]] for e in (3, 7, 11, 14)}
    mfma = T > 8  # a group holds all T rows: GEMV path up to 8 rows
    for r in range(T * K):
        t, j = divmod(int(perm[r]), K)
        e = int(ids[t, j])
        exact32 = cols[e].float()
        if fmt == "nvfp4":
            want = exact32  # the fp32 rounding of the exact decode, both paths
        else:
            assert torch.equal(exact32.double(), cols[e]), "decoded value not exact in fp32"
            want = exact32.to(torch.bfloat16).float() if mfma else exact32
        got = yp[r]
        if not torch.equal(got, want):
            bad = int((got != want).sum())
            raise AssertionError(f"{fmt} T={T} pick row {r} (expert {e}, column {i0[e]}): {bad} of {H} "
                                 f"values differ, e.g. got {got[got != want][:3].tolist()} want "
                                 f"{want[got != want][:3].tolist()}")
    path = "MFMA path" if mfma else "GEMV path"
    kind = "fp32" if fmt == "nvfp4" or not mfma else "bf16 RNE"
    log(f"{fmt} T={T} I={I}: {T * K} pick rows x {H} values bit-exact ({kind}, {path})")
