"""Pins for the oracle's decode of the two other 4-bit checkpoint formats.

[P5] "GLM-5.3-Flash and full GLM-5.3 on the native CUDA engine (tracker)
#593", "The pieces, in order": the family's checkpoint formats include MLX
affine 4-bit and NVIDIA's NVFP4 read as stored (W4A16); [P4] "GLM-5.3-Flash
on CUDA over three ranks (--tp 3) ... #310", comments: NVFP4's 16-input
groups, MLX's 64.

MLX affine: weight = s * q + b, bf16 s and b per 64 inputs.  NVFP4: weight =
e2m1(q) * e4m3(s) * g, an FP8 E4M3 scale per 16 inputs and an fp32 scale per
matrix.  The pins check the element decodes against published value tables
and an independent library decode, and the matrix layouts against closed
forms whose group boundaries differ from the other formats', so a wrong
group width, array or scale fails.
"""

import math

import pytest
import torch

import synth
from oracle import oracle as orc


def bf16(a):
    return torch.as_tensor(a, dtype=torch.float32).to(torch.bfloat16)


def _pack(q):
    q = q.to(torch.int32)
    return (q[..., 0::2] | (q[..., 1::2] << 4)).to(torch.uint8)


# --------------------------------------------------------------------------
# Element decodes.
# --------------------------------------------------------------------------

# The FP4 E2M1 value set of the OCP Microscaling formats specification, in
# code order (bit 3 the sign).
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_fp4_e2m1_value_table():
    for c in range(16):
        v = orc.fp4_e2m1(c)
        want = (-1.0 if c & 8 else 1.0) * E2M1[c & 7]
        assert v == want, c
        assert math.copysign(1.0, v) == (-1.0 if c & 8 else 1.0)  # code 8 is -0.0


def test_fp8_e4m3_matches_the_library_decode():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double()
    for b in range(256):
        v = orc.fp8_e4m3(b)
        r = float(ref[b])
        if math.isnan(r):
            assert math.isnan(v), b
        else:
            assert v == r and math.copysign(1.0, v) == math.copysign(1.0, r), b
    # published landmarks: 1, the largest finite, the smallest normal and subnormal
    assert orc.fp8_e4m3(0x38) == 1.0 and orc.fp8_e4m3(0x7E) == 448.0
    assert orc.fp8_e4m3(0x08) == 2.0 ** -6 and orc.fp8_e4m3(0x01) == 2.0 ** -9


# --------------------------------------------------------------------------
# MLX affine 4-bit matrices: s * q + b per 64 inputs.
# --------------------------------------------------------------------------

def _affine(H, I, gu, dn):
    return {"fmt": "affine4", "q_gate_up": _pack(gu[0]), "s_gate_up": gu[1], "z_gate_up": gu[2],
            "q_down": _pack(dn[0]), "s_down": dn[1], "z_down": dn[2]}


def _affine_noise(N, K, g):
    return (torch.randint(0, 16, (1, N, K), generator=g),
            bf16(torch.rand(1, N, K // 64, generator=g) * 0.015 + 0.005),
            bf16(-(torch.rand(1, N, K // 64, generator=g) * 2 + 7) * 0.01))


@pytest.mark.parametrize("which", [0, 1])
def test_affine_unit_scale_zero_bias_is_codes(which):
    H, I = 128, 64
    g = torch.Generator().manual_seed(31)
    N, K = (2 * I, H) if which == 0 else (H, I)
    q = torch.randint(0, 16, (1, N, K), generator=g)
    plain = (q, bf16(torch.ones(1, N, K // 64)), bf16(torch.zeros(1, N, K // 64)))
    other = _affine_noise(H if which == 0 else 2 * I, I if which == 0 else H, g)
    ex = orc.Experts(_affine(H, I, plain, other) if which == 0 else _affine(H, I, other, plain), 1, H, I)
    assert torch.equal(orc.expert_matrix(ex, 0, which), q[0].double())


@pytest.mark.parametrize("which", [0, 1])
def test_affine_groups_are_64_wide(which):
    # codes 0 give the group's bias and codes 1 its scale + bias, with a
    # different (s, b) per 64 inputs: 32-wide groups would repeat group 0's
    # values at inputs 32..63 only if they read the same entries -- they
    # read entry 1 instead
    H, I = 256, 128
    g = torch.Generator().manual_seed(32)
    N, K = (2 * I, H) if which == 0 else (H, I)
    s = bf16(torch.rand(1, N, K // 64, generator=g) * 0.5 + 0.25)
    b = bf16(torch.rand(1, N, K // 64, generator=g) - 0.5)
    q = torch.zeros(1, N, K, dtype=torch.int64)
    q[..., 1::2] = 1
    plain = (q, s, b)
    other = _affine_noise(H if which == 0 else 2 * I, I if which == 0 else H, g)
    ex = orc.Experts(_affine(H, I, plain, other) if which == 0 else _affine(H, I, other, plain), 1, H, I)
    m = orc.expert_matrix(ex, 0, which)
    want = b[0].double().repeat_interleave(64, dim=1) + q[0].double() * s[0].double().repeat_interleave(64, dim=1)
    assert torch.equal(m, want)


def test_affine_scale_and_bias_not_interchangeable():
    # s = 2, b = 3: code 5 decodes to 13 (not 3 * 5 + 2 = 17)
    H, I = 128, 64
    gu = (torch.full((1, 2 * I, H), 5), bf16(torch.full((1, 2 * I, H // 64), 2.0)),
          bf16(torch.full((1, 2 * I, H // 64), 3.0)))
    dn = (torch.full((1, H, I), 5), bf16(torch.full((1, H, I // 64), 2.0)), bf16(torch.full((1, H, I // 64), 3.0)))
    ex = orc.Experts(_affine(H, I, gu, dn), 1, H, I)
    assert (orc.expert_matrix(ex, 0, 0) == 13.0).all() and (orc.expert_matrix(ex, 0, 1) == 13.0).all()


# --------------------------------------------------------------------------
# NVFP4 matrices: e2m1(q) * e4m3(s) * g, 16-input groups, one g per matrix.
# --------------------------------------------------------------------------

def _e4m3(v):
    return torch.as_tensor(v, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)


def _nvfp4(gu, dn, g_gu, g_d):
    return {"fmt": "nvfp4", "q_gate_up": _pack(gu[0]), "s_gate_up": gu[1], "q_down": _pack(dn[0]),
            "s_down": dn[1], "g_gate_up": g_gu, "g_down": g_d}


def _nv_noise(N, K, g):
    return (torch.randint(0, 16, (1, N, K), generator=g),
            _e4m3(torch.rand(1, N, K // 16, generator=g) * 2.5 + 1.5))


@pytest.mark.parametrize("which", [0, 1])
def test_nvfp4_unit_scales_give_the_e2m1_values(which):
    H, I = 128, 64
    g = torch.Generator().manual_seed(33)
    N, K = (2 * I, H) if which == 0 else (H, I)
    q = torch.randint(0, 16, (1, N, K), generator=g)
    plain = (q, _e4m3(torch.ones(1, N, K // 16)))
    other = _nv_noise(H if which == 0 else 2 * I, I if which == 0 else H, g)
    ones2, ones1 = torch.ones(1, 2), torch.ones(1)
    ex = orc.Experts(_nvfp4(plain, other, ones2, ones1) if which == 0 else _nvfp4(other, plain, ones2, ones1),
                     1, H, I)
    table = torch.tensor([(-1.0 if c & 8 else 1.0) * E2M1[c & 7] for c in range(16)], dtype=torch.float64)
    assert torch.equal(orc.expert_matrix(ex, 0, which), table[q[0]])


def test_nvfp4_block_scales_are_16_wide_and_matrix_scales_apply():
    # code 2 (= 1.0) everywhere; a different power-of-two block scale per 16
    # inputs; gate, up and down matrix scales 0.5, 4 and 0.25
    H, I = 128, 64
    nb_gu, nb_d = H // 16, I // 16
    sg = 2.0 ** torch.arange(-3, nb_gu - 3, dtype=torch.float32)
    sd = 2.0 ** torch.arange(-2, nb_d - 2, dtype=torch.float32)
    gu = (torch.full((1, 2 * I, H), 2), _e4m3(sg.repeat(2 * I, 1)[None]))
    dn = (torch.full((1, H, I), 2), _e4m3(sd.repeat(H, 1)[None]))
    ex = orc.Experts(_nvfp4(gu, dn, torch.tensor([[0.5, 4.0]]), torch.tensor([0.25])), 1, H, I)
    m = orc.expert_matrix(ex, 0, 0)
    assert torch.equal(m[:I], (0.5 * sg.double().repeat_interleave(16)).repeat(I, 1))
    assert torch.equal(m[I:], (4.0 * sg.double().repeat_interleave(16)).repeat(I, 1))
    assert torch.equal(orc.expert_matrix(ex, 0, 1), (0.25 * sd.double().repeat_interleave(16)).repeat(H, 1))


# --------------------------------------------------------------------------
# The expert FFN through both matrices, one-hot rows (closed form).
# --------------------------------------------------------------------------

def _onehot_codes(N, K, pick, base, top):
    q = torch.full((N, K), base)
    q[torch.arange(N), pick] = top
    return q[None]


@pytest.mark.parametrize("fmt", ["affine4", "nvfp4"])
def test_expert_ffn_closed_form_one_hot_rows(fmt):
    # gate row i = a e_{pg[i]}, up row i = b e_{pu[i]}, down row c =
    # d e_{sigma[c]}: y[c] = d silu(a x[pg[s]]) b x[pu[s]], s = sigma[c]
    H, I = 256, 64
    g = torch.Generator().manual_seed(34)
    pg, pu = torch.randint(0, H, (I,), generator=g), torch.randint(0, H, (I,), generator=g)
    sigma = torch.randint(0, I, (H,), generator=g)
    x = bf16(torch.randn(H, generator=g)).double()
    if fmt == "affine4":
        # codes 0 with bias 0 give 0; the picked input has code 1: weight = s
        sc = bf16(torch.rand(2 * I + H, generator=g) * 0.75 + 0.25).float()
        gu = (_onehot_codes(2 * I, H, torch.cat([pg, pu]), 0, 1),
              bf16(sc[:2 * I, None].repeat(1, H // 64)[None]), bf16(torch.zeros(1, 2 * I, H // 64)))
        dn = (_onehot_codes(H, I, sigma, 0, 1), bf16(sc[2 * I:, None].repeat(1, I // 64)[None]),
              bf16(torch.zeros(1, H, I // 64)))
        ex = orc.Experts(_affine(H, I, gu, dn), 1, H, I)
        a_, b_, d_ = sc[:I].double(), sc[I:2 * I].double(), sc[2 * I:].double()
    else:
        # code 0 is +0; the picked input has code 4 (= 2.0) with block scale
        # 1.5 and matrix scales 0.5 (gate), 0.25 (up), 2 (down)
        gu = (_onehot_codes(2 * I, H, torch.cat([pg, pu]), 0, 4), _e4m3(torch.full((1, 2 * I, H // 16), 1.5)))
        dn = (_onehot_codes(H, I, sigma, 0, 4), _e4m3(torch.full((1, H, I // 16), 1.5)))
        ex = orc.Experts(_nvfp4(gu, dn, torch.tensor([[0.5, 0.25]]), torch.tensor([2.0])), 1, H, I)
        a_ = torch.full((I,), 3.0 * 0.5, dtype=torch.float64)
        b_ = torch.full((I,), 3.0 * 0.25, dtype=torch.float64)
        d_ = torch.full((H,), 3.0 * 2.0, dtype=torch.float64)
    y = orc.expert_ffn(x, ex, 0)
    for c in range(H):
        s_ = int(sigma[c])
        gate = float(a_[s_]) * float(x[pg[s_]])
        up = float(b_[s_]) * float(x[pu[s_]])
        ref = float(d_[c]) * gate / (1.0 + math.exp(-gate)) * up
        assert y[c].item() == pytest.approx(ref, rel=1e-14, abs=1e-300)


@pytest.mark.parametrize("fmt", ["affine4", "nvfp4"])
def test_full_band_is_the_monolith(fmt):
    w = synth.Workload("fmt", T=6, H=256, E=8, topk=2, I=128, Is=64, fmt=fmt)
    d = synth.make_inputs(w, "cpu")
    full, _, _ = orc.moe_ffn(d, w.E, w.I, w.Is, 0, w.E, w.topk)
    mono = orc.moe_ffn_monolith(d, w.E, w.I, w.Is, w.topk)
    assert torch.equal(full, mono)
