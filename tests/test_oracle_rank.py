"""Pins for the oracle's rank-order merge of rank partials.

[P4] "GLM-5.3-Flash on CUDA over three ranks (--tp 3) ... #310": each rank
returns a full-width fp32 partial and the partials are added in rank order;
the shared expert's output comes after them and the residual last.  The pins
fix the order with values where fp32 addition is not associative (so any
other order gives another number), the identities of a single part, exact
integer sums, and the widening of the bf16 residual.
"""

import numpy as np
import torch

from oracle import oracle as orc


def _t(v):
    return torch.tensor(v, dtype=torch.float32)


def test_left_fold_order():
    # ulp(2^27) = 16: (2^27 + 1) rounds back to 2^27, then - 2^27 gives 0;
    # any order that pairs 2^27 with -2^27 first gives 1
    a, b, c = _t([2.0 ** 27]), _t([1.0]), _t([-(2.0 ** 27)])
    assert orc.rank_merge([a, b, c]).item() == 0.0
    assert orc.rank_merge([a, c, b]).item() == 1.0
    assert orc.rank_merge([b, a, c]).item() == 0.0  # (1 + 2^27) rounds to 2^27 as well


def test_ties_to_even_inside_the_fold():
    # 2^24 + 1 is a tie between 2^24 and 2^24 + 2: to even (2^24); a second
    # + 1 from there is again a tie: 2^24 stays
    x = _t([2.0 ** 24])
    one = _t([1.0])
    assert orc.rank_merge([x, one, one]).item() == 2.0 ** 24
    # 1 + 1 first (exact), then + 2^24: 2^24 + 2 exactly
    assert orc.rank_merge([one, one, x]).item() == 2.0 ** 24 + 2


def test_shared_after_the_parts_and_residual_last():
    big = _t([2.0 ** 27])
    sh = _t([1.0])
    res = torch.tensor([-(2.0 ** 27)], dtype=torch.bfloat16)  # exact in bf16
    # ((2^27) + 1) + (-2^27) = 0; residual before the shared output would give 1
    assert orc.rank_merge([big], shared=sh, residual=res).item() == 0.0
    # the shared output after all parts: (2^27 + (-2^27)) + 1 = 1
    assert orc.rank_merge([big, _t([-(2.0 ** 27)])], shared=sh).item() == 1.0


def test_single_part_is_the_identity_and_integers_are_exact():
    g = torch.Generator().manual_seed(0)
    p = torch.randn(4, 33, generator=g)
    assert torch.equal(orc.rank_merge([p]), p)
    ints = [torch.randint(-1000, 1000, (3, 17), generator=g).float() for _ in range(6)]
    want = sum(t.double() for t in ints)
    assert torch.equal(orc.rank_merge(ints).double(), want)


def test_residual_widened_exactly():
    # every bf16 value widens to the fp32 with the same bits followed by 16 zeros
    bits = torch.arange(0, 1 << 16, 97, dtype=torch.int32)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF].to(torch.int16)  # finite values
    res = bits.view(torch.bfloat16)
    zero = torch.zeros(res.shape)
    out = orc.rank_merge([zero], residual=res)
    want = (bits.to(torch.int32) & 0xFFFF) << 16
    got = out.view(torch.int32)
    # 0 + x = x for every x except -0 (+0 + -0 = +0)
    neg0 = want == np.int32(-(2 ** 31))
    assert torch.equal(got[~neg0], want[~neg0])
    assert (got[neg0] == 0).all()
