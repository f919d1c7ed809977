"""GPU tests of cp_attn_merge: agreement with the oracle's combine, identity,
bit-exact commutativity and associativity within fp32 rounding."""
import math

import numpy as np
import pytest
import torch

import oracle as orc
import context_causal_attention_amd as cpa
from gpu_cases import announce

pytestmark = pytest.mark.gpu


def _operands(rows, d, seed, empty_frac=0.1):
    g = torch.Generator().manual_seed(seed)
    o = torch.randn(rows, d, generator=g)
    l = torch.randn(rows, generator=g) * 4
    e = torch.rand(rows, generator=g) < empty_frac
    o[e] = 0
    l[e] = -math.inf
    return o, l


@pytest.mark.parametrize("rows,d", [(1, 64), (1000, 128), (4099, 64)])
def test_merge_matches_oracle(rows, d):
    announce(f"merge rows={rows} d={d}")
    o1, l1 = _operands(rows, d, 1)
    o2, l2 = _operands(rows, d, 2)
    oa, la = o1.cuda(), l1.cuda()
    cpa.cp_attn_merge(oa, la, o2.cuda(), l2.cuda())
    O, L = orc.lse_merge(o1.double().numpy(), l1.double().numpy(), o2.double().numpy(), l2.double().numpy())
    got_l = la.double().cpu().numpy()
    fin = np.isfinite(L)
    assert np.array_equal(np.isneginf(got_l), np.isneginf(L))
    assert np.abs(got_l[fin] - L[fin]).max() <= 1e-5
    assert np.abs(oa.double().cpu().numpy() - O).max() <= 1e-5


def test_merge_identity_and_empty():
    o1, l1 = _operands(256, 128, 3, empty_frac=0)
    oa, la = o1.cuda(), l1.cuda()
    cpa.cp_attn_merge(oa, la, torch.zeros(256, 128, device="cuda"), torch.full((256,), -math.inf, device="cuda"))
    assert torch.allclose(oa.cpu(), o1, atol=1e-6, rtol=1e-6) and torch.allclose(la.cpu(), l1, atol=1e-6)
    z, zl = torch.zeros(8, 64, device="cuda"), torch.full((8,), -math.inf, device="cuda")
    cpa.cp_attn_merge(z, zl, torch.zeros(8, 64, device="cuda"), torch.full((8,), -math.inf, device="cuda"))
    assert torch.all(z == 0) and torch.all(torch.isneginf(zl))


def test_merge_commutative_bit_exact_and_associative():
    ops = [_operands(2048, 128, s) for s in (4, 5, 6)]
    a = [(o.cuda(), l.cuda()) for o, l in ops]

    def merged(x, y):
        o, l = x[0].clone(), x[1].clone()
        cpa.cp_attn_merge(o, l, y[0], y[1])
        return o, l

    ab, ba = merged(a[0], a[1]), merged(a[1], a[0])
    assert torch.equal(ab[0], ba[0]) and torch.equal(ab[1], ba[1])
    left = merged(merged(a[0], a[1]), a[2])
    right = merged(a[0], merged(a[1], a[2]))
    fin = torch.isfinite(left[1])
    assert torch.equal(torch.isneginf(left[1]), torch.isneginf(right[1]))
    assert (left[1][fin] - right[1][fin]).abs().max() <= 1e-5
    rel = (left[0] - right[0]).abs().max() / left[0].abs().max()
    assert rel <= 1e-6
