"""Pins for the fp64 oracle: each checks it against something other than itself
(brute-force scalar loops, closed forms, torch fp64 library routines and
autograd, finite differences, the pages' figures).  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as orc
import seeded_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- brute force
def _brute_forward(q, k, v, scale, cu=None, causal=True):
    """Scalar loops with math.exp / math.fsum; independent of numpy's BLAS."""
    B, Hq, S, d = q.shape
    g = Hq // k.shape[1]
    bounds = [0, S] if cu is None else list(cu)
    O = np.zeros_like(q)
    L = np.zeros(q.shape[:3])
    for b in range(B):
        for h in range(Hq):
            kh = h // g
            for i in range(S):
                doc = max(t for t in range(len(bounds) - 1) if bounds[t] <= i)
                lo, hi = bounds[doc], bounds[doc + 1]
                js = range(lo, i + 1) if causal else range(lo, hi)
                s = [scale * math.fsum(q[b, h, i, t] * k[b, kh, j, t] for t in range(d)) for j in js]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                Z = math.fsum(e)
                for t in range(d):
                    O[b, h, i, t] = math.fsum(e[n] * v[b, kh, j, t] for n, j in enumerate(js)) / Z
                L[b, h, i] = m + math.log(Z)
    return O, L


@pytest.mark.parametrize("cu", [None, [0, 5, 13, 24], [0, 1, 2, 24]])
@pytest.mark.parametrize("causal", [True, False])
def test_forward_matches_brute_force(cu, causal):
    B, Hq, Hkv, S, d = 1, 4, 2, 24, 6
    q, k, v = _rand((B, Hq, S, d), 1), _rand((B, Hkv, S, d), 2), _rand((B, Hkv, S, d), 3)
    scale = 0.37
    O, L = orc.attention_fwd(q, k, v, scale, cu_seqlens=cu, causal=causal, row_block=7)
    Ob, Lb = _brute_forward(q, k, v, scale, cu, causal)
    assert np.abs(O - Ob).max() < 1e-12
    assert np.abs(L - Lb).max() < 1e-12


def test_row_subset_equals_full_rows():
    B, Hq, Hkv, S, d = 2, 2, 1, 40, 5
    q, k, v = _rand((B, Hq, S, d), 4), _rand((B, Hkv, S, d), 5), _rand((B, Hkv, S, d), 6)
    rows = np.array([39, 0, 17, 3, 22])
    O, L = orc.attention_fwd(q, k, v, 0.5)
    Os, Ls = orc.attention_fwd(q, k, v, 0.5, rows=rows)
    assert np.array_equal(Os, O[:, :, rows]) or np.abs(Os - O[:, :, rows]).max() < 1e-13
    assert np.abs(Ls - L[:, :, rows]).max() < 1e-13


# ---------------------------------------------------------------- closed forms
def test_zero_query_gives_prefix_mean_and_log_count():
    S, d = 50, 7
    cu = [0, 9, 30, 50]
    q = np.zeros((1, 1, S, d))
    k, v = _rand((1, 1, S, d), 7), _rand((1, 1, S, d), 8)
    O, L = orc.attention_fwd(q, k, v, 0.3, cu_seqlens=cu)
    for i in range(S):
        lo = max(c for c in cu[:-1] if c <= i)
        assert np.allclose(O[0, 0, i], v[0, 0, lo:i + 1].mean(axis=0), atol=1e-14, rtol=0)
        assert abs(L[0, 0, i] - math.log(i - lo + 1)) < 1e-14


def test_document_start_row_sees_only_itself():
    S, d = 40, 4
    cu = [0, 11, 12, 40]
    q, k, v = _rand((1, 1, S, d), 9), _rand((1, 1, S, d), 10), _rand((1, 1, S, d), 11)
    O, L = orc.attention_fwd(q, k, v, 0.9, cu_seqlens=cu)
    for i in cu[:-1]:
        assert np.abs(O[0, 0, i] - v[0, 0, i]).max() < 1e-15
        assert abs(L[0, 0, i] - 0.9 * float(q[0, 0, i] @ k[0, 0, i])) < 1e-14


def test_identical_keys_give_prefix_mean():
    S, d = 30, 5
    q, v = _rand((1, 1, S, d), 12), _rand((1, 1, S, d), 13)
    k = np.broadcast_to(_rand((1, 1, 1, d), 14), (1, 1, S, d)).copy()
    O, L = orc.attention_fwd(q, k, v, 1.1)
    for i in range(S):
        assert np.abs(O[0, 0, i] - v[0, 0, :i + 1].mean(axis=0)).max() < 1e-13
        assert abs(L[0, 0, i] - (1.1 * float(q[0, 0, i] @ k[0, 0, 0]) + math.log(i + 1))) < 1e-12


def test_common_key_offset_shifts_lse_only():
    S, d = 33, 6
    q, k, v = _rand((1, 2, S, d), 15), _rand((1, 1, S, d), 16), _rand((1, 1, S, d), 17)
    u = _rand((d,), 18)
    O1, L1 = orc.attention_fwd(q, k, v, 0.6)
    O2, L2 = orc.attention_fwd(q, k + u, v, 0.6)
    assert np.abs(O1 - O2).max() < 1e-12
    shift = 0.6 * (q @ u)
    assert np.abs(L2 - L1 - shift).max() < 1e-12


def test_worked_example_linear_weights():
    """scale 1, q_i = (1, 0), k_j = (ln(j+1), 0): the weights are (j+1)/T_i with
    T_i = (i+1)(i+2)/2, so O_i = sum (j+1) v_j / T_i and LSE_i = ln T_i."""
    S = 20
    q = np.zeros((1, 1, S, 2))
    q[..., 0] = 1.0
    k = np.zeros((1, 1, S, 2))
    k[0, 0, :, 0] = np.log(np.arange(1, S + 1))
    v = _rand((1, 1, S, 2), 19)
    O, L = orc.attention_fwd(q, k, v, 1.0)
    for i in range(S):
        T = (i + 1) * (i + 2) / 2
        w = np.arange(1, i + 2) / T
        assert np.abs(O[0, 0, i] - w @ v[0, 0, :i + 1]).max() < 1e-14
        assert abs(L[0, 0, i] - math.log(T)) < 1e-13


# ---------------------------------------------------------------- library routines
def _torch_mask(S, cu, causal=True):
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    if cu is None:
        same = torch.ones(S, S, dtype=torch.bool)
    else:
        doc = torch.bucketize(torch.arange(S), torch.tensor(cu[1:-1]), right=True)
        same = doc[:, None] == doc[None, :]
    return same & (j <= i) if causal else same


@pytest.mark.parametrize("cu", [None, [0, 17, 40, 41, 96]])
def test_forward_matches_torch_sdpa_fp64(cu):
    B, Hq, Hkv, S, d = 2, 8, 2, 96, 16
    q, k, v = _rand((B, Hq, S, d), 20), _rand((B, Hkv, S, d), 21), _rand((B, Hkv, S, d), 22)
    scale = 1 / math.sqrt(d)
    O, L = orc.attention_fwd(q, k, v, scale, cu_seqlens=cu, row_block=33)
    g = Hq // Hkv
    tq = torch.from_numpy(q)
    tk = torch.from_numpy(k).repeat_interleave(g, dim=1)
    tv = torch.from_numpy(v).repeat_interleave(g, dim=1)
    mask = _torch_mask(S, cu)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    sc = (tq @ tk.transpose(-1, -2)) * scale
    lse = torch.logsumexp(sc.masked_fill(~mask, -math.inf), dim=-1)
    assert np.abs(O - ref.numpy()).max() < 1e-12
    assert np.abs(L - lse.numpy()).max() < 1e-12


def test_noncausal_single_document_is_plain_softmax():
    from scipy.special import softmax, logsumexp
    S, d = 64, 8
    q, k, v = _rand((1, 1, S, d), 23), _rand((1, 1, S, d), 24), _rand((1, 1, S, d), 25)
    O, L = orc.attention_fwd(q, k, v, 0.25, cu_seqlens=[0, S], causal=False)
    s = 0.25 * q[0, 0] @ k[0, 0].T
    assert np.abs(O[0, 0] - softmax(s, axis=1) @ v[0, 0]).max() < 1e-12
    assert np.abs(L[0, 0] - logsumexp(s, axis=1)).max() < 1e-12


# ---------------------------------------------------------------- backward
def _torch_attention(q, k, v, scale, mask, g):
    k = k.repeat_interleave(g, dim=1)
    v = v.repeat_interleave(g, dim=1)
    s = (q @ k.transpose(-1, -2)) * scale
    s = s.masked_fill(~mask, -math.inf)
    return torch.softmax(s, dim=-1) @ v


@pytest.mark.parametrize("cu", [None, [0, 6, 19, 40]])
def test_backward_matches_torch_autograd(cu):
    B, Hq, Hkv, S, d = 1, 4, 2, 40, 8
    q, k, v, do = (_rand((B, Hq, S, d), 26), _rand((B, Hkv, S, d), 27),
                   _rand((B, Hkv, S, d), 28), _rand((B, Hq, S, d), 29))
    scale = 0.31
    dq, dk, dv = orc.attention_bwd(q, k, v, do, scale, cu_seqlens=cu, row_block=13)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = _torch_attention(tq, tk, tv, scale, _torch_mask(S, cu), Hq // Hkv)
    (out * torch.from_numpy(do)).sum().backward()
    assert np.abs(dq - tq.grad.numpy()).max() < 1e-10
    assert np.abs(dk - tk.grad.numpy()).max() < 1e-10
    assert np.abs(dv - tv.grad.numpy()).max() < 1e-10


def test_backward_row_subset_is_zeroed_upstream_gradient():
    B, Hq, Hkv, S, d = 1, 2, 1, 32, 4
    q, k, v, do = (_rand((B, Hq, S, d), 30), _rand((B, Hkv, S, d), 31),
                   _rand((B, Hkv, S, d), 32), _rand((B, Hq, S, d), 33))
    rows = np.array([3, 31, 10, 11, 0])
    dq_s, dk_s, dv_s = orc.attention_bwd(q, k, v, do[:, :, rows], 0.5, rows=rows)
    dz = np.zeros_like(do)
    dz[:, :, rows] = do[:, :, rows]
    dq, dk, dv = orc.attention_bwd(q, k, v, dz, 0.5)
    assert np.abs(dq_s - dq[:, :, rows]).max() < 1e-13
    assert np.abs(dk_s - dk).max() < 1e-13
    assert np.abs(dv_s - dv).max() < 1e-13


def test_backward_matches_central_differences():
    B, Hq, Hkv, S, d = 1, 2, 1, 12, 3
    cu = [0, 5, 12]
    q, k, v, do = (_rand((B, Hq, S, d), 34), _rand((B, Hkv, S, d), 35),
                   _rand((B, Hkv, S, d), 36), _rand((B, Hq, S, d), 37))
    scale = 0.8
    dq, dk, dv = orc.attention_bwd(q, k, v, do, scale, cu_seqlens=cu)

    def f(q_, k_, v_):
        O, _ = orc.attention_fwd(q_, k_, v_, scale, cu_seqlens=cu)
        return float((O * do).sum())

    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        dirn = _rand(grad.shape, 40 + which)
        args_p = [q, k, v]
        args_m = [q, k, v]
        args_p[which] = args_p[which] + h * dirn
        args_m[which] = args_m[which] - h * dirn
        fd = (f(*args_p) - f(*args_m)) / (2 * h)
        an = float((grad * dirn).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an))


def test_delta_is_rowwise_dot():
    do, o = _rand((2, 3, 5, 4), 41), _rand((2, 3, 5, 4), 42)
    dl = orc.bwd_delta(do, o)
    for idx in np.ndindex(2, 3, 5):
        assert abs(dl[idx] - math.fsum(do[idx] * o[idx])) < 1e-14


def test_partial_bwd_single_step_over_all_keys_is_attention_bwd():
    """One step holding every key, with the full attention's LSE and delta,
    is the whole causal backward (documents included)."""
    B, Hq, Hkv, S, d = 1, 4, 2, 30, 5
    cu = [0, 11, 30]
    q, k, v, do = (_rand((B, Hq, S, d), 50), _rand((B, Hkv, S, d), 51),
                   _rand((B, Hkv, S, d), 52), _rand((B, Hq, S, d), 53))
    scale = 0.45
    pos = np.arange(S)
    lo = orc.doc_start_of(pos, cu)
    O, L = orc.attention_fwd(q, k, v, scale, cu_seqlens=cu)
    got = orc.partial_attention_bwd(q, k, v, do, L, orc.bwd_delta(do, O), scale, pos, lo, pos)
    ref = orc.attention_bwd(q, k, v, do, scale, cu_seqlens=cu)
    for a, b_ in zip(got, ref):
        assert np.abs(a - b_).max() < 1e-12


def test_partial_bwd_ring_steps_sum_to_attention_bwd():
    """Per rank and ring step, with the merged LSE and delta: dQ of a rank is
    the sum over its steps, dK/dV the sum over every rank and step."""
    B, Hq, Hkv, S, d, cp = 1, 2, 1, 24, 4, 3
    q, k, v, do = (_rand((B, Hq, S, d), 54), _rand((B, Hkv, S, d), 55),
                   _rand((B, Hkv, S, d), 56), _rand((B, Hq, S, d), 57))
    scale = 0.6
    O, L = orc.attention_fwd(q, k, v, scale)
    dl = orc.bwd_delta(do, O)
    dq_ref, dk_ref, dv_ref = orc.attention_bwd(q, k, v, do, scale)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for rank in range(cp):
        rows = orc.zigzag_positions(S, cp, rank)
        dq = np.zeros((B, Hq, len(rows), d))
        for src in range(cp):
            keys = orc.zigzag_positions(S, cp, src)
            a, b_, c = orc.partial_attention_bwd(q[:, :, rows], k[:, :, keys], v[:, :, keys], do[:, :, rows],
                                                 L[:, :, rows], dl[:, :, rows], scale, rows, np.zeros_like(rows),
                                                 keys)
            dq += a
            dk[:, :, keys] += b_
            dv[:, :, keys] += c
        assert np.abs(dq - dq_ref[:, :, rows]).max() < 1e-12
    assert np.abs(dk - dk_ref).max() < 1e-12
    assert np.abs(dv - dv_ref).max() < 1e-12


def test_partial_bwd_own_step_matches_central_differences():
    """With the step's own LSE and delta the result is the gradient of that
    step's attention output alone, rows without any allowed key included
    (their output is the constant 0)."""
    B, Hq, Hkv, d = 1, 2, 1, 3
    q_pos = np.array([2, 9, 10, 15, 4])      # rows 0 and 4 see no key of the step
    q_lo = np.array([0, 0, 8, 8, 0])
    k_pos = np.array([8, 9, 10, 11, 12, 13])
    nq, nk = len(q_pos), len(k_pos)
    q, k, v, do = (_rand((B, Hq, nq, d), 58), _rand((B, Hkv, nk, d), 59),
                   _rand((B, Hkv, nk, d), 60), _rand((B, Hq, nq, d), 61))
    scale = 0.7
    O, L = orc.partial_attention_fwd(q, k, v, scale, q_pos, q_lo, k_pos)
    assert np.isneginf(L[0, :, 0]).all() and np.isneginf(L[0, :, 4]).all()
    dq, dk, dv = orc.partial_attention_bwd(q, k, v, do, L, orc.bwd_delta(do, O), scale, q_pos, q_lo, k_pos)
    assert np.all(dq[0, :, 0] == 0) and np.all(dq[0, :, 4] == 0)

    def f(q_, k_, v_):
        O_, _ = orc.partial_attention_fwd(q_, k_, v_, scale, q_pos, q_lo, k_pos)
        return float((O_ * do).sum())

    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        dirn = _rand(grad.shape, 62 + which)
        args_p = [q, k, v]
        args_m = [q, k, v]
        args_p[which] = args_p[which] + h * dirn
        args_m[which] = args_m[which] - h * dirn
        fd = (f(*args_p) - f(*args_m)) / (2 * h)
        an = float((grad * dirn).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an))


# ---------------------------------------------------------------- per-document zigzag
def test_per_doc_positions_worked_example():
    """Documents of 8 and 4 tokens (S = 12), cp = 2, so 2cp = 4 chunks per
    document: 2-token chunks of [0, 8) and 1-token chunks of [8, 12).  Rank 0
    takes chunks 0 and 3 of each: {0, 1, 6, 7} then {8, 11}; rank 1 chunks 1
    and 2: {2, 3, 4, 5} then {9, 10}."""
    assert orc.per_doc_positions([0, 8, 12], 2, 0).tolist() == [0, 1, 6, 7, 8, 11]
    assert orc.per_doc_positions([0, 8, 12], 2, 1).tolist() == [2, 3, 4, 5, 9, 10]
    with pytest.raises(ValueError, match="multiple of 2"):
        orc.per_doc_positions([0, 6, 16], 2, 0)


@pytest.mark.parametrize("cp,seed", [(2, 1), (4, 2), (8, 3)])
def test_per_doc_positions_balance(cp, seed):
    """Every position on exactly one rank; within each document a rank holds
    2/(2cp) of its tokens; and every rank gets the same number of causal
    pairs inside documents: a document of n = 2cp*c tokens gives each rank
    (2cp*c^2 + c) pairs, the dense zigzag identity applied per document."""
    L = si.round_doc_lengths(si.doc_lengths(total=2 * cp * 600, mean=300, sigma=1.0, lo=8, hi=2500, seed=seed),
                             2 * cp)
    cu = si.cu_seqlens_from_lengths(L)
    S = int(cu[-1])
    parts = [orc.per_doc_positions(cu, cp, r) for r in range(cp)]
    assert np.array_equal(np.sort(np.concatenate(parts)), np.arange(S))
    expect = sum((n // (2 * cp)) * (2 * cp * (n // (2 * cp)) + 1) for n in L)
    for p in parts:
        assert orc.pair_count(p, orc.doc_start_of(p, cu), np.arange(S)) == expect
        for a, b in zip(cu[:-1], cu[1:]):
            assert np.sum((p >= a) & (p < b)) == (b - a) // cp


# ---------------------------------------------------------------- whole-document placement
def test_whole_doc_deal_worked_example():
    """Documents of 7, 2, 1, 2 tokens (S = 12), cp = 3, room 4 per rank.
    Longest first: the 7-token document fits nowhere whole, so it is cut: [0,4)
    fills rank 0 (most room, lowest rank), [4,7) goes to rank 1 (room 4 > 4 - 0).
    The 2-token document [7,9) fits only rank 2 (rank 1 has 1 left); the other
    2-token document [10,12) fits only rank 2 as well (room 2); the 1-token
    document [9,10) fits only rank 1."""
    got = orc.whole_doc_deal([0, 7, 9, 10, 12], 3)
    assert [g.tolist() for g in got] == [[0, 1, 2, 3], [4, 5, 6, 9], [7, 8, 10, 11]]


def test_whole_doc_deal_least_loaded_rank_wins():
    """Lengths 4, 3, 3, 2 (S = 12), cp = 2, room 6: the 4-token document goes to
    rank 0 (tie, lower rank; work 10), the first 3-token one to rank 1 (work 0 <
    10; gets 6), the second 3-token one fits only rank 1 (room 3), the 2-token
    one only rank 0."""
    got = orc.whole_doc_deal([0, 4, 7, 10, 12], 2)
    assert [g.tolist() for g in got] == [[0, 1, 2, 3, 10, 11], [4, 5, 6, 7, 8, 9]]


def test_causal_piece_work_closed_form():
    for s, n in ((0, 1), (5, 7), (100, 33)):
        assert orc.causal_piece_work(s, s, s + n) == n * (n + 1) // 2
        for cut in range(s, s + n + 1):
            assert orc.causal_piece_work(s, s, cut) + orc.causal_piece_work(s, cut, s + n) == n * (n + 1) // 2


@pytest.mark.parametrize("cp,seed", [(2, 1), (4, 2), (8, 3), (3, 4)])
def test_whole_doc_deal_properties(cp, seed):
    """Every position on exactly one rank, S/cp positions per rank; at most
    cp - 1 documents are cut (a document is cut only when it is longer than
    every rank's room, so its first piece fills a rank completely, and once a
    single rank has room every remaining document fits it); the per-rank
    causal work counted by the pair counter equals the work of the pieces."""
    total = 2 * cp * 1000
    L = si.doc_lengths(total=total, mean=300, sigma=1.0, lo=8, hi=2500, seed=seed)
    cu = si.cu_seqlens_from_lengths(L)
    parts = orc.whole_doc_deal(cu, cp)
    allpos = np.concatenate(parts)
    assert np.array_equal(np.sort(allpos), np.arange(total))
    assert all(len(p) == total // cp for p in parts)
    owner = np.empty(total, dtype=np.int64)
    for r, p in enumerate(parts):
        owner[p] = r
    whole = sum(1 for i in range(len(L)) if L[i] > 0 and len(set(owner[cu[i]:cu[i + 1]])) == 1)
    assert whole >= len(L) - (cp - 1)
    for p in parts:
        lo = orc.doc_start_of(p, cu)
        work = orc.pair_count(p, lo, allpos)
        assert work == sum(orc.causal_piece_work(int(l), int(x), int(x) + 1) for x, l in zip(p, lo))


# ---------------------------------------------------------------- all-to-all head exchange
def test_a2a_small_example_by_hand():
    """rows = 2, H = 4, d = 1, g = 2, x[t, h] = 10 t + h."""
    x = np.array([[[0], [1], [2], [3]], [[10], [11], [12], [13]]])
    send = orc.a2a_pack(x, 2)
    assert send[:, :, :, 0].tolist() == [[[0, 10], [1, 11]], [[2, 12], [3, 13]]]
    y = orc.a2a_unpack(send)
    assert y[:, :, 0].tolist() == [[0, 10, 2, 12], [1, 11, 3, 13]]


@pytest.mark.parametrize("g,H,rows,d", [(2, 4, 3, 2), (4, 8, 5, 3), (1, 3, 4, 2), (8, 32, 2, 4)])
def test_a2a_exchange_is_a_global_transpose(g, H, rows, d):
    """The sequence-sharded tensor X [S, H, d] (rank i holds rows i*rows..),
    packed, exchanged and unpacked, leaves on rank j exactly heads j*H/g.. of
    X for all S rows, head-major: the block of numpy's transpose of X."""
    rng = np.random.default_rng(70 + g)
    S = g * rows
    X = rng.integers(-1000, 1000, (S, H, d))
    sends = [orc.a2a_pack(X[i * rows:(i + 1) * rows], g) for i in range(g)]
    recvs = orc.a2a_exchange(sends)
    Hg = H // g
    XT = np.transpose(X, (1, 0, 2))
    for j in range(g):
        y = orc.a2a_unpack(recvs[j])
        assert np.array_equal(y, XT[j * Hg:(j + 1) * Hg])
        # the reverse direction restores each rank's shard
        back = orc.a2a_exchange([orc.a2a_pack_unpack(orc.a2a_unpack(recvs[jj]), g) for jj in range(g)])
        for i in range(g):
            assert np.array_equal(orc.a2a_unpack_pack(back[i]), X[i * rows:(i + 1) * rows])


def test_a2a_inverses_round_trip():
    rng = np.random.default_rng(71)
    x = rng.standard_normal((7, 12, 5))
    for g in (1, 2, 3, 4, 6, 12):
        assert np.array_equal(orc.a2a_unpack_pack(orc.a2a_pack(x, g)), x)
        r = rng.standard_normal((g, 12 // g, 7, 5))
        assert np.array_equal(orc.a2a_pack_unpack(orc.a2a_unpack(r), g), r)


# ---------------------------------------------------------------- sharding, merge
def test_zigzag_positions_are_a_permutation_and_cp1_is_identity():
    for S, cp in [(1024, 2), (64, 8), (48, 3), (32768, 8)]:
        allp = orc.all_rank_positions(S, cp)
        assert np.array_equal(np.sort(allp), np.arange(S))
    assert np.array_equal(orc.zigzag_positions(64, 1, 0), np.arange(64))
    # rank r holds chunk r then chunk 2cp-1-r (two contiguous runs of S/(2cp))
    p = orc.zigzag_positions(32, 4, 1)
    assert p.tolist() == [4, 5, 6, 7, 24, 25, 26, 27]


def test_seq_multiple_rule_from_pages():
    fig = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))["seq_multiple_of_2cp"]
    for S, cp in fig["valid"]:
        orc.zigzag_positions(S, cp, cp - 1)
    for S, cp in fig["invalid"]:
        with pytest.raises(ValueError):
            orc.zigzag_positions(S, cp, 0)


def test_pair_count_matches_mask_sum():
    rng = np.random.default_rng(43)
    for _ in range(20):
        qp = rng.integers(0, 200, 37)
        ql = np.minimum(qp, rng.integers(0, 200, 37))
        kp = rng.permutation(200)[:61]
        assert orc.pair_count(qp, ql, kp) == int(orc.allowed_mask(qp, ql, kp).sum())


@pytest.mark.parametrize("cp", list(range(1, 17)))
def test_zigzag_balance_closed_form(cp):
    """Every rank's unmasked pair count equals S(S+1)/(2cp): chunk pairs (i,j)
    give c^2 if j<i and c(c+1)/2 if j=i, so ranks holding chunks r and 2cp-1-r
    all get (2cp-1)c^2 + c^2 + c = S(S+1)/(2cp)."""
    for c in (1, 3, 8):
        S = 2 * cp * c
        kp = np.arange(S)
        want = S * (S + 1) // (2 * cp)
        for r in range(cp):
            pos = orc.zigzag_positions(S, cp, r)
            assert orc.pair_count(pos, np.zeros_like(pos), kp) == want


def test_balance_values_at_workload_sizes():
    for name, want in [("c0_f32_s1024_cp2", 262400), ("llama8b_s32k_cp8", 67110912),
                       ("llama8b_s128k_cp8", 1073750016)]:
        w = si.WORKLOADS[name]
        assert w.S * (w.S + 1) // (2 * w.cp) == want
        pos = orc.zigzag_positions(w.S, w.cp, w.cp - 1)
        assert orc.pair_count(pos, np.zeros_like(pos), np.arange(w.S)) == want


def test_attention_matrix_size_from_pages():
    fig = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))["attention_matrix_bytes"]
    got = orc.attention_matrix_bytes(fig["seq_len"], fig["num_heads"], fig["bytes_per_elem"])
    assert got == fig["bytes"] == 32 * 2 ** 30


def test_merge_identity_commutativity_associativity():
    rng = np.random.default_rng(44)
    o = [rng.standard_normal((6, 9, 5)) for _ in range(3)]
    l = [rng.standard_normal((6, 9)) * 3 for _ in range(3)]
    l[2][0, :] = -np.inf
    o[2][0, :] = 0.0
    e_o, e_l = np.zeros((6, 9, 5)), np.full((6, 9), -np.inf)
    Oi, Li = orc.lse_merge(o[0], l[0], e_o, e_l)
    assert np.abs(Oi - o[0]).max() < 1e-15 and np.abs(Li - l[0]).max() < 1e-15
    Oa, La = orc.lse_merge(o[0], l[0], o[1], l[1])
    Ob, Lb = orc.lse_merge(o[1], l[1], o[0], l[0])
    assert np.array_equal(Oa, Ob) and np.array_equal(La, Lb)
    O1, L1 = orc.lse_merge(*orc.lse_merge(o[0], l[0], o[1], l[1]), o[2], l[2])
    O2, L2 = orc.lse_merge(o[0], l[0], *orc.lse_merge(o[1], l[1], o[2], l[2]))
    assert np.abs(O1 - O2).max() < 1e-12 and np.abs(L1 - L2).max() < 1e-12
    Oe, Le = orc.lse_merge(e_o, e_l, e_o, e_l)
    assert np.all(Oe == 0) and np.all(np.isneginf(Le))


def test_merge_recovers_softmax_over_union():
    """Splitting a row's keys into two disjoint sets and merging the two partial
    softmaxes equals the softmax over all keys (checked with scipy)."""
    from scipy.special import softmax, logsumexp
    rng = np.random.default_rng(45)
    s = rng.standard_normal((4, 30)) * 2
    v = rng.standard_normal((30, 3))
    a, b = slice(0, 11), slice(11, 30)
    Oa, La = softmax(s[:, a], 1) @ v[a], logsumexp(s[:, a], 1)
    Ob, Lb = softmax(s[:, b], 1) @ v[b], logsumexp(s[:, b], 1)
    O, L = orc.lse_merge(Oa, La, Ob, Lb)
    assert np.abs(O - softmax(s, 1) @ v).max() < 1e-13
    assert np.abs(L - logsumexp(s, 1)).max() < 1e-13


def _sharded_vs_full(B, Hq, Hkv, S, d, cp, cu=None, seed=46):
    q, k, v = _rand((B, Hq, S, d), seed), _rand((B, Hkv, S, d), seed + 1), _rand((B, Hkv, S, d), seed + 2)
    scale = 1 / math.sqrt(d)
    allp = orc.all_rank_positions(S, cp)
    kall, vall = k[:, :, allp], v[:, :, allp]
    worst = 0.0
    for r in range(cp):
        pos = orc.zigzag_positions(S, cp, r)
        lo = orc.doc_start_of(pos, cu)
        O, L = orc.ring_partials_fwd(q[:, :, pos], kall, vall, scale, cp, r, pos, lo, allp)
        Of, Lf = orc.attention_fwd(q, k, v, scale, cu_seqlens=cu, rows=pos)
        worst = max(worst, np.abs(O - Of).max(), np.abs(L - Lf).max())
    return worst


def test_sharded_then_merged_equals_unsharded_c0_shape():
    assert _sharded_vs_full(1, 1, 1, 1024, 64, 2) < 1e-12


def test_sharded_then_merged_equals_unsharded_gqa_cp8():
    assert _sharded_vs_full(1, 4, 1, 2048, 32, 8) < 1e-12


def test_sharded_then_merged_equals_unsharded_varlen():
    L = si.doc_lengths(total=1536, mean=160, sigma=1.0, lo=8, hi=900, seed=3)
    cu = si.cu_seqlens_from_lengths(L)
    assert _sharded_vs_full(1, 2, 1, 1536, 16, 4, cu=cu) < 1e-12


def test_partial_empty_rows_are_merge_identity():
    q, k, v = _rand((1, 1, 4, 3), 47), _rand((1, 1, 5, 3), 48), _rand((1, 1, 5, 3), 49)
    O, L = orc.partial_attention_fwd(q, k, v, 1.0, q_pos=[0, 1, 9, 9], q_lo=[0, 0, 9, 0],
                                     k_pos=[5, 6, 7, 8, 2])
    assert np.all(O[0, 0, :3] == 0) and np.all(np.isneginf(L[0, 0, :3]))
    assert np.isfinite(L[0, 0, 3])


def test_local_only_attention_is_rejected():
    """Attending only the local shard (ring communication silently off, the
    pitfall on the hierarchical-CP skill page) must fail parity by far."""
    B, Hq, Hkv, S, d, cp = 1, 2, 1, 512, 32, 4
    q, k, v = _rand((B, Hq, S, d), 50), _rand((B, Hkv, S, d), 51), _rand((B, Hkv, S, d), 52)
    scale = 1 / math.sqrt(d)
    r = cp - 1
    pos = orc.zigzag_positions(S, cp, r)
    Ol, Ll = orc.partial_attention_fwd(q[:, :, pos], k[:, :, pos], v[:, :, pos], scale,
                                       pos, np.zeros_like(pos), pos)
    Of, Lf = orc.attention_fwd(q, k, v, scale, rows=pos)
    assert np.abs(Ol - Of).max() > 100 * 2e-2
    assert np.abs(Ll - Lf).max() > 100 * 1e-3


def test_seeded_inputs_are_exact_in_fp64():
    q, k, v, do = si.make_qkv(1, 2, 1, 64, 8, "bf16", seed=0, with_dout=True)
    q32 = si.make_qkv(1, 2, 1, 64, 8, "f32", seed=0)[0]
    assert torch.equal(q.to(torch.float32), q32.to(torch.bfloat16).to(torch.float32))
    assert np.array_equal(q.double().numpy().astype(np.float32), q.float().numpy())
    L = si.doc_lengths()
    assert L.sum() == 65536 and L[:-1].min() >= 128 and L.max() <= 16384
