"""GPU parity of the backward (cp_attn_bwd_delta, cp_attn_partial_bwd,
cp_attn_ring_bwd) against the fp64 oracle's gradients, through the C ABI.
Gradients of bf16 inputs must be within 5e-2 max-abs of the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle as orc
import seeded_inputs as si
import context_causal_attention_amd as cpa
from gpu_cases import Rank, announce, max_err, pair_error_bounds

pytestmark = pytest.mark.gpu

GTOL = 5e-2


def _np(t):
    return t.double().cpu().numpy()


def _check_grads(got, ref, what):
    errs = []
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        e = max_err(g, r)
        errs.append(e)
        assert np.isfinite(e) and e <= GTOL, f"{what}: {name} max-abs error {e:.3e} > {GTOL}"
    return errs


@pytest.mark.parametrize("o_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
def test_delta_matches_oracle(o_dtype, d):
    announce(f"delta d={d} o={o_dtype}")
    g = torch.Generator().manual_seed(3)
    B, H, S = 2, 3, 333
    dout = torch.randn(B, S, H, d, generator=g).to(torch.bfloat16).transpose(1, 2)  # strided rows
    o = torch.randn(B, H, S, d, generator=g).to(o_dtype)
    delta = cpa.cp_attn_bwd_delta(dout.cuda(), o.cuda())
    ref = orc.bwd_delta(_np(dout), _np(o))
    assert max_err(delta, ref) <= 1e-4


def test_delta_many_batch_heads():
    # 70 000 (batch, head) pairs of 5 rows each: more than 65 535 pairs, and
    # rows that split across workgroups.
    announce("delta B=2 H=35000 S=5 d=64")
    g = torch.Generator().manual_seed(4)
    dout = torch.randn(2, 35000, 5, 64, generator=g).to(torch.bfloat16)
    o = torch.randn(2, 35000, 5, 64, generator=g)
    delta = cpa.cp_attn_bwd_delta(dout.cuda(), o.cuda())
    ref = orc.bwd_delta(_np(dout), _np(o))
    assert max_err(delta, ref) <= 1e-4


@pytest.mark.parametrize("B,Hq,Hkv,S,d,cp", [
    (1, 2, 1, 1024, 64, 2),     # the C0 shape, bf16
    (1, 4, 2, 768, 128, 3),     # 256 rows a rank: 4 full 64-row tiles
    (1, 2, 2, 1200, 64, 3),     # 400 rows a rank: ragged key and query tiles
    (2, 8, 2, 640, 128, 5),     # batch 2, four query heads a group
    (1, 4, 1, 4096, 128, 1),    # cp = 1: plain causal attention
])
def test_ring_bwd_all_ranks_sum_to_full_gradients(B, Hq, Hkv, S, d, cp):
    """Every rank's ring backward, summed, gives the gradients of the whole
    sequence: dq row by row, dk and dv from every rank's contribution."""
    q, k, v, do = si.make_qkv(B, Hq, Hkv, S, d, "bf16", seed=4, with_dout=True)
    scale = 1 / math.sqrt(d)
    dq_ref, dk_ref, dv_ref = orc.attention_bwd(_np(q), _np(k), _np(v), _np(do), scale)
    dk_sum = dv_sum = None
    for rank in range(cp):
        announce(f"ring bwd B={B} Hq={Hq} Hkv={Hkv} S={S} d={d} cp={cp} rank {rank}")
        R = Rank(B, Hq, Hkv, S, d, cp, rank, "bf16", full=(q, k, v, do))
        _, _, dq, dk, dv = R.ring_bwd()
        e = max_err(dq, dq_ref[:, :, R.pos])
        assert e <= GTOL, f"rank {rank}: dq max-abs error {e:.3e}"
        dk_sum = dk if dk_sum is None else dk_sum + dk
        dv_sum = dv if dv_sum is None else dv_sum + dv
    allp = orc.all_rank_positions(S, cp)
    for name, g, r in (("dk", dk_sum, dk_ref[:, :, allp]), ("dv", dv_sum, dv_ref[:, :, allp])):
        e = max_err(g, r)
        assert e <= GTOL, f"{name} summed over ranks: max-abs error {e:.3e}"


@pytest.mark.parametrize("kvh", [0, 7])
def test_c4_all_ranks_sum_to_full_gradients(kvh):
    """The backward workload itself (32 768 tokens, cp = 8, 32 query / 8 kv
    heads, d = 128, bf16, dO ~ N(0,1)): all 8 virtual ranks' ring backwards
    over every head, their dK/dV summed, against the oracle's gradients of the
    whole sequence for one kv group (query heads 4kvh..4kvh+3): dQ row by row
    on every rank, dK and dV from every rank's contribution.  kv groups 0 and
    7, the first and the last."""
    w = si.WORKLOADS["bwd_s32k_cp8"]
    full = si.make_qkv(w.B, w.Hq, w.Hkv, w.S, w.d, "bf16", seed=w.seed, with_dout=True)
    g = w.Hq // w.Hkv
    hs, ks = slice(kvh * g, (kvh + 1) * g), slice(kvh, kvh + 1)
    q, k, v, do = (_np(t) for t in full)
    dq_ref, dk_ref, dv_ref = orc.attention_bwd(q[:, hs], k[:, ks], v[:, ks], do[:, hs], w.scale)
    dk_sum = dv_sum = None
    for rank in range(w.cp):
        announce(f"c4 all ranks summed, kv group {kvh}: rank {rank}")
        R = Rank(w.B, w.Hq, w.Hkv, w.S, w.d, w.cp, rank, "bf16", full=full)
        _, _, dq, dk, dv = R.ring_bwd()
        e = max_err(dq[:, hs], dq_ref[:, :, R.pos])
        assert e <= GTOL, f"rank {rank}: dq max-abs error {e:.3e}"
        dk_sum = dk[:, ks].clone() if dk_sum is None else dk_sum + dk[:, ks]
        dv_sum = dv[:, ks].clone() if dv_sum is None else dv_sum + dv[:, ks]
        del R, dq, dk, dv
    allp = orc.all_rank_positions(w.S, w.cp)
    for name, got, ref in (("dk", dk_sum, dk_ref[:, :, allp]), ("dv", dv_sum, dv_ref[:, :, allp])):
        e = max_err(got, ref)
        assert e <= GTOL, f"{name} summed over ranks, kv group {kvh}: max-abs error {e:.3e}"


@pytest.mark.parametrize("rank", [0, 7])
def test_ring_bwd_32k_cp8_per_rank(rank):
    """The backward on the Llama-3-8B-shaped 32 768-token cp=8 workload (32
    query / 8 kv heads, d = 128, bf16): the whole ring of one virtual rank,
    checked on the first kv group (query heads 0-3, kv head 0) against the
    oracle's gradients of that rank's loss."""
    w = si.WORKLOADS["bwd_s32k_cp8"]
    announce(f"ring bwd 32k cp8 rank {rank}")
    R = Rank(w.B, w.Hq, w.Hkv, w.S, w.d, w.cp, rank, "bf16", seed=w.seed, with_dout=True)
    _, _, dq, dk, dv = R.ring_bwd()
    torch.cuda.synchronize()
    g = w.Hq // w.Hkv
    ref = R.oracle_grads(q_heads=slice(0, g))
    _check_grads((dq[:, :g], dk[:, :1], dv[:, :1]), ref, f"32k rank {rank}")
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()


def test_ring_bwd_32k_cp8_rank0_every_head():
    """Virtual rank 0 of the 32 768-token backward, every kv group (all 32
    query heads and 8 kv heads), against the oracle's gradients of that rank's
    loss: the full dQ of its rows and the full dK/dV of every shard."""
    w = si.WORKLOADS["bwd_s32k_cp8"]
    R = Rank(w.B, w.Hq, w.Hkv, w.S, w.d, w.cp, 0, "bf16", seed=w.seed, with_dout=True)
    _, _, dq, dk, dv = R.ring_bwd()
    torch.cuda.synchronize()
    g = w.Hq // w.Hkv
    for kvh in range(w.Hkv):
        announce(f"ring bwd 32k cp8 rank 0, kv group {kvh}")
        ref = R.oracle_grads(q_heads=slice(kvh * g, (kvh + 1) * g))
        _check_grads((dq[:, kvh * g:(kvh + 1) * g], dk[:, kvh:kvh + 1], dv[:, kvh:kvh + 1]), ref,
                     f"32k rank 0 group {kvh}")


@pytest.mark.parametrize("rank", [0, 7])
def test_ring_bwd_128k_cp8_sampled(rank):
    """The backward at the bench workload's size (131072 tokens, cp=8, 32q/8kv
    heads, d=128, bf16), in the launch configuration the bench times.
    dQ: sampled rows of the rank, all heads, against the oracle's gradient of
    those rows' loss terms (row i's dQ depends on its own term only).
    dK, dV: the last 128 keys of the rank's second chunk are attended, among the
    rank's rows, only by its last 128 rows, so the oracle restricted to those
    rows gives their gradients exactly; checked for kv heads 0 and 7."""
    w = si.WORKLOADS["llama8b_s128k_cp8"]
    full = si.make_qkv(w.B, w.Hq, w.Hkv, w.S, w.d, "bf16", seed=w.seed, with_dout=True)
    announce(f"ring bwd 128k cp8 rank {rank}")
    R = Rank(w.B, w.Hq, w.Hkv, w.S, w.d, w.cp, rank, "bf16", full=full)
    _, _, dq, dk, dv = R.ring_bwd()
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
    q64, k64, v64, do64 = (t.double().numpy() for t in full)
    n = w.S // w.cp
    c = n // 2
    rng = np.random.default_rng(2)
    idx = np.unique(np.concatenate([[0, c - 1, c, n - 1], rng.integers(0, n, 6)]))
    rows = R.pos[idx]
    dq_ref, _, _ = orc.attention_bwd(q64, k64, v64, do64[:, :, rows], R.scale, rows=rows)
    e = max_err(dq[:, :, idx], dq_ref)
    assert e <= GTOL, f"dq on sampled rows: max-abs error {e:.3e}"
    g = w.Hq // w.Hkv
    last = R.pos[-128:]  # last 128 positions of the rank's second chunk
    where = np.argsort(R.allp)[last]  # their rows in k_all
    for kvh in (0, w.Hkv - 1):
        hs = slice(kvh * g, (kvh + 1) * g)
        _, dk_ref, dv_ref = orc.attention_bwd(q64[:, hs], k64[:, kvh:kvh + 1], v64[:, kvh:kvh + 1],
                                              do64[:, hs][:, :, last], R.scale, rows=last)
        for name, got, ref in (("dk", dk[:, kvh:kvh + 1, where], dk_ref[:, :, last]),
                               ("dv", dv[:, kvh:kvh + 1, where], dv_ref[:, :, last])):
            e = max_err(got, ref)
            assert e <= GTOL, f"{name} of the last 128 keys, kv head {kvh}: max-abs error {e:.3e}"


@pytest.mark.parametrize("rank", [0, 7])
def test_ring_bwd_128k_cp8_every_key_of_sampled_rows(rank):
    """dK and dV of every key of the 131072-token ring (cp=8, 32q/8kv heads,
    d=128, bf16), in the launch configuration the bench times, elementwise
    against the oracle.  dO is zero except on sampled rows of the rank.  The
    gradients are linear in dO (delta = rowsum(dO.O) too), so dK and dV are
    exactly those rows' contributions, which the oracle computes from those
    rows alone; the other rows' dQ is exactly zero.

    The bound per element (gpu_cases.pair_error_bounds) follows the
    arithmetic of one pair: bf16 P and dS, the kernel's LSE and delta errors,
    fp32 sums; about 2^-6 of each gradient's own magnitude, far below the
    5e-2 acceptance bar.  tests/test_bounds_cpu.py checks it against an
    emulation of that arithmetic and a planted mistake."""
    w = si.WORKLOADS["llama8b_s128k_cp8"]
    q, k, v, do = si.make_qkv(w.B, w.Hq, w.Hkv, w.S, w.d, "bf16", seed=w.seed, with_dout=True)
    announce(f"ring bwd 128k cp8 rank {rank}, every key, dO on sampled rows")
    n = w.S // w.cp
    c = n // 2
    pos_r = orc.zigzag_positions(w.S, w.cp, rank)
    rng = np.random.default_rng(11 + rank)
    idx = np.unique(np.concatenate([[0, 1, c - 1, c, c + 1, n - 1], rng.integers(0, n, 10)]))
    rows = pos_r[idx]
    keep = torch.zeros(w.S, dtype=torch.bool)
    keep[torch.from_numpy(rows.astype(np.int64))] = True
    do = torch.where(keep[None, None, :, None], do, torch.zeros((), dtype=do.dtype))
    R = Rank(w.B, w.Hq, w.Hkv, w.S, w.d, w.cp, rank, "bf16", full=(q, k, v, do))
    o, lse = R.ring_fwd()
    delta = cpa.cp_attn_bwd_delta(R.do_loc, o)
    dq, dk, dv = cpa.cp_attn_ring_bwd(R.q_loc, R.k_all, R.v_all, R.do_loc, lse, delta, R.cp, R.rank, R.pos,
                                      R.lo, R.allp, scale=R.scale)
    torch.cuda.synchronize()
    others = np.setdiff1d(np.arange(n), idx)
    assert torch.count_nonzero(dq[:, :, torch.from_numpy(others)]) == 0, "dQ of rows with zero dO is not zero"

    q64, k64, v64 = (t.double().numpy() for t in (q, k, v))
    do_r = do[:, :, torch.from_numpy(rows.astype(np.int64))].double().numpy()
    dq_ref, dk_ref, dv_ref = orc.attention_bwd(q64, k64, v64, do_r, R.scale, rows=rows)
    O_ref, L_ref = orc.attention_fwd(q64, k64, v64, R.scale, rows=rows)
    dl_ref = orc.bwd_delta(do_r, O_ref)
    # The kernels' own LSE and delta errors at the sampled rows enter the bound.
    dL = np.abs(_np(lse[:, :, idx]) - L_ref)
    ddl = np.abs(_np(delta[:, :, idx]) - dl_ref)
    assert dL.max() <= 1e-3, f"LSE at the sampled rows: {dL.max():.3e}"

    # Per-element bounds, from the pair errors (fp64, sampled rows only).
    tol_dv, tol_dk, tol_dq = pair_error_bounds(q64, k64, v64, do_r, rows, R.scale, L_ref, dl_ref, dL, ddl,
                                               w.Hq // w.Hkv)
    where = np.argsort(R.allp)  # natural position -> row of k_all
    for name, got, ref, tol in (("dv", _np(dv)[:, :, where], dv_ref, tol_dv),
                                ("dk", _np(dk)[:, :, where], dk_ref, tol_dk),
                                ("dq", _np(dq[:, :, idx]), dq_ref, tol_dq)):
        err = np.abs(got - ref)
        worst = np.unravel_index(np.argmax(err / tol), err.shape)
        assert np.all(err <= tol), (f"{name}: error {err[worst]:.3e} above its bound {tol[worst]:.3e} at {worst} "
                                    f"(reference {ref[worst]:.3e})")
        assert err.max() <= GTOL


@pytest.mark.parametrize("mode", [cpa.CP_STREAM, cpa.CP_PER_DOC, cpa.CP_WHOLE_DOC])
def test_ring_bwd_varlen(mode):
    """Block-diagonal document masks: each rank's loss against the oracle with
    the same cu_seqlens."""
    cp, d = 2, 128
    # whole-document deal: the 300-token document fits no rank whole and is cut
    lens = [900, 300, 500, 348] if mode == cpa.CP_WHOLE_DOC else [256, 512, 128, 640, 512]
    cu = si.cu_seqlens_from_lengths(lens)
    S = int(cu[-1])
    full = si.make_qkv(1, 4, 2, S, d, "bf16", seed=5, with_dout=True)
    for rank in range(cp):
        announce(f"ring bwd varlen mode={mode} rank {rank}")
        R = Rank(1, 4, 2, S, d, cp, rank, "bf16", cu=cu, mode=mode, full=full)
        _, _, dq, dk, dv = R.ring_bwd()
        _check_grads((dq, dk, dv), R.oracle_grads(), f"varlen mode {mode} rank {rank}")


@pytest.mark.parametrize("rank", [0, 3])
def test_ring_bwd_varlen_s64k_cp4_whole_doc_sampled(rank):
    """The packed-document backward at the bench workload's size (65536 tokens,
    42 lognormal documents, 32q/8kv heads, d=128, bf16, cp=4, whole-document
    deal), with the dispatch orders the bench runs.  dQ: sampled rows, all
    heads, against the oracle's gradient of those rows' loss terms.  dK, dV: a
    document that lies whole on the rank is attended only by its own rows, so
    the oracle restricted to them gives its keys' gradients exactly."""
    w = si.WORKLOADS["varlen_s64k_cp4"]
    cu = si.workload_cu_seqlens(w)
    full = si.make_qkv(w.B, w.Hq, w.Hkv, w.S, w.d, "bf16", seed=w.seed, with_dout=True)
    announce(f"ring bwd varlen 64k cp4 whole-doc rank {rank}")
    R = Rank(w.B, w.Hq, w.Hkv, w.S, w.d, w.cp, rank, "bf16", cu=cu, mode=cpa.CP_WHOLE_DOC, full=full)
    _, _, dq, dk, dv = R.ring_bwd()
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
    q64, k64, v64, do64 = (t.double().numpy() for t in full)
    n = len(R.pos)
    rng = np.random.default_rng(7)
    starts = np.flatnonzero(R.pos == R.lo)
    idx = np.unique(np.concatenate([[0, n - 1], rng.choice(starts, 3, replace=False), rng.integers(0, n, 5)]))
    rows = R.pos[idx]
    dq_ref, _, _ = orc.attention_bwd(q64, k64, v64, do64[:, :, rows], R.scale, cu_seqlens=cu, rows=rows)
    e = max_err(dq[:, :, idx], dq_ref)
    assert e <= GTOL, f"dq on sampled rows: max-abs error {e:.3e}"
    # a document of 300-1500 tokens whose every row is on this rank
    mine = set(R.pos.tolist())
    docs = [(int(a), int(b)) for a, b in zip(cu[:-1], cu[1:])
            if 300 <= b - a <= 1500 and all(p in mine for p in range(int(a), int(b)))]
    assert docs, "no whole document of 300-1500 tokens on this rank"
    a, b = min(docs, key=lambda ab: ab[1] - ab[0])
    doc = np.arange(a, b)
    _, dk_ref, dv_ref = orc.attention_bwd(q64, k64, v64, do64[:, :, doc], R.scale, cu_seqlens=cu, rows=doc)
    where = np.argsort(R.allp)[doc]  # the document's rows in k_all
    for name, got, ref in (("dk", dk[:, :, where], dk_ref[:, :, doc]), ("dv", dv[:, :, where], dv_ref[:, :, doc])):
        e = max_err(got, ref)
        assert e <= GTOL, f"{name} of document [{a}, {b}): max-abs error {e:.3e}"


def test_ring_bwd_shuffled_rows_and_keys():
    """The backward with a rank's rows and every shard's keys in random order
    (whole-document deal): per-tile key gaps, per-wave and per-tile row holes
    and the dK/dV waves' key gaps must hold for any order."""
    cp, S, d = 2, 2048, 64
    cu = si.cu_seqlens_from_lengths([900, 300, 500, 348])
    full = si.make_qkv(1, 4, 2, S, d, "bf16", seed=24, with_dout=True)
    rng = np.random.default_rng(25)
    for rank in range(cp):
        announce(f"ring bwd shuffled rows/keys rank {rank}")
        R = Rank(1, 4, 2, S, d, cp, rank, "bf16", cu=cu, mode=cpa.CP_WHOLE_DOC, full=full)
        pq = rng.permutation(len(R.pos))
        R.pos, R.lo = R.pos[pq], R.lo[pq]
        R.q_loc = R.q_loc[:, :, torch.from_numpy(pq)].contiguous()
        R.do_loc = R.do_loc[:, :, torch.from_numpy(pq)].contiguous()
        n = S // cp
        pk = np.concatenate([s * n + rng.permutation(n) for s in range(cp)])
        R.allp = R.allp[pk]
        R.k_all = R.k_all[:, :, torch.from_numpy(pk)].contiguous()
        R.v_all = R.v_all[:, :, torch.from_numpy(pk)].contiguous()
        _, _, dq, dk, dv = R.ring_bwd()
        _check_grads((dq, dk, dv), R.oracle_grads(), f"shuffled rank {rank}")


def test_partial_bwd_steps_match_ring():
    """The per-step path (one cp_attn_partial_bwd a ring step, each with the
    final LSE and delta) adds up to the fused ring backward and to the oracle."""
    B, Hq, Hkv, S, d, cp = 1, 4, 1, 1536, 64, 3
    full = si.make_qkv(B, Hq, Hkv, S, d, "bf16", seed=6, with_dout=True)
    for rank in range(cp):
        announce(f"partial bwd steps rank {rank}")
        R = Rank(B, Hq, Hkv, S, d, cp, rank, "bf16", full=full)
        o, lse, dq_r, dk_r, dv_r = R.ring_bwd()
        delta = cpa.cp_attn_bwd_delta(R.do_loc, o)
        n = S // cp
        dq = torch.zeros_like(dq_r)
        dk = torch.zeros_like(dk_r)
        dv = torch.zeros_like(dv_r)
        for t in range(cp):
            src = cpa.cp_ring_source(cp, rank, t)
            sl = slice(src * n, (src + 1) * n)
            cpa.cp_attn_partial_bwd(R.q_loc, R.k_all[:, :, sl], R.v_all[:, :, sl], R.do_loc, lse, delta, R.pos,
                                    None, R.allp[sl], dq=dq, dk=dk[:, :, sl], dv=dv[:, :, sl], scale=R.scale)
        for a, b_ in ((dq, dq_r), (dk, dk_r), (dv, dv_r)):
            assert (a - b_).abs().max().item() <= 1e-3
        _check_grads((dq, dk, dv), R.oracle_grads(), f"partial steps rank {rank}")


def test_partial_bwd_rows_without_keys():
    """One ring step alone, with the step's own LSE and delta: rank 0 of cp=2
    (positions 0..255 and 768..1023 of 1024) against keys at positions
    100..611.  Rows 0..99 have no allowed key (LSE -inf), rows 100..255 some,
    and query tiles mix both kinds; the gradients must be finite, zero in dQ
    for the rows without keys, and match the oracle's per-step backward."""
    B, Hq, Hkv, S, d, cp = 1, 4, 2, 1024, 128, 2
    q, k, v, do = si.make_qkv(B, Hq, Hkv, S, d, "bf16", seed=9, with_dout=True)
    rows = orc.zigzag_positions(S, cp, 0)
    keys = np.arange(100, 612)
    scale = 1.0 / math.sqrt(d)
    announce("partial bwd, rows without keys")
    ri, ki = torch.from_numpy(rows.astype(np.int64)), torch.from_numpy(keys)
    qg, dog = q.index_select(2, ri).cuda(), do.index_select(2, ri).cuda()
    kg, vg = k.index_select(2, ki).cuda(), v.index_select(2, ki).cuda()
    o, lse = cpa.cp_attn_partial_fwd(qg, kg, vg, rows, None, keys, scale=scale)
    none = rows < 100
    assert torch.isneginf(lse[:, :, torch.from_numpy(none).cuda()]).all()
    delta = cpa.cp_attn_bwd_delta(dog, o)
    dq, dk, dv = cpa.cp_attn_partial_bwd(qg, kg, vg, dog, lse, delta, rows, None, keys, scale=scale)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
    assert torch.all(dq[:, :, torch.from_numpy(none).cuda()] == 0)
    q64, k64, v64, do64 = (x.double().numpy() for x in (q, k, v, do))
    O_ref, L_ref = orc.partial_attention_fwd(q64[:, :, rows], k64[:, :, keys], v64[:, :, keys], scale, rows,
                                             np.zeros_like(rows), keys)
    ref = orc.partial_attention_bwd(q64[:, :, rows], k64[:, :, keys], v64[:, :, keys], do64[:, :, rows], L_ref,
                                    orc.bwd_delta(do64[:, :, rows], O_ref), scale, rows, np.zeros_like(rows), keys)
    _check_grads((dq, dk, dv), ref, "partial bwd rows without keys")


def test_bwd_accumulates_and_is_deterministic():
    """Calls add into the gradient buffers: a second identical call doubles
    them exactly, and two fresh runs agree bit for bit."""
    R = Rank(1, 4, 2, 1024, 128, 2, 1, "bf16", seed=7, with_dout=True)
    announce("bwd accumulate / determinism")
    o, lse = R.ring_fwd()
    delta = cpa.cp_attn_bwd_delta(R.do_loc, o)
    args = (R.q_loc, R.k_all, R.v_all, R.do_loc, lse, delta, R.cp, R.rank, R.pos, R.lo, R.allp)
    dq1, dk1, dv1 = cpa.cp_attn_ring_bwd(*args, scale=R.scale)
    dq1, dk1, dv1 = dq1.clone(), dk1.clone(), dv1.clone()
    dq2, dk2, dv2 = cpa.cp_attn_ring_bwd(*args, scale=R.scale)
    assert torch.equal(dq2, dq1) and torch.equal(dk2, dk1) and torch.equal(dv2, dv1)
    cpa.cp_attn_ring_bwd(*args, scale=R.scale, dq=dq2, dk=dk2, dv=dv2)
    assert torch.equal(dq2, 2 * dq1) and torch.equal(dk2, 2 * dk1) and torch.equal(dv2, 2 * dv1)


def test_bwd_strided_inputs():
    """q and dO as [B, S, H, D] storage viewed as [B, H, S, D] (row stride H*D)."""
    B, Hq, Hkv, S, d, cp = 1, 4, 2, 1024, 128, 2
    q, k, v, do = si.make_qkv(B, Hq, Hkv, S, d, "bf16", seed=8, with_dout=True)
    for rank in range(cp):
        announce(f"bwd strided rank {rank}")
        R = Rank(B, Hq, Hkv, S, d, cp, rank, "bf16", full=(q, k, v, do))
        R.q_loc = R.q_loc.transpose(1, 2).contiguous().transpose(1, 2)
        R.do_loc = R.do_loc.transpose(1, 2).contiguous().transpose(1, 2)
        R.k_all = R.k_all.transpose(1, 2).contiguous().transpose(1, 2)
        _, _, dq, dk, dv = R.ring_bwd()
        _check_grads((dq, dk, dv), R.oracle_grads(), f"strided rank {rank}")


def test_bwd_empty_inputs():
    announce("bwd empty inputs")
    q = torch.zeros(1, 2, 0, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.randn(1, 1, 64, 64, device="cuda").to(torch.bfloat16)
    e = torch.zeros(1, 2, 0, device="cuda")
    dq, dk, dv = cpa.cp_attn_partial_bwd(q, k, k, q, e, e, [], None, list(range(64)))
    assert dq.numel() == 0 and torch.all(dk == 0) and torch.all(dv == 0)
    q = torch.randn(1, 2, 64, 64, device="cuda").to(torch.bfloat16)
    k0 = torch.zeros(1, 1, 0, 64, dtype=torch.bfloat16, device="cuda")
    l = torch.zeros(1, 2, 64, device="cuda")
    dq, dk, dv = cpa.cp_attn_partial_bwd(q, k0, k0, q, l, l, list(range(64)), None, [])
    assert torch.all(dq == 0)
