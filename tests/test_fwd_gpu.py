"""GPU parity of the forward path (cp_attn_partial_fwd, cp_attn_merge,
cp_attn_ring_fwd) against the fp64 oracle, through the C ABI."""
import math

import numpy as np
import pytest
import torch

import oracle as orc
import seeded_inputs as si
import context_causal_attention_amd as cpa
from gpu_cases import Rank, announce, assert_close, max_err, TOL

pytestmark = pytest.mark.gpu


def _np(t):
    return t.double().cpu().numpy()


# ------------------------------------------------------------------ one ring step, per chunk-pair class
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_partial_chunk_pair_classes(dtype, d):
    """Rank 0 of cp=2 holds chunks 0 and 3 (c = 192 rows each, not a multiple
    of the tile sizes): Q[a] x K[a] is diagonal-causal, Q[b] x K[a] full,
    Q[a] x K[b] fully masked (O = 0, LSE = -inf), Q[b] x K[b] diagonal."""
    B, Hq, Hkv, S, cp = 1, 4, 2, 768, 2
    c = S // (2 * cp)
    q, k, v = si.make_qkv(B, Hq, Hkv, S, d, dtype, seed=1)
    scale = 1 / math.sqrt(d)
    qd, kd, vd = (t.double().numpy() for t in (q, k, v))
    chunks = {"a": np.arange(0, c), "b": np.arange(3 * c, 4 * c)}
    for qa in "ab":
        for ka in "ab":
            announce(f"partial {dtype} d={d} Q[{qa}] x K[{ka}]")
            qi, ki = chunks[qa], chunks[ka]
            qt = q[:, :, qi].cuda()
            kt, vt = k[:, :, ki].cuda(), v[:, :, ki].cuda()
            o, lse = cpa.cp_attn_partial_fwd(qt, kt, vt, qi, None, ki, scale=scale)
            O_ref, L_ref = orc.partial_attention_fwd(qd[:, :, qi], kd[:, :, ki], vd[:, :, ki], scale, qi,
                                                     np.zeros_like(qi), ki)
            assert_close(o, lse, O_ref, L_ref, dtype, f"Q[{qa}] x K[{ka}]")
            if qa == "a" and ka == "b":
                assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_partial_then_merge_equals_ring(dtype):
    """The per-step path (partial + merge, ring order) and the fused ring kernel
    both match the oracle."""
    B, Hq, Hkv, S, d, cp = 1, 4, 1, 1536, 64, 3
    for rank in range(cp):
        announce(f"per-step vs ring {dtype} rank {rank}")
        R = Rank(B, Hq, Hkv, S, d, cp, rank, dtype, seed=2)
        O_ref, L_ref = R.oracle()
        n = S // cp
        o_acc = torch.zeros(B, Hq, n, d, device="cuda")
        l_acc = torch.full((B, Hq, n), -math.inf, device="cuda")
        for t in range(cp):
            src = cpa.cp_ring_source(cp, rank, t)
            sl = slice(src * n, (src + 1) * n)
            o_p, l_p = cpa.cp_attn_partial_fwd(R.q_loc, R.k_all[:, :, sl], R.v_all[:, :, sl], R.pos, None,
                                               R.allp[sl], scale=R.scale)
            cpa.cp_attn_merge(o_acc, l_acc, o_p, l_p)
        assert_close(o_acc, l_acc, O_ref, L_ref, dtype, f"per-step rank {rank}")
        o, lse = R.ring_fwd()
        assert_close(o, lse, O_ref, L_ref, dtype, f"ring rank {rank}")


# ------------------------------------------------------------------ whole virtual-rank ring
def test_c0_config_fp32():
    """1 head, d=64, S=1024, cp=2, fp32 N(0,1) from seed 0, scale 1/8: each rank's
    2-step ring forward against full attention."""
    w = si.WORKLOADS["c0_f32_s1024_cp2"]
    full = si.make_qkv(w.B, w.Hq, w.Hkv, w.S, w.d, w.dtype, seed=w.seed)
    for rank in range(w.cp):
        announce(f"c0 rank {rank}")
        R = Rank(w.B, w.Hq, w.Hkv, w.S, w.d, w.cp, rank, w.dtype, full=full)
        assert R.scale == 1 / 8
        o, lse = R.ring_fwd()
        O_ref, L_ref = R.oracle()
        assert_close(o, lse, O_ref, L_ref, "f32", f"c0 rank {rank}")


@pytest.mark.parametrize("S,cp,Hq,Hkv,d", [(2048, 4, 4, 2, 128), (1200, 2, 2, 1, 128), (4096, 8, 8, 2, 64),
                                           (640, 1, 2, 2, 128)])
def test_ring_bf16_all_ranks(S, cp, Hq, Hkv, d):
    full = si.make_qkv(1, Hq, Hkv, S, d, "bf16", seed=3)
    for rank in range(cp):
        announce(f"ring bf16 S={S} cp={cp} H={Hq}/{Hkv} d={d} rank {rank}")
        R = Rank(1, Hq, Hkv, S, d, cp, rank, "bf16", full=full)
        o, lse = R.ring_fwd()
        assert_close(o, lse, *R.oracle(), "bf16", f"rank {rank}")


def test_ring_batch_and_bf16_output():
    B, Hq, Hkv, S, d, cp = 2, 4, 2, 1024, 128, 2
    full = si.make_qkv(B, Hq, Hkv, S, d, "bf16", seed=4)
    R = Rank(B, Hq, Hkv, S, d, cp, 1, "bf16", full=full)
    announce("ring batch 2, bf16 output")
    o32, l32 = R.ring_fwd()
    o16, l16 = R.ring_fwd(out_dtype=torch.bfloat16)
    assert o16.dtype == torch.bfloat16
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.equal(l16, l32)
    assert_close(o16, l16, *R.oracle(), "bf16", "bf16 out")


def test_ring_fp32_d128_and_gqa_groups():
    B, Hq, Hkv, S, d, cp = 1, 8, 2, 512, 128, 2
    full = si.make_qkv(B, Hq, Hkv, S, d, "f32", seed=5)
    for rank in range(cp):
        announce(f"ring f32 d128 gqa rank {rank}")
        R = Rank(B, Hq, Hkv, S, d, cp, rank, "f32", full=full)
        o, lse = R.ring_fwd()
        assert_close(o, lse, *R.oracle(), "f32", f"rank {rank}")


@pytest.mark.parametrize("mode", [cpa.CP_STREAM, cpa.CP_PER_DOC, cpa.CP_WHOLE_DOC])
def test_ring_varlen_documents(mode):
    cp = 4
    if mode != cpa.CP_PER_DOC:
        L = si.doc_lengths(total=4096, mean=400, sigma=1.0, lo=16, hi=3000, seed=7)
    else:
        L = (si.doc_lengths(total=4096, mean=400, sigma=1.0, lo=16, hi=3000, seed=7) // 8) * 8
        L = np.append(L[L > 0], 4096 - L.sum())
        L = L[L > 0]
    cu = si.cu_seqlens_from_lengths(L)
    S = int(cu[-1])
    full = si.make_qkv(1, 4, 2, S, 128, "bf16", seed=8)
    for rank in range(cp):
        announce(f"varlen mode {mode} rank {rank} ({len(L)} docs)")
        R = Rank(1, 4, 2, S, 128, cp, rank, "bf16", full=full, cu=cu, mode=mode)
        o, lse = R.ring_fwd()
        assert_close(o, lse, *R.oracle(), "bf16", f"varlen rank {rank}")


def test_ring_varlen_one_query_tile():
    """Packed documents with 128 rows a rank (one query tile, so no dispatch
    order and no key lists precomputed for it: the workgroup lists its key
    tiles itself, masks included): every rank, every row, against the oracle."""
    cp = 4
    L = si.doc_lengths(total=512, mean=60, sigma=1.0, lo=4, hi=400, seed=17)
    cu = si.cu_seqlens_from_lengths(L)
    S = int(cu[-1])
    full = si.make_qkv(1, 4, 2, S, 128, "bf16", seed=18)
    for rank in range(cp):
        announce(f"varlen one query tile rank {rank} ({len(L)} docs)")
        R = Rank(1, 4, 2, S, 128, cp, rank, "bf16", full=full, cu=cu)
        assert len(R.pos) == 128
        o, lse = R.ring_fwd()
        assert_close(o, lse, *R.oracle(), "bf16", f"varlen one tile rank {rank}")


def test_llama8b_s32k_cp8_all_ranks_sampled():
    """32q/8kv heads, d=128, S=32768, cp=8: every rank's full ring, checked on
    sampled rows (first/last rows of both chunks plus random rows)."""
    w = si.WORKLOADS["llama8b_s32k_cp8"]
    full = si.make_qkv(w.B, w.Hq, w.Hkv, w.S, w.d, w.dtype, seed=w.seed)
    rng = np.random.default_rng(0)
    n = w.S // w.cp
    c = n // 2
    for rank in range(w.cp):
        announce(f"llama8b 32k rank {rank}")
        R = Rank(w.B, w.Hq, w.Hkv, w.S, w.d, w.cp, rank, w.dtype, full=full)
        o, lse = R.ring_fwd()
        idx = np.unique(np.concatenate([[0, 1, c - 1, c, c + 1, n - 1], rng.integers(0, n, 58)]))
        O_ref, L_ref = R.oracle(idx)
        assert_close(o[:, :, idx], lse[:, :, idx], O_ref, L_ref, "bf16", f"rank {rank}")


@pytest.mark.parametrize("name,mode", [("varlen_s64k_cp4", cpa.CP_STREAM), ("varlen_s64k_cp4", cpa.CP_WHOLE_DOC),
                                       ("varlen8_s64k_cp4", cpa.CP_STREAM), ("varlen8_s64k_cp4", cpa.CP_PER_DOC),
                                       ("varlen8_s64k_cp4", cpa.CP_WHOLE_DOC)])
def test_varlen_s64k_cp4_all_ranks_sampled(name, mode):
    """The packed-document workloads themselves (65536 tokens of 42 lognormal
    documents, and the same documents with lengths rounded to multiples of
    2cp = 8 so that the per-document deal applies; 32q/8kv heads, d=128,
    bf16, cp=4), in every deal the bench times: every rank's ring, checked on
    sampled rows (each rank's first and last rows, rows at its document
    starts, random rows) against the oracle."""
    w = si.WORKLOADS[name]
    cu = si.workload_cu_seqlens(w)
    full = si.make_qkv(w.B, w.Hq, w.Hkv, w.S, w.d, w.dtype, seed=w.seed)
    rng = np.random.default_rng(3)
    n = w.S // w.cp
    for rank in range(w.cp):
        announce(f"{name} mode {mode} rank {rank}")
        R = Rank(w.B, w.Hq, w.Hkv, w.S, w.d, w.cp, rank, w.dtype, full=full, cu=cu, mode=mode)
        o, lse = R.ring_fwd()
        starts = np.flatnonzero(R.pos == R.lo)  # rows that begin a document
        idx = np.unique(np.concatenate([[0, n - 1], rng.choice(starts, min(8, len(starts)), replace=False),
                                        rng.integers(0, n, 40)]))
        O_ref, L_ref = R.oracle(idx)
        assert_close(o[:, :, idx], lse[:, :, idx], O_ref, L_ref, "bf16", f"rank {rank}")


def test_llama8b_s32k_cp8_rank0_every_row():
    """Every row of virtual rank 0 of the 32768-token workload (32q/8kv heads,
    d=128, bf16, cp=8: chunks 0 and 15, 4096 rows per head) against the oracle
    computed for all of them: the full output, not a sample."""
    w = si.WORKLOADS["llama8b_s32k_cp8"]
    announce("llama8b 32k rank 0, every row")
    R = Rank(w.B, w.Hq, w.Hkv, w.S, w.d, w.cp, 0, w.dtype, seed=w.seed)
    o, lse = R.ring_fwd()
    O_ref, L_ref = R.oracle()
    assert_close(o, lse, O_ref, L_ref, "bf16", "rank 0 every row")


def test_llama8b_s128k_cp8_all_ranks_sampled():
    """The bench workload itself (131072 tokens, 32q/8kv heads, d=128, cp=8,
    bf16), in the launch configuration the bench times: every rank's full ring,
    checked on sampled rows (chunk ends plus random rows) against the oracle
    computed row by row."""
    w = si.WORKLOADS["llama8b_s128k_cp8"]
    full = si.make_qkv(w.B, w.Hq, w.Hkv, w.S, w.d, w.dtype, seed=w.seed)
    q64, k64, v64 = (t.double().numpy() for t in full)
    rng = np.random.default_rng(1)
    n = w.S // w.cp
    c = n // 2
    for rank in range(w.cp):
        announce(f"llama8b 128k rank {rank}")
        R = Rank(w.B, w.Hq, w.Hkv, w.S, w.d, w.cp, rank, w.dtype, full=full)
        o, lse = R.ring_fwd()
        idx = np.unique(np.concatenate([[0, c - 1, c, n - 1], rng.integers(0, n, 8)]))
        O_ref, L_ref = orc.attention_fwd(q64, k64, v64, R.scale, rows=R.pos[idx])
        assert_close(o[:, :, idx], lse[:, :, idx], O_ref, L_ref, "bf16", f"rank {rank}")
        del R, o, lse
        torch.cuda.empty_cache()


@pytest.mark.parametrize("d", [64, 128])
def test_long_dense_ring_sampled(d):
    """A dense ring of 65536 keys, which the forward launches with 8-wave
    workgroups (shorter rings and document masks use 4), at both head
    dimensions: sampled rows of the first and last rank against the oracle."""
    S, cp, Hq, Hkv = 65536, 4, 4, 1
    full = si.make_qkv(1, Hq, Hkv, S, d, "bf16", seed=5)
    q64, k64, v64 = (t.double().numpy() for t in full)
    rng = np.random.default_rng(2)
    n = S // cp
    for rank in (0, cp - 1):
        announce(f"dense ring S={S} d={d} rank {rank}")
        R = Rank(1, Hq, Hkv, S, d, cp, rank, "bf16", full=full)
        o, lse = R.ring_fwd()
        idx = np.unique(np.concatenate([[0, n // 2 - 1, n // 2, n - 1], rng.integers(0, n, 12)]))
        O_ref, L_ref = orc.attention_fwd(q64, k64, v64, R.scale, rows=R.pos[idx])
        assert_close(o[:, :, idx], lse[:, :, idx], O_ref, L_ref, "bf16", f"rank {rank}")
        del R, o, lse
        torch.cuda.empty_cache()


@pytest.mark.parametrize("rank", [0, 3])
def test_long_dense_ring_every_row(rank):
    """Every row of one rank of a dense ring of 65536 keys (cp = 4, 4 query
    heads on 1 kv head, d = 128): the 8-wave launch the bench times for its
    131072-token workload, checked in full against the oracle."""
    S, cp, Hq, Hkv, d = 65536, 4, 4, 1, 128
    announce(f"dense ring S={S} rank {rank}, every row (8-wave launch)")
    R = Rank(1, Hq, Hkv, S, d, cp, rank, "bf16", seed=5)
    o, lse = R.ring_fwd()
    O_ref, L_ref = R.oracle()
    assert_close(o, lse, O_ref, L_ref, "bf16", f"rank {rank} every row")


def test_local_only_schedule_fails_parity():
    """Attending only the local shard (the silent no-communication pitfall) is
    rejected by the same tolerance."""
    R = Rank(1, 2, 1, 2048, 128, 4, 3, "bf16", seed=9)
    n = R.S // R.cp
    sl = slice(R.rank * n, (R.rank + 1) * n)
    o, lse = cpa.cp_attn_partial_fwd(R.q_loc, R.k_all[:, :, sl], R.v_all[:, :, sl], R.pos, None, R.allp[sl],
                                     scale=R.scale)
    O_ref, L_ref = R.oracle()
    assert max_err(o, O_ref) > 10 * TOL["bf16"][0]
    assert max_err(lse, L_ref) > 10 * TOL["bf16"][1]


def test_deterministic_reruns():
    R = Rank(1, 4, 2, 2048, 128, 4, 1, "bf16", seed=10)
    o1, l1 = (t.clone() for t in R.ring_fwd())
    o2, l2 = R.ring_fwd()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_empty_inputs():
    d = 128
    q = torch.randn(1, 2, 0, d, device="cuda").bfloat16()
    k = torch.randn(1, 1, 64, d, device="cuda").bfloat16()
    o, lse = cpa.cp_attn_partial_fwd(q, k, k, np.zeros(0), None, np.arange(64), scale=0.1)
    assert o.numel() == 0
    q = torch.randn(1, 2, 10, d, device="cuda").bfloat16()
    k0 = torch.zeros(1, 1, 0, d, device="cuda").bfloat16()
    o, lse = cpa.cp_attn_partial_fwd(q, k0, k0, np.arange(10), None, np.zeros(0), scale=0.1)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_strided_row_views():
    """Q and O as row-range views of larger tensors (legal per the ABI)."""
    B, Hq, Hkv, S, d, cp = 1, 2, 1, 1024, 128, 2
    R = Rank(B, Hq, Hkv, S, d, cp, 0, "bf16", seed=11)
    big = torch.zeros(B, Hq, 2 * (S // cp), d, dtype=torch.bfloat16, device="cuda")
    big[:, :, 3:3 + S // cp] = R.q_loc
    qv = big[:, :, 3:3 + S // cp]
    # row stride stays 16-byte aligned; the base offset of 3 rows (768 B) too
    obig = torch.zeros(B, Hq, S // cp + 8, d, device="cuda")
    ov = obig[:, :, 4:4 + S // cp]
    o, lse = cpa.cp_attn_ring_fwd(qv, R.k_all, R.v_all, cp, 0, R.pos, None, R.allp, scale=R.scale, out=ov)
    assert_close(o, lse, *R.oracle(), "bf16", "views")
    assert torch.all(obig[:, :, :4] == 0) and torch.all(obig[:, :, 4 + S // cp:] == 0)


# ------------------------------------------------------------------ the ring as separate steps
@pytest.mark.parametrize("dtype,cp,S", [("bf16", 4, 2048), ("f32", 2, 1024), ("bf16", 8, 4096)])
def test_ring_fwd_stepwise_matches_oracle(dtype, cp, S):
    """Partial forward + merge per ring step, shards read in place, copied
    step by step into the two-slot stage on a second stream, or copied on the
    compute stream itself: all three match the oracle, and the staged runs are
    bit-identical to the in-place run (the same kernels read the same values,
    so a slot refilled too early would show)."""
    B, Hq, Hkv, d = 1, 8, 2, 128
    full = si.make_qkv(B, Hq, Hkv, S, d, dtype, seed=11)
    for rank in range(cp):
        announce(f"stepwise ring {dtype} cp={cp} S={S} rank {rank}")
        R = Rank(B, Hq, Hkv, S, d, cp, rank, dtype, full=full)
        args = (R.q_loc, R.k_all, R.v_all, cp, rank, R.pos, R.lo, R.allp)
        o0, l0 = cpa.cp_attn_ring_fwd_stepwise(*args, scale=R.scale, staged=False)
        o1, l1 = cpa.cp_attn_ring_fwd_stepwise(*args, scale=R.scale, staged=True)
        o2, l2 = cpa.cp_attn_ring_fwd_stepwise(*args, scale=R.scale, staged=True,
                                               copy_stream=torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert torch.equal(o1, o0) and torch.equal(l1, l0)
        assert torch.equal(o2, o0) and torch.equal(l2, l0)
        assert_close(o0, l0, *R.oracle(), dtype, f"stepwise rank {rank}")


def test_ring_fwd_stepwise_varlen_and_replay():
    """Packed documents (stream deal), and one plan replayed: every replay of
    the staged plan equals the first run bit for bit and the oracle."""
    cp = 4
    L = si.doc_lengths(total=4096, mean=400, sigma=1.0, lo=16, hi=3000, seed=12)
    cu = si.cu_seqlens_from_lengths(L)
    S = int(cu[-1])
    full = si.make_qkv(1, 4, 2, S, 64, "bf16", seed=13)
    for rank in (0, 3):
        announce(f"stepwise ring varlen rank {rank} ({len(L)} docs), replays")
        R = Rank(1, 4, 2, S, 64, cp, rank, "bf16", full=full, cu=cu)
        plan = cpa.RingFwdStepwisePlan(R.q_loc, R.k_all, R.v_all, cp, rank, R.pos, R.lo, R.allp, scale=R.scale)
        o, lse = plan.run()
        o_first, l_first = o.clone(), lse.clone()
        for _ in range(3):
            plan.run()
        torch.cuda.synchronize()
        assert torch.equal(plan.out, o_first) and torch.equal(plan.lse, l_first)
        assert_close(o_first, l_first, *R.oracle(), "bf16", f"stepwise varlen rank {rank}")


@pytest.mark.parametrize("mode", [cpa.CP_STREAM, cpa.CP_WHOLE_DOC])
def test_ring_shuffled_rows_and_keys(mode):
    """Packed documents with the rank's rows in random order and the keys of
    every shard in random order: tile bounds, key gaps and row holes must not
    assume ascending positions (a hole found between adjacent rows is checked
    against every row)."""
    cp, S = 4, 4096
    L = si.doc_lengths(total=S, mean=300, sigma=1.0, lo=16, hi=2000, seed=21)
    cu = si.cu_seqlens_from_lengths(L)
    full = si.make_qkv(1, 4, 2, S, 64, "bf16", seed=22)
    rng = np.random.default_rng(23)
    for rank in (0, 2):
        announce(f"shuffled rows/keys mode {mode} rank {rank}")
        R = Rank(1, 4, 2, S, 64, cp, rank, "bf16", full=full, cu=cu, mode=mode)
        pq = rng.permutation(len(R.pos))
        R.pos, R.lo = R.pos[pq], R.lo[pq]
        R.q_loc = R.q_loc[:, :, torch.from_numpy(pq)].contiguous()
        n = S // cp
        pk = np.concatenate([s * n + rng.permutation(n) for s in range(cp)])
        R.allp = R.allp[pk]
        R.k_all = R.k_all[:, :, torch.from_numpy(pk)].contiguous()
        R.v_all = R.v_all[:, :, torch.from_numpy(pk)].contiguous()
        o, lse = R.ring_fwd()
        assert_close(o, lse, *R.oracle(), "bf16", f"shuffled rank {rank}")
