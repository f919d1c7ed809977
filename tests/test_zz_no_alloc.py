"""GPU parity of the allocation-free forward (cp_attn_ring_fwd_noalloc, its
tile tables in the library's static per-device scratch) against the
workspace entry point cp_attn_ring_fwd on the same inputs, through the C ABI:
two calls in a row, the second on a smaller ring than the first, each equal
to cp_attn_ring_fwd bit for bit (the same kernels' arithmetic; V read in place
instead of from its transposed copy) and within the acceptance bars of the
oracle on sampled rows."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
import context_causal_attention_amd as cpa
from gpu_cases import Rank, announce, assert_close

pytestmark = pytest.mark.gpu


def _noalloc(R, out_dtype=torch.float32):
    out = torch.empty(R.q_loc.shape, dtype=out_dtype, device="cuda")
    lse = torch.empty(R.q_loc.shape[:3], dtype=torch.float32, device="cuda")
    return cpa.cp_attn_ring_fwd_noalloc(R.q_loc, R.k_all, R.v_all, R.cp, R.rank, R.pos, R.lo, R.allp, out, lse,
                                        scale=R.scale)


def test_noalloc_matches_workspace_entry_two_calls():
    # first: a dense ring of 65536 keys (the wide launch: the workspace entry
    # reads a transposed copy of V, this one reads V in place)
    announce("noalloc ring fwd: 65536 keys, cp=4, rank 3")
    big = Rank(1, 4, 1, 65536, 128, 4, 3, "bf16", seed=41)
    o1, l1 = _noalloc(big)
    r1, rl1 = big.ring_fwd()
    torch.cuda.synchronize()
    assert torch.equal(o1, r1) and torch.equal(l1, rl1)
    rng = np.random.default_rng(4)
    idx = np.unique(np.concatenate([[0, len(big.pos) - 1], rng.integers(0, len(big.pos), 12)]))
    O_ref, L_ref = big.oracle(idx)
    assert_close(o1[:, :, idx], l1[:, :, idx], O_ref, L_ref, "bf16", "noalloc 65536 keys")
    # second: a smaller ring with packed documents (the scratch keeps the first
    # call's larger tables; every entry this call reads is rewritten)
    announce("noalloc ring fwd: 4096 packed tokens, cp=4, rank 1, bf16 output")
    cu = si.cu_seqlens_from_lengths(si.doc_lengths(total=4096, mean=400, sigma=1.0, lo=16, hi=3000, seed=42))
    small = Rank(1, 4, 2, 4096, 64, 4, 1, "bf16", seed=43, cu=cu, mode=cpa.CP_WHOLE_DOC)
    o2, l2 = _noalloc(small, torch.bfloat16)
    r2, rl2 = small.ring_fwd(out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o2, r2) and torch.equal(l2, rl2)
    assert_close(o2, l2, *small.oracle(), "bf16", "noalloc packed documents")


def test_noalloc_without_key_lists():
    """Rows whose per-query-tile key lists do not fit the static scratch (1024
    query tiles x 1024 key tiles x 4 bytes beside the tables): the
    allocation-free call then lets each workgroup list its key tiles, the
    workspace entry reads the precomputed lists; the two agree bit for bit and
    with the oracle on sampled rows."""
    announce("noalloc ring fwd without key lists: 65536 packed tokens, cp=1, every row twice")
    cu = si.cu_seqlens_from_lengths(si.doc_lengths(total=65536, mean=1500, sigma=1.0, lo=16, hi=16384, seed=44))
    R = Rank(1, 2, 1, 65536, 64, 1, 0, "bf16", seed=45, cu=cu, mode=cpa.CP_STREAM)
    # 131072 query rows: the rank's rows twice (1024 query tiles of 128 rows)
    R.pos, R.lo = np.concatenate([R.pos, R.pos]), np.concatenate([R.lo, R.lo])
    R.q_loc = torch.cat([R.q_loc, R.q_loc], dim=2).contiguous()
    o1, l1 = _noalloc(R)
    r1, rl1 = R.ring_fwd()
    torch.cuda.synchronize()
    assert torch.equal(o1, r1) and torch.equal(l1, rl1)
    rng = np.random.default_rng(5)
    n = len(R.pos)
    idx = np.unique(np.concatenate([[0, n // 2 - 1, n // 2, n - 1], rng.integers(0, n, 24)]))
    O_ref, L_ref = R.oracle(idx)
    assert_close(o1[:, :, idx], l1[:, :, idx], O_ref, L_ref, "bf16", "noalloc without key lists")


def test_noalloc_fp32_and_size_limit():
    announce("noalloc ring fwd: fp32, 1024 tokens, cp=2")
    w = si.WORKLOADS["c0_f32_s1024_cp2"]
    for rank in range(w.cp):
        R = Rank(w.B, w.Hq, w.Hkv, w.S, w.d, w.cp, rank, "f32", seed=w.seed)
        o, lse = _noalloc(R)
        ro, rl = R.ring_fwd()
        torch.cuda.synchronize()
        assert torch.equal(o, ro) and torch.equal(lse, rl)
        assert_close(o, lse, *R.oracle(), "f32", f"noalloc fp32 rank {rank}")
    # a ring whose tables exceed the static scratch is rejected before any launch
    n = 1 << 21  # 2^21 keys: 32768 tiles x 272 bytes > 4 MiB
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 1, n, 64, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(1, 1, 64, 64, device="cuda")
    lse = torch.empty(1, 1, 64, device="cuda")
    pos = np.arange(64)
    kp = np.arange(n)
    with pytest.raises(ValueError, match="static scratch"):
        cpa.cp_attn_ring_fwd_noalloc(q, k, k, 2, 0, pos, None, kp, out, lse, scale=0.1)
