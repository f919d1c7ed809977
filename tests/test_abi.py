"""CPU tests of the C ABI: the library loads and exports every declared symbol,
the host index builder is bit-exact against the oracle's deal, and invalid
arguments return error codes before anything is launched (so they need no GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import oracle as orc
import seeded_inputs as si
import context_causal_attention_amd as cpa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "cpattn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cp_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = cpa.lib()
    names = _declared_functions()
    # The boundary's calls: the index map, one step, the merge, the whole ring and
    # its workspace query, the backward, then the stepwise ring and the head exchange.
    for must in ("cp_shard_zigzag", "cp_unshard_zigzag", "cp_varlen_index", "cp_ring_source", "cp_pairs",
                 "cp_attn_partial_fwd", "cp_attn_merge", "cp_attn_ring_fwd", "cp_attn_ring_fwd_workspace",
                 "cp_attn_bwd_delta", "cp_attn_partial_bwd", "cp_attn_ring_bwd", "cp_last_error", "cp_version",
                 "cp_attn_ring_fwd_stepwise", "cp_a2a_pack", "cp_a2a_unpack"):
        assert must in names
    assert "cp_attn_fwd_workspace" not in names
    for n in names:
        assert hasattr(L, n), f"{n} declared in cpattn.h but not exported"
    assert cpa.cp_version() >= 100


@pytest.mark.parametrize("S,cp", [(1024, 2), (32768, 8), (64, 1), (48, 3), (16, 8), (131072, 8)])
def test_shard_zigzag_bit_exact(S, cp):
    for r in range(cp):
        assert np.array_equal(cpa.cp_shard_zigzag(S, cp, r), orc.zigzag_positions(S, cp, r))
    perm = cpa.cp_unshard_zigzag(S, cp)
    assert np.array_equal(perm, orc.all_rank_positions(S, cp))
    assert np.array_equal(np.sort(perm), np.arange(S))


def test_seq_multiple_rule_and_argument_errors():
    with pytest.raises(ValueError, match="multiple of 2"):
        cpa.cp_shard_zigzag(1000, 8, 0)
    with pytest.raises(ValueError, match="rank"):
        cpa.cp_shard_zigzag(1024, 2, 2)
    with pytest.raises(ValueError, match="cp must be"):
        cpa.cp_shard_zigzag(1024, 0, 0)
    with pytest.raises(ValueError):
        cpa.cp_unshard_zigzag(30, 4)
    assert cpa.lib().cp_shard_zigzag(1024, 2, 0, None) == cpa.CP_EINVAL


def test_cp_one_is_identity():
    assert np.array_equal(cpa.cp_shard_zigzag(64, 1, 0), np.arange(64))


def test_ring_source():
    for cp in (1, 2, 3, 8):
        for r in range(cp):
            srcs = [cpa.cp_ring_source(cp, r, t) for t in range(cp)]
            assert srcs[0] == r and sorted(srcs) == list(range(cp))
            assert all(s == (r - t) % cp for t, s in enumerate(srcs))
    with pytest.raises(ValueError):
        cpa.cp_ring_source(4, 0, 4)
    with pytest.raises(ValueError):
        cpa.cp_ring_source(0, 0, 0)


@pytest.mark.parametrize("cp", [1, 2, 3, 5, 8, 16])
def test_pairs_balance(cp):
    c = 7
    S = 2 * cp * c
    allp = cpa.cp_unshard_zigzag(S, cp)
    for r in range(cp):
        pos = cpa.cp_shard_zigzag(S, cp, r)
        assert cpa.cp_pairs(pos, None, allp) == S * (S + 1) // (2 * cp)


def test_pairs_matches_oracle_random():
    rng = np.random.default_rng(3)
    for _ in range(10):
        qp = rng.integers(0, 500, 100)
        ql = np.minimum(qp, rng.integers(0, 500, 100))
        kp = rng.integers(0, 500, 80)
        assert cpa.cp_pairs(qp, ql, kp) == orc.pair_count(qp, ql, kp)


def test_varlen_stream_index_matches_oracle():
    L = si.doc_lengths()
    cu = si.cu_seqlens_from_lengths(L)
    S = int(cu[-1])
    allp = cpa.cp_unshard_zigzag(S, 4)
    for r in range(4):
        pos, lo = cpa.cp_varlen_index(cu, 4, r, cpa.CP_STREAM)
        assert np.array_equal(pos, orc.zigzag_positions(S, 4, r))
        assert np.array_equal(lo, orc.doc_start_of(pos, cu))
        assert cpa.cp_pairs(pos, lo, allp) == orc.pair_count(pos, lo, allp)


def test_varlen_per_doc_index():
    cp = 2
    lengths = np.array([8, 4, 12, 0, 8])
    cu = si.cu_seqlens_from_lengths(lengths)
    S = int(cu[-1])
    got = [cpa.cp_varlen_index(cu, cp, r, cpa.CP_PER_DOC) for r in range(cp)]
    allpos = np.concatenate([g[0] for g in got])
    assert np.array_equal(np.sort(allpos), np.arange(S))
    for r, (pos, lo) in enumerate(got):
        assert np.array_equal(lo, orc.doc_start_of(pos, cu))
        # per document: chunk r then chunk 2cp-1-r of that document
        off = 0
        for d in range(len(lengths)):
            n = lengths[d]
            if n == 0:
                continue
            sub = orc.zigzag_positions(n, cp, r) + cu[d]
            assert np.array_equal(pos[off:off + n // cp], sub)
            off += n // cp
    # every rank gets the same number of causal pairs inside documents
    kp = np.arange(S)
    counts = [cpa.cp_pairs(p, l, kp) for p, l in got]
    assert len(set(counts)) == 1
    with pytest.raises(ValueError, match="multiple of 2"):
        cpa.cp_varlen_index([0, 6, 16], 2, 0, cpa.CP_PER_DOC)


def test_varlen_deals_balance_at_workload_size():
    """The 65536-token documents rounded to multiples of 2cp: the per-document
    deal gives every rank the same causal work, the stream deal does not; the
    library's pair counts equal the oracle's for both."""
    w = si.WORKLOADS["varlen8_s64k_cp4"]
    cu = si.workload_cu_seqlens(w)
    assert np.all(np.diff(cu) % (2 * w.cp) == 0)
    counts = {}
    for mode in (cpa.CP_STREAM, cpa.CP_PER_DOC):
        every = [cpa.cp_varlen_index(cu, w.cp, r, mode) for r in range(w.cp)]
        allp = np.concatenate([e[0] for e in every])
        assert np.array_equal(np.sort(allp), np.arange(w.S))
        got = [cpa.cp_pairs(p, l, allp) for p, l in every]
        ref = [orc.pair_count(p, orc.doc_start_of(p, cu), np.arange(w.S)) for p, _ in every]
        assert got == ref
        counts[mode] = got
    assert len(set(counts[cpa.CP_PER_DOC])) == 1
    assert sum(counts[cpa.CP_PER_DOC]) == sum(counts[cpa.CP_STREAM])
    assert max(counts[cpa.CP_STREAM]) > 1.2 * min(counts[cpa.CP_PER_DOC])


@pytest.mark.parametrize("cp,seed", [(2, 5), (3, 6), (4, 7), (8, 8)])
def test_varlen_whole_doc_index_matches_oracle(cp, seed):
    total = 2 * cp * 1500
    L = si.doc_lengths(total=total, mean=350, sigma=1.0, lo=8, hi=3000, seed=seed)
    cu = si.cu_seqlens_from_lengths(L)
    ref = orc.whole_doc_deal(cu, cp)
    for r in range(cp):
        pos, lo = cpa.cp_varlen_index(cu, cp, r, cpa.CP_WHOLE_DOC)
        assert np.array_equal(pos, ref[r])
        assert np.array_equal(lo, orc.doc_start_of(pos, cu))


def test_varlen_whole_doc_at_workload_size():
    """The 65536-token packed documents (cp = 4): the whole-document deal
    matches the oracle and keeps the causal work within 3% of the mean."""
    w = si.WORKLOADS["varlen_s64k_cp4"]
    cu = si.workload_cu_seqlens(w)
    ref = orc.whole_doc_deal(cu, w.cp)
    every = [cpa.cp_varlen_index(cu, w.cp, r, cpa.CP_WHOLE_DOC) for r in range(w.cp)]
    for (pos, _), rp in zip(every, ref):
        assert np.array_equal(pos, rp)
    allp = np.concatenate([e[0] for e in every])
    work = [cpa.cp_pairs(p, l, allp) for p, l in every]
    assert work == [orc.pair_count(p, orc.doc_start_of(p, cu), allp) for p, _ in every]
    assert max(work) <= 1.03 * (sum(work) / len(work))


def test_varlen_errors():
    with pytest.raises(ValueError, match="must be 0"):
        cpa.cp_varlen_index([1, 8], 2, 0)
    with pytest.raises(ValueError, match="decreases"):
        cpa.cp_varlen_index([0, 8, 4, 16], 2, 0)
    with pytest.raises(ValueError, match="multiple of 2"):
        cpa.cp_varlen_index([0, 5, 10], 2, 0)
    with pytest.raises(ValueError, match="shard mode"):
        cpa.cp_varlen_index([0, 8], 2, 0, mode=7)


# ------------------------------------------------------------------ device-call validation (no launch)
def _shape(**kw):
    s = cpa.CpShape()
    s.b, s.hq, s.hkv, s.d = kw.get("b", 1), kw.get("hq", 4), kw.get("hkv", 2), kw.get("d", 128)
    s.sq, s.sk = kw.get("sq", 256), kw.get("sk", 512)
    s.scale = kw.get("scale", 0.088)
    s.in_dtype, s.out_dtype = kw.get("in_dtype", cpa.CP_BF16), kw.get("out_dtype", cpa.CP_F32)
    d = s.d
    s.q_str = (ctypes.c_int64 * 3)(s.hq * s.sq * d, s.sq * d, kw.get("q_row", d))
    s.k_str = (ctypes.c_int64 * 3)(s.hkv * s.sk * d, s.sk * d, d)
    s.v_str = (ctypes.c_int64 * 3)(s.hkv * s.sk * d, s.sk * d, d)
    s.o_str = (ctypes.c_int64 * 3)(s.hq * s.sq * d, s.sq * d, d)
    return s


FAKE = 0x10000  # 16-byte aligned non-null address; never dereferenced (validation fails first)


def _ring(s, cp=2, rank=0, ws=FAKE, ws_bytes=1 << 40, q=FAKE, qpos=FAKE):
    L = cpa.lib()
    return L.cp_attn_ring_fwd(ctypes.byref(s) if s is not None else None, cp, rank, q, FAKE, FAKE, qpos, None,
                              FAKE, FAKE, FAKE, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(hq=3, hkv=2), cpa.CP_EINVAL),
    (dict(d=96), cpa.CP_EINVAL),
    (dict(d=256), cpa.CP_EINVAL),
    (dict(b=0), cpa.CP_EINVAL),
    (dict(scale=0.0), cpa.CP_EINVAL),
    (dict(scale=float("nan")), cpa.CP_EINVAL),
    (dict(in_dtype=7), cpa.CP_EDTYPE),
    (dict(out_dtype=3), cpa.CP_EDTYPE),
    (dict(q_row=129), cpa.CP_EINVAL),
    (dict(sk=502), cpa.CP_ESHAPE),
])
def test_ring_fwd_rejects_bad_shapes(kw, code):
    assert _ring(_shape(**kw)) == code
    assert cpa.cp_last_error() != ""


def test_ring_fwd_rejects_bad_args():
    s = _shape()
    assert _ring(None) == cpa.CP_EINVAL
    assert _ring(s, cp=0) == cpa.CP_EINVAL
    assert _ring(s, rank=2) == cpa.CP_EINVAL
    assert _ring(s, rank=-1) == cpa.CP_EINVAL
    assert _ring(s, q=0) == cpa.CP_EINVAL
    assert _ring(s, q=FAKE + 8) == cpa.CP_EINVAL
    assert _ring(s, qpos=0) == cpa.CP_EINVAL
    assert _ring(s, ws=0) == cpa.CP_EWORKSPACE
    assert _ring(s, ws=FAKE + 16) == cpa.CP_EWORKSPACE
    need = cpa.lib().cp_attn_ring_fwd_workspace(ctypes.byref(s), 2)
    assert need > 0
    assert _ring(s, ws_bytes=need - 1) == cpa.CP_EWORKSPACE


def test_ring_fwd_rejects_keys_beyond_one_buffer_descriptor():
    # The bf16 kernel reads one (batch, kv head) of K and of V through 32-bit
    # buffer offsets.  A row stride that stretches 2^22 keys of K beyond 4 GiB:
    s = _shape(sk=1 << 22, hkv=1, hq=1)
    s.k_str[2] = 1024
    assert _ring(s, cp=8) == cpa.CP_EINVAL
    assert "4 GiB" in cpa.cp_last_error()
    # The same for V alone (K rows of d elements stay inside the reach).
    s = _shape(sk=1 << 22, hkv=1, hq=1)
    s.v_str[2] = 1024
    assert _ring(s, cp=8) == cpa.CP_EINVAL
    assert "4 GiB" in cpa.cp_last_error()
    # 16777200 keys of d = 128 (row stride d, cp = 8): K and V take 4294963200
    # bytes each, inside the reach, but the transposed V copy of the wide
    # launch (rings of >= 65536 keys) over the padded tiles (8 x 32768 tiles
    # of 64 keys) takes 2^32 bytes.
    s = _shape(sk=16777200, hkv=1, hq=1)
    assert _ring(s, cp=8) == cpa.CP_EINVAL
    assert "V^T" in cpa.cp_last_error()


def _stepwise(s, cp=2, rank=0, ws=FAKE, ws_bytes=1 << 40, stage=None, stage_bytes=0, o=FAKE):
    return cpa.lib().cp_attn_ring_fwd_stepwise(ctypes.byref(s), cp, rank, FAKE, FAKE, FAKE, FAKE, None, FAKE, o,
                                               FAKE, ws, ws_bytes, stage, stage_bytes, None, None)


def test_ring_fwd_stepwise_validation():
    L = cpa.lib()
    s = _shape()
    need = L.cp_attn_ring_fwd_stepwise_workspace(ctypes.byref(s), 2)
    # Only the step kernel's tables: every later step merges into (o, lse) in
    # its epilogue, so no partial is stored.  That is the one-step forward's
    # workspace over one shard of sk / cp = 256 keys.
    one = _shape(sk=256)
    assert need == L.cp_attn_ring_fwd_workspace(ctypes.byref(one), 1) > 0
    # two slots of K and V, one shard each: 2 kv heads x 256 rows x 128 x bf16
    assert L.cp_attn_ring_stage_bytes(ctypes.byref(s), 2) == 4 * 2 * 256 * 128 * 2
    assert L.cp_attn_ring_fwd_stepwise_workspace(ctypes.byref(_shape(d=96)), 2) == 0
    assert _stepwise(_shape(out_dtype=cpa.CP_BF16)) == cpa.CP_EDTYPE
    t = _shape()
    t.o_str = (ctypes.c_int64 * 3)(4 * 256 * 256, 256 * 256, 256)  # rows padded: not contiguous
    assert _stepwise(t) == cpa.CP_EINVAL
    assert _stepwise(_shape(sk=510)) == cpa.CP_ESHAPE
    assert _stepwise(s, rank=2) == cpa.CP_EINVAL
    assert _stepwise(s, cp=0) == cpa.CP_EINVAL
    assert _stepwise(s, ws=0) == cpa.CP_EWORKSPACE
    assert _stepwise(s, ws=FAKE + 16) == cpa.CP_EWORKSPACE
    assert _stepwise(s, ws_bytes=need - 1) == cpa.CP_EWORKSPACE
    st = L.cp_attn_ring_stage_bytes(ctypes.byref(s), 2)
    assert _stepwise(s, ws_bytes=need, stage=FAKE, stage_bytes=st - 1) == cpa.CP_EWORKSPACE
    assert _stepwise(s, ws_bytes=need, stage=FAKE + 16, stage_bytes=st) == cpa.CP_EWORKSPACE
    u = _shape()
    u.k_str = (ctypes.c_int64 * 3)(2 * 512 * 256, 512 * 256, 256)  # K rows strided: cannot be staged by rows
    assert _stepwise(u, ws_bytes=need, stage=FAKE, stage_bytes=st) == cpa.CP_EINVAL
    assert _stepwise(s, o=FAKE + 8) == cpa.CP_EINVAL
    assert _stepwise(_shape(sq=0)) == cpa.CP_OK  # no query rows: nothing to do, nothing launched


def test_a2a_validation():
    L = cpa.lib()
    ok = dict(g=2, heads=32, rows=64, d=128, dtype=cpa.CP_BF16)

    def pack(**kw):
        a = dict(ok, **kw)
        return L.cp_a2a_pack(a["g"], a["heads"], a["rows"], a["d"], a["dtype"], kw.get("x", FAKE),
                             kw.get("rs", 32 * 128), kw.get("send", FAKE), 0, None)

    def unpack(**kw):
        a = dict(ok, **kw)
        return L.cp_a2a_unpack(a["g"], a["heads"], a["rows"], a["d"], a["dtype"], kw.get("recv", FAKE),
                               kw.get("y", FAKE), 1, None)

    for f in (pack, unpack):
        assert f(g=0) == cpa.CP_EINVAL
        assert f(g=3) == cpa.CP_EINVAL          # 32 heads not a multiple of 3
        assert f(heads=0) == cpa.CP_EINVAL
        assert f(heads=70000, g=1) == cpa.CP_EINVAL
        assert f(rows=-1) == cpa.CP_EINVAL
        assert f(d=96) == cpa.CP_EINVAL
        assert f(dtype=9) == cpa.CP_EDTYPE
        assert f(rows=0) == cpa.CP_OK        # nothing to move, nothing launched
    assert pack(rs=32 * 128 - 8) == cpa.CP_EINVAL   # row stride below heads*d
    assert pack(rs=32 * 128 + 1) == cpa.CP_EINVAL   # not a multiple of 16 bytes
    assert pack(x=0) == cpa.CP_EINVAL
    assert pack(send=FAKE + 8) == cpa.CP_EINVAL
    assert unpack(y=0) == cpa.CP_EINVAL
    assert unpack(recv=FAKE + 4) == cpa.CP_EINVAL


def test_workspace_query():
    # 131072 keys: the wide launch's V^T copy (8 heads x 128 x 131072 x 2 B),
    # then per 64-key tile its bounds (16 B) and 64 padded key positions
    # and per 128-row query tile two ints (listed key tiles, dispatch order)
    s = _shape(sk=131072, sq=16384, hq=32, hkv=8)
    n = cpa.lib().cp_attn_ring_fwd_workspace(ctypes.byref(s), 8)
    tiles = 131072 // 64
    assert n == tiles * 16 + tiles * 64 * 4 + 2 * 128 * 4 + 8 * 128 * 131072 * 2
    # 32768 keys read V in place: the tables, then per 128-row query tile one
    # int per ring key tile (the key tiles a document-masked launch lists)
    s = _shape(sk=32768, sq=4096, hq=32, hkv=8)
    tiles = 32768 // 64
    assert cpa.lib().cp_attn_ring_fwd_workspace(ctypes.byref(s), 8) == tiles * 16 + tiles * 64 * 4 + 256 + 32 * tiles * 4
    # one query tile: no dispatch order, hence no lists
    s = _shape(sk=32768, sq=128, hq=32, hkv=8)
    assert cpa.lib().cp_attn_ring_fwd_workspace(ctypes.byref(s), 8) == tiles * 16 + tiles * 64 * 4 + 256
    assert cpa.lib().cp_attn_ring_fwd_workspace(ctypes.byref(_shape(d=96)), 8) == 0


def test_merge_and_partial_validation():
    L = cpa.lib()
    assert L.cp_attn_merge(-1, 128, FAKE, FAKE, FAKE, FAKE, None) == cpa.CP_EINVAL
    assert L.cp_attn_merge(16, 96, FAKE, FAKE, FAKE, FAKE, None) == cpa.CP_EINVAL
    assert L.cp_attn_merge(16, 128, 0, FAKE, FAKE, FAKE, None) == cpa.CP_EINVAL
    assert L.cp_attn_merge(0, 128, FAKE, FAKE, FAKE, FAKE, None) == cpa.CP_OK
    s = _shape(hq=5, hkv=2)
    assert L.cp_attn_partial_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                                 1 << 30, None) == cpa.CP_EINVAL


def test_python_wrappers_raise_value_error():
    q = torch.zeros(1, 2, 8, 96)
    with pytest.raises(ValueError):
        cpa.cp_attn_ring_fwd_workspace(q, q, q, 1)
    with pytest.raises(ValueError):
        cpa.cp_attn_merge(torch.zeros(4, 64), torch.zeros(3), torch.zeros(4, 64), torch.zeros(4))


# ------------------------------------------------------------------ backward validation (no launch)
def _ring_bwd(s, cp=2, rank=0, ws=FAKE, ws_bytes=1 << 40, q=FAKE, dout=FAKE, lse=FAKE, dk=FAKE):
    L = cpa.lib()
    return L.cp_attn_ring_bwd(ctypes.byref(s) if s is not None else None, cp, rank, q, FAKE, FAKE, dout, lse, FAKE,
                              FAKE, None, FAKE, FAKE, dk, FAKE, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(hq=3, hkv=2), cpa.CP_EINVAL),
    (dict(d=96), cpa.CP_EINVAL),
    (dict(scale=-1.0), cpa.CP_EINVAL),
    (dict(in_dtype=cpa.CP_F32), cpa.CP_EDTYPE),
    (dict(q_row=129), cpa.CP_EINVAL),
    (dict(sk=502), cpa.CP_ESHAPE),
])
def test_ring_bwd_rejects_bad_shapes(kw, code):
    assert _ring_bwd(_shape(**kw)) == code
    assert cpa.cp_last_error() != ""


def test_ring_bwd_rejects_bad_args():
    s = _shape()
    assert _ring_bwd(None) == cpa.CP_EINVAL
    assert _ring_bwd(s, cp=0) == cpa.CP_EINVAL
    assert _ring_bwd(s, rank=2) == cpa.CP_EINVAL
    assert _ring_bwd(s, q=0) == cpa.CP_EINVAL
    assert _ring_bwd(s, dout=FAKE + 4) == cpa.CP_EINVAL
    assert _ring_bwd(s, lse=0) == cpa.CP_EINVAL
    assert _ring_bwd(s, dk=0) == cpa.CP_EINVAL
    assert _ring_bwd(s, ws=0) == cpa.CP_EWORKSPACE
    assert _ring_bwd(s, ws=FAKE + 16) == cpa.CP_EWORKSPACE
    need = cpa.lib().cp_attn_bwd_workspace(ctypes.byref(s), 2)
    assert need > 0
    assert _ring_bwd(s, ws_bytes=need - 1) == cpa.CP_EWORKSPACE


def test_ring_bwd_rejects_v_rows_beyond_32_bit_offsets():
    # The dK/dV kernel reads 256 rows of V through one buffer descriptor:
    # a V row stride of 2^22 elements puts them 2 GiB apart.
    s = _shape()
    s.v_str[2] = 1 << 22
    assert _ring_bwd(s) == cpa.CP_EINVAL
    assert "32-bit" in cpa.cp_last_error()


def test_bwd_workspace_query():
    s = _shape(sk=131072, sq=16384, hq=32, hkv=8)
    n = cpa.lib().cp_attn_bwd_workspace(ctypes.byref(s), 8)
    # per-row tables (-LSE log2 e and delta for 32 heads x 16384 rows, document
    # start and span) and per-key tables (bounds, padded positions)
    rows = 2 * 32 * 16384 * 4 + 2 * 16384 * 4
    keys = 131072 * 4
    assert rows + keys <= n < rows + keys + (1 << 20)
    assert cpa.lib().cp_attn_bwd_workspace(ctypes.byref(_shape(d=96)), 8) == 0


def test_bwd_delta_and_partial_validation():
    L = cpa.lib()
    s = _shape()
    assert L.cp_attn_bwd_delta(ctypes.byref(_shape(in_dtype=cpa.CP_F32)), FAKE, FAKE, FAKE, None) == cpa.CP_EDTYPE
    assert L.cp_attn_bwd_delta(ctypes.byref(s), 0, FAKE, FAKE, None) == cpa.CP_EINVAL
    assert L.cp_attn_bwd_delta(ctypes.byref(s), FAKE, FAKE, 0, None) == cpa.CP_EINVAL
    assert L.cp_attn_bwd_delta(ctypes.byref(_shape(sq=0)), 0, 0, 0, None) == cpa.CP_OK
    # 2^31 rows or more (the kernel's row index is 32-bit)
    assert L.cp_attn_bwd_delta(ctypes.byref(_shape(b=4, hq=512, hkv=512, sq=1 << 20)), FAKE, FAKE, FAKE,
                               None) == cpa.CP_EINVAL
    assert "2^31" in cpa.cp_last_error()
    s5 = _shape(hq=5, hkv=2)
    assert L.cp_attn_partial_bwd(ctypes.byref(s5), *([FAKE] * 6), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 1 << 30, None) == cpa.CP_EINVAL
    # no query rows or no keys: nothing to add, and nothing is read
    assert L.cp_attn_partial_bwd(ctypes.byref(_shape(sq=0)), *([0] * 6), 0, None, 0, 0, 0, 0, 0, 0,
                                 None) == cpa.CP_OK


def test_bwd_python_wrappers_raise_value_error():
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        cpa.cp_attn_bwd_workspace(torch.zeros(1, 2, 8, 96), torch.zeros(1, 2, 8, 96), torch.zeros(1, 2, 8, 96))
    with pytest.raises(ValueError):  # dout strides differ from q's
        cpa.cp_attn_partial_bwd(q, q, q, q.transpose(1, 2).contiguous().transpose(1, 2), torch.zeros(1, 2, 8),
                                torch.zeros(1, 2, 8), [0] * 8, None, [0] * 8)
