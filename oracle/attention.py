"""fp64 CPU oracle for causal context-parallel (zigzag ring) attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares no
code with the HIP library (``context_causal_attention_amd``) and imports nothing
from it; the only thing both sides use is the seeded input generator in
``seeded_inputs``, which holds none of the method's arithmetic.

What it computes, and where the pages fix it
--------------------------------------------
* Sharding Q, K and V along the sequence dimension, Q_i staying on its rank and
  each rank attending its Q_i to every K_j/V_j shard, then combining the partial
  results: Accelerate concept guide "Context Parallel in accelerate", sections
  "Technical details" and "So how does it work?" (the pseudocode there).
* Cutting the sequence into 2*cp chunks: the sequence length must be a multiple
  of 2*context_parallel_size (NeMo Megatron-Bridge "Hierarchical Context
  Parallel Skill", section "Required constraints").  Which two chunks a rank
  holds (chunk r and chunk 2*cp-1-r, the "zigzag" deal) is not printed on any
  page; it is the plainest deal that balances causal work, which static
  sharding does not (FlashCP abstract).
* Everything inside ``attn(...)`` and ``combine(...)`` is plain softmax
  attention written out from its definition: s = scale * q.k, a causal (and, for
  packed documents, block-diagonal) mask, softmax over the allowed keys, the
  weighted sum of values, and LSE = log of the softmax normaliser (natural log).
  The pages name ``combine`` but give no formula; the LSE-weighted merge used
  here is the exact identity that recombines softmax over a union of disjoint
  key sets.

Every function is a direct transcription of a definition: row-blocking of the
fp64 matmuls is the only restructuring, and rows are independent, so it does
not change the arithmetic being checked.

Pins (tests/test_oracle.py) tie each function to something other than itself:
brute-force scalar loops, closed forms, torch fp64 SDPA and autograd, finite
differences and the pair-count balance identity.  No function here is
"parity unpinned".
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "zigzag_positions",
    "all_rank_positions",
    "doc_start_of",
    "doc_end_of",
    "causal_piece_work",
    "whole_doc_deal",
    "allowed_mask",
    "pair_count",
    "attention_fwd",
    "partial_attention_fwd",
    "lse_merge",
    "bwd_delta",
    "attention_bwd",
    "partial_attention_bwd",
    "a2a_pack",
    "a2a_unpack_pack",
    "a2a_exchange",
    "a2a_unpack",
    "a2a_pack_unpack",
    "ring_partials_fwd",
    "per_doc_positions",
    "attention_matrix_bytes",
]


# --------------------------------------------------------------------------
# Sharding: which global sequence positions a rank holds
# --------------------------------------------------------------------------
def zigzag_positions(S: int, cp: int, rank: int) -> np.ndarray:
    """Global positions held by ``rank``: chunk ``rank`` then chunk ``2cp-1-rank``.

    The sequence is cut into 2*cp equal chunks (length must divide, per the
    "Required constraints" of the hierarchical-CP skill page).  cp == 1 gives the
    identity (the Accelerate plugin treats a CP size of 1 as CP switched off).
    """
    if cp < 1 or not (0 <= rank < cp):
        raise ValueError("need cp >= 1 and 0 <= rank < cp")
    if S % (2 * cp) != 0:
        raise ValueError("sequence length must be a multiple of 2*cp")
    c = S // (2 * cp)
    first = np.arange(rank * c, (rank + 1) * c, dtype=np.int64)
    second_chunk = 2 * cp - 1 - rank
    second = np.arange(second_chunk * c, (second_chunk + 1) * c, dtype=np.int64)
    return np.concatenate([first, second])


def all_rank_positions(S: int, cp: int) -> np.ndarray:
    """Rank-major concatenation of every rank's positions (what gathering all
    shards yields, as in the guide's "all-gather" section)."""
    return np.concatenate([zigzag_positions(S, cp, r) for r in range(cp)])


# --------------------------------------------------------------------------
# Masks
# --------------------------------------------------------------------------
def causal_piece_work(doc_start: int, a: int, b: int) -> int:
    """Causal (query, key) pairs of rows [a, b) of a document that starts at
    doc_start: row p attends the p - doc_start + 1 positions doc_start..p."""
    return sum(p - doc_start + 1 for p in range(a, b))


def whole_doc_deal(cu_seqlens, cp: int):
    """Whole-document placement: an own design.  The FlashCP abstract names
    Whole-Doc sharding (entire documents on one rank) next to Per-Doc, but
    gives no algorithm; this is a plain greedy under the ring's constraint
    that every rank holds S/cp positions.

    Documents are taken longest first (ties: lower index first).  A document
    that fits whole in the remaining room of some rank goes whole to the
    fitting rank with the least causal work so far (ties: lower rank).  A
    document that fits nowhere is cut into consecutive pieces from its start,
    each piece filling the rank with the most room left (ties: lower rank).
    Work is counted with causal_piece_work.  Returns, per rank, its positions
    in ascending order."""
    cu = [int(x) for x in cu_seqlens]
    n = len(cu) - 1
    S = cu[-1]
    C = S // cp
    room = [C] * cp
    load = [0] * cp
    pieces = [[] for _ in range(cp)]
    for i in sorted(range(n), key=lambda i: (-(cu[i + 1] - cu[i]), i)):
        s, e = cu[i], cu[i + 1]
        if e == s:
            continue
        fits = [r for r in range(cp) if room[r] >= e - s]
        if fits:
            r = min(fits, key=lambda r: (load[r], r))
            pieces[r].append((s, e))
            room[r] -= e - s
            load[r] += causal_piece_work(s, s, e)
            continue
        a = s
        while a < e:
            r = max(range(cp), key=lambda r: (room[r], -r))
            m = min(room[r], e - a)
            pieces[r].append((a, a + m))
            room[r] -= m
            load[r] += causal_piece_work(s, a, a + m)
            a += m
    out = []
    for r in range(cp):
        pos = [p for a, b in pieces[r] for p in range(a, b)]
        out.append(np.array(sorted(pos), dtype=np.int64))
    return out


def per_doc_positions(cu_seqlens, cp: int, rank: int) -> np.ndarray:
    """Per-document zigzag (the Per-Doc sharding named in the FlashCP
    abstract): every document is cut into 2*cp equal chunks on its own and rank
    ``rank`` takes chunks ``rank`` and ``2cp-1-rank`` of each, documents kept in
    their packed order.  Every document length must be a multiple of 2*cp (the
    divisibility rule of the hierarchical-CP page's "Required constraints",
    applied per document)."""
    cu = [int(x) for x in cu_seqlens]
    out = []
    for s, e in zip(cu[:-1], cu[1:]):
        n = e - s
        if n % (2 * cp) != 0:
            raise ValueError("every document length must be a multiple of 2*cp")
        if n:
            out.append(s + zigzag_positions(n, cp, rank))
    return np.concatenate(out) if out else np.zeros(0, dtype=np.int64)


def doc_start_of(positions, cu_seqlens) -> np.ndarray:
    """Start of the packed document that holds each global position."""
    positions = np.asarray(positions, dtype=np.int64)
    if cu_seqlens is None:
        return np.zeros_like(positions)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    idx = np.searchsorted(cu, positions, side="right") - 1
    return cu[idx]


def doc_end_of(positions, cu_seqlens, S: int) -> np.ndarray:
    """One past the end of the packed document that holds each position."""
    positions = np.asarray(positions, dtype=np.int64)
    if cu_seqlens is None:
        return np.full_like(positions, S)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    idx = np.searchsorted(cu, positions, side="right") - 1
    return cu[idx + 1]


def allowed_mask(q_pos, q_lo, k_pos) -> np.ndarray:
    """allowed[i, j] = q_lo[i] <= k_pos[j] <= q_pos[i] (causal within a document)."""
    q_pos = np.asarray(q_pos, dtype=np.int64)[:, None]
    q_lo = np.asarray(q_lo, dtype=np.int64)[:, None]
    k_pos = np.asarray(k_pos, dtype=np.int64)[None, :]
    return (k_pos >= q_lo) & (k_pos <= q_pos)


def pair_count(q_pos, q_lo, k_pos) -> int:
    """Exact number of allowed (query, key) pairs: for every query row, the
    number of keys whose position lies in [q_lo, q_pos]."""
    ks = np.sort(np.asarray(k_pos, dtype=np.int64))
    q_pos = np.asarray(q_pos, dtype=np.int64)
    q_lo = np.asarray(q_lo, dtype=np.int64)
    hi = np.searchsorted(ks, q_pos, side="right")
    lo = np.searchsorted(ks, q_lo, side="left")
    return int(np.maximum(hi - lo, 0).sum())


# --------------------------------------------------------------------------
# Forward
# --------------------------------------------------------------------------
def _as64(x):
    return np.asarray(x, dtype=np.float64)


def attention_fwd(q, k, v, scale, cu_seqlens=None, rows=None, causal=True, row_block=512):
    """Full-sequence softmax attention in fp64, for a subset of query rows.

    q: [B, Hq, S, d]; k, v: [B, Hkv, S, d] in natural (unsharded) order.
    Query head h reads key/value head h // (Hq // Hkv).
    rows: global query positions to return (default: all S).
    Returns O [B, Hq, len(rows), d] and LSE [B, Hq, len(rows)] (natural log).

    For row i: allowed keys J(i) = {j : lo(i) <= j <= i} (causal; lo = start of
    i's document, 0 without documents) or {j : lo(i) <= j < hi(i)} (non-causal).
    s_ij = scale * q_i . k_j ; m_i = max s_ij ; Z_i = sum exp(s_ij - m_i) ;
    O_i = sum exp(s_ij - m_i) v_j / Z_i ; LSE_i = m_i + ln Z_i.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, Hq, S, d = q.shape
    Hkv = k.shape[1]
    assert Hq % Hkv == 0
    g = Hq // Hkv
    rows = np.arange(S, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    lo = doc_start_of(rows, cu_seqlens)
    hi = rows + 1 if causal else doc_end_of(rows, cu_seqlens, S)
    n = rows.shape[0]
    O = np.zeros((B, Hq, n, d))
    L = np.zeros((B, Hq, n))
    for b in range(B):
        for h in range(Hq):
            kvh = h // g
            for s0 in range(0, n, row_block):
                r = rows[s0:s0 + row_block]
                rl, rh = lo[s0:s0 + row_block], hi[s0:s0 + row_block]
                kmin, kmax = int(rl.min()), int(rh.max())
                keys = np.arange(kmin, kmax)
                s = scale * (q[b, h, r] @ k[b, kvh, kmin:kmax].T)
                ok = (keys[None, :] >= rl[:, None]) & (keys[None, :] < rh[:, None])
                s = np.where(ok, s, -np.inf)
                m = s.max(axis=1)
                p = np.exp(s - m[:, None])
                Z = p.sum(axis=1)
                O[b, h, s0:s0 + len(r)] = (p @ v[b, kvh, kmin:kmax]) / Z[:, None]
                L[b, h, s0:s0 + len(r)] = m + np.log(Z)
    return O, L


def partial_attention_fwd(q_rows, k_rows, v_rows, scale, q_pos, q_lo, k_pos):
    """One ring step: attention of a set of query rows against one set of key
    rows, with allowed[i, j] = q_lo[i] <= k_pos[j] <= q_pos[i].

    q_rows: [B, Hq, nq, d]; k_rows, v_rows: [B, Hkv, nk, d].
    Returns the partial (O, LSE) normalised over the allowed keys of this step
    only; a row with no allowed key gets O = 0 and LSE = -inf, which is the
    identity of ``lse_merge``.
    """
    q, k, v = _as64(q_rows), _as64(k_rows), _as64(v_rows)
    B, Hq, nq, d = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    ok = allowed_mask(q_pos, q_lo, k_pos)
    has = ok.any(axis=1)
    O = np.zeros((B, Hq, nq, d))
    L = np.full((B, Hq, nq), -np.inf)
    if not has.any():
        return O, L
    for b in range(B):
        for h in range(Hq):
            kvh = h // g
            s = scale * (q[b, h] @ k[b, kvh].T)
            s = np.where(ok, s, -np.inf)
            m = np.where(has, s.max(axis=1), 0.0)
            p = np.exp(s - m[:, None])
            Z = p.sum(axis=1)
            Zs = np.where(has, Z, 1.0)
            O[b, h] = np.where(has[:, None], (p @ v[b, kvh]) / Zs[:, None], 0.0)
            L[b, h] = np.where(has, m + np.log(Zs), -np.inf)
    return O, L


def lse_merge(o1, l1, o2, l2):
    """combine(): merge two partial results over disjoint key sets.

    L = M + ln(exp(l1 - M) + exp(l2 - M)) with M = max(l1, l2);
    O = exp(l1 - L) o1 + exp(l2 - L) o2.  (0, -inf) is the identity and two
    empty partials give (0, -inf).
    """
    o1, l1, o2, l2 = _as64(o1), _as64(l1), _as64(o2), _as64(l2)
    M = np.maximum(l1, l2)
    empty = np.isneginf(M)
    Ms = np.where(empty, 0.0, M)
    e1 = np.exp(l1 - Ms)
    e2 = np.exp(l2 - Ms)
    L = np.where(empty, -np.inf, Ms + np.log(np.where(empty, 1.0, e1 + e2)))
    Ls = np.where(empty, 0.0, L)
    w1 = np.where(empty, 0.0, np.exp(l1 - Ls))
    w2 = np.where(empty, 0.0, np.exp(l2 - Ls))
    O = w1[..., None] * o1 + w2[..., None] * o2
    return O, L


def ring_partials_fwd(q_loc, k_all, v_all, scale, cp, rank, q_pos, q_lo, k_pos_all):
    """A rank's ring schedule done the sharded way: for step t the rank attends
    its local rows to the K/V shard of rank (rank - t) mod cp, then every
    partial is folded in with ``lse_merge`` (guide, "So how does it work?":
    each shard attended once, then combined).

    k_all / v_all hold every rank's shard in rank-major order, as gathering the
    shards yields; k_pos_all are their global positions.
    """
    nk = k_all.shape[2]
    R = nk // cp
    B, Hq, nq, d = q_loc.shape
    O = np.zeros((B, Hq, nq, d))
    L = np.full((B, Hq, nq), -np.inf)
    for t in range(cp):
        src = (rank - t) % cp
        sl = slice(src * R, (src + 1) * R)
        Op, Lp = partial_attention_fwd(q_loc, k_all[:, :, sl], v_all[:, :, sl], scale,
                                       q_pos, q_lo, np.asarray(k_pos_all)[sl])
        O, L = lse_merge(O, L, Op, Lp)
    return O, L


# --------------------------------------------------------------------------
# Backward (recompute P from the saved LSE)
# --------------------------------------------------------------------------
def bwd_delta(dout, o):
    """delta_i = sum_t dO[i, t] * O[i, t] (per row and head)."""
    return (_as64(dout) * _as64(o)).sum(axis=-1)


def attention_bwd(q, k, v, dout, scale, cu_seqlens=None, rows=None, row_block=512):
    """Gradients of sum_{i in rows} dO_i . O_i with respect to q, k, v (causal).

    dout: [B, Hq, len(rows), d], aligned with ``rows`` (default all rows).
    Returns dq [B, Hq, len(rows), d] (rows of ``rows`` only) and dk, dv
    [B, Hkv, S, d] in natural order.

    P_ij = exp(s_ij - LSE_i) on allowed pairs; dV_j = sum_i P_ij dO_i ;
    dP_ij = dO_i . v_j ; dS_ij = P_ij (dP_ij - delta_i) ;
    dQ_i = scale sum_j dS_ij k_j ; dK_j = scale sum_i dS_ij q_i ;
    dK and dV of a key/value head sum over the query heads that read it.
    """
    q, k, v, dout = _as64(q), _as64(k), _as64(v), _as64(dout)
    B, Hq, S, d = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    rows = np.arange(S, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    O, L = attention_fwd(q, k, v, scale, cu_seqlens=cu_seqlens, rows=rows, row_block=row_block)
    delta = bwd_delta(dout, O)
    lo = doc_start_of(rows, cu_seqlens)
    n = rows.shape[0]
    dq = np.zeros((B, Hq, n, d))
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            kvh = h // g
            for s0 in range(0, n, row_block):
                r = rows[s0:s0 + row_block]
                rl = lo[s0:s0 + row_block]
                kmin, kmax = int(rl.min()), int(r.max()) + 1
                keys = np.arange(kmin, kmax)
                ok = (keys[None, :] >= rl[:, None]) & (keys[None, :] <= r[:, None])
                s = scale * (q[b, h, r] @ k[b, kvh, kmin:kmax].T)
                P = np.where(ok, np.exp(np.where(ok, s, 0.0) - L[b, h, s0:s0 + len(r)][:, None]), 0.0)
                do = dout[b, h, s0:s0 + len(r)]
                dv[b, kvh, kmin:kmax] += P.T @ do
                dP = do @ v[b, kvh, kmin:kmax].T
                dS = P * (dP - delta[b, h, s0:s0 + len(r)][:, None])
                dq[b, h, s0:s0 + len(r)] = scale * (dS @ k[b, kvh, kmin:kmax])
                dk[b, kvh, kmin:kmax] += scale * (dS.T @ q[b, h, r])
    return dq, dk, dv


def partial_attention_bwd(q_rows, k_rows, v_rows, dout, lse, delta, scale, q_pos, q_lo, k_pos):
    """One ring step's share of the gradients, given each row's LSE and delta
    (those of the merged output when the steps of a ring are summed, or those
    of this step's own output for the gradient of one step alone).

    P_ij = exp(s_ij - LSE_i) on allowed pairs, 0 elsewhere (a row whose LSE is
    -inf has no allowed key and gets P = 0); dV_j = sum_i P_ij dO_i ;
    dS_ij = P_ij (dO_i . v_j - delta_i) ; dQ_i = scale sum_j dS_ij k_j ;
    dK_j = scale sum_i dS_ij q_i ; dK and dV of a key/value head sum over the
    query heads that read it.

    q_rows, dout: [B, Hq, nq, d]; k_rows, v_rows: [B, Hkv, nk, d]; lse, delta:
    [B, Hq, nq].  Returns dq [B, Hq, nq, d] and dk, dv [B, Hkv, nk, d].
    """
    q, k, v, do = _as64(q_rows), _as64(k_rows), _as64(v_rows), _as64(dout)
    L, dl = _as64(lse), _as64(delta)
    B, Hq, nq, d = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    ok = allowed_mask(q_pos, q_lo, k_pos)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            kvh = h // g
            s = scale * (q[b, h] @ k[b, kvh].T)
            use = ok & np.isfinite(L[b, h])[:, None]
            P = np.where(use, np.exp(np.where(use, s - L[b, h][:, None], 0.0)), 0.0)
            dv[b, kvh] += P.T @ do[b, h]
            dS = P * (do[b, h] @ v[b, kvh].T - dl[b, h][:, None])
            dq[b, h] = scale * (dS @ k[b, kvh])
            dk[b, kvh] += scale * (dS.T @ q[b, h])
    return dq, dk, dv


# --------------------------------------------------------------------------
# All-to-all level of hierarchical context parallelism: the head exchange
# --------------------------------------------------------------------------
# NeMo Megatron-Bridge "Hierarchical Context Parallel Skill": with cp_comm_type
# "a2a+p2p" the first level is a group of g ranks that communicate all-to-all.
# The page gives no layout; the reading here is the head exchange: before it a
# rank holds all heads of its rows, after it all rows of the group for H/g of
# the heads.  These functions move data only; every value is copied exactly.
def a2a_pack(x, g):
    """Send buffer of one rank before the exchange.  x: [rows, H, d], the rank's
    sequence shard, token-major.  Returns [g, H/g, rows, d]: block j holds
    heads j*H/g .. (j+1)*H/g - 1 of every row, head-major, the part rank j
    receives: send[j, hh, t] = x[t, j*H/g + hh]."""
    rows, H, d = x.shape
    Hg = H // g
    send = np.empty((g, Hg, rows, d), dtype=x.dtype)
    for j in range(g):
        for hh in range(Hg):
            send[j, hh] = x[:, j * Hg + hh]
    return send


def a2a_unpack_pack(send):
    """Inverse of a2a_pack: x[t, j*H/g + hh] = send[j, hh, t]."""
    g, Hg, rows, d = send.shape
    x = np.empty((rows, g * Hg, d), dtype=send.dtype)
    for j in range(g):
        for hh in range(Hg):
            x[:, j * Hg + hh] = send[j, hh]
    return x


def a2a_exchange(sends):
    """The all-to-all itself: rank j receives block j of every rank's send
    buffer, in source-rank order (recv_j[i] = send_i[j])."""
    g = len(sends)
    return [np.stack([sends[i][j] for i in range(g)]) for j in range(g)]


def a2a_unpack(recv):
    """Layout after the exchange.  recv: [g, H/g, rows, d], block i from rank i.
    Returns [H/g, g*rows, d]: the rank's heads over all g*rows rows of the
    group, rows in source-rank order: y[hh, i*rows + t] = recv[i, hh, t]."""
    g, Hg, rows, d = recv.shape
    y = np.empty((Hg, g * rows, d), dtype=recv.dtype)
    for i in range(g):
        y[:, i * rows:(i + 1) * rows] = recv[i]
    return y


def a2a_pack_unpack(y, g):
    """Inverse of a2a_unpack: recv[i, hh, t] = y[hh, i*rows + t]."""
    Hg, n, d = y.shape
    rows = n // g
    recv = np.empty((g, Hg, rows, d), dtype=y.dtype)
    for i in range(g):
        recv[i] = y[:, i * rows:(i + 1) * rows]
    return recv


# --------------------------------------------------------------------------
# Sizes
# --------------------------------------------------------------------------
def attention_matrix_bytes(seq_len: int, num_heads: int = 1, bytes_per_elem: int = 2) -> int:
    """Memory of a materialised seq_len x seq_len attention matrix per the
    guide's "Why context parallelism?" estimate (bf16: 2 bytes an entry)."""
    return int(seq_len) * int(seq_len) * int(bytes_per_elem) * int(num_heads)

