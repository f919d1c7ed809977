"""Shared set-up for the GPU parity tests: seeded inputs, the shard
materialisation of one virtual rank, and the oracle's rows for it."""
import math

import numpy as np
import torch

import oracle as orc
import seeded_inputs as si
import context_causal_attention_amd as cpa

# Acceptance bars: bf16 inputs O <= 2e-2 and LSE <= 1e-3 max-abs against the
# fp64 oracle; fp32 inputs 1e-5 for both.
TOL = {"bf16": (2e-2, 1e-3), "f32": (1e-5, 1e-5)}


def announce(msg):
    print(f"[case] {msg}", flush=True)


def oracle_deal(S, cp, rank, cu=None, mode=cpa.CP_STREAM):
    """The oracle's positions and document starts of `rank`'s rows: the zigzag
    deal of the sequence (or packed stream), the per-document zigzag, or the
    whole-document placement."""
    if cu is None:
        return orc.zigzag_positions(S, cp, rank), None
    if mode == cpa.CP_STREAM:
        pos = orc.zigzag_positions(S, cp, rank)
    elif mode == cpa.CP_PER_DOC:
        pos = orc.per_doc_positions(cu, cp, rank)
    elif mode == cpa.CP_WHOLE_DOC:
        pos = orc.whole_doc_deal(cu, cp)[rank]
    else:
        raise ValueError(f"unknown deal {mode}")
    return pos, orc.doc_start_of(pos, cu)


class Rank:
    """Inputs of one virtual rank, on the GPU, plus fp64 copies for the oracle."""

    def __init__(self, B, Hq, Hkv, S, d, cp, rank, dtype, seed=0, cu=None, mode=cpa.CP_STREAM,
                 with_dout=False, full=None):
        self.B, self.Hq, self.Hkv, self.S, self.d, self.cp, self.rank = B, Hq, Hkv, S, d, cp, rank
        self.dtype, self.cu = dtype, cu
        if full is None:
            full = si.make_qkv(B, Hq, Hkv, S, d, dtype, seed=seed, with_dout=with_dout)
        self.full = full
        q, k, v = full[:3]
        # Every index map comes from the oracle's own deal; the library's map
        # must equal it bit for bit before anything runs on the GPU.
        self.pos, self.lo = oracle_deal(S, cp, rank, cu, mode)
        self.allp = np.concatenate([oracle_deal(S, cp, r, cu, mode)[0] for r in range(cp)])
        if cu is None:
            lib_pos, lib_lo = cpa.cp_shard_zigzag(S, cp, rank), None
            assert np.array_equal(cpa.cp_unshard_zigzag(S, cp), self.allp)
        else:
            lib_pos, lib_lo = cpa.cp_varlen_index(cu, cp, rank, mode)
            assert np.array_equal(lib_lo, self.lo)
        assert np.array_equal(lib_pos, self.pos), "library index map differs from the oracle's deal"
        pi = torch.from_numpy(self.pos.astype(np.int64))
        ai = torch.from_numpy(self.allp.astype(np.int64))
        self.q_loc = q.index_select(2, pi).cuda()
        self.do_loc = full[3].index_select(2, pi).cuda() if len(full) > 3 else None
        self.k_all = k.index_select(2, ai).cuda()
        self.v_all = v.index_select(2, ai).cuda()
        self.scale = 1.0 / math.sqrt(d)

    def ring_fwd(self, out_dtype=None):
        return cpa.cp_attn_ring_fwd(self.q_loc, self.k_all, self.v_all, self.cp, self.rank, self.pos, self.lo,
                                    self.allp, scale=self.scale, out_dtype=out_dtype)

    def ring_bwd(self):
        """Forward, delta and ring backward of this rank's rows: (o, lse, dq, dk_all, dv_all)."""
        o, lse = self.ring_fwd()
        delta = cpa.cp_attn_bwd_delta(self.do_loc, o)
        dq, dk, dv = cpa.cp_attn_ring_bwd(self.q_loc, self.k_all, self.v_all, self.do_loc, lse, delta, self.cp,
                                          self.rank, self.pos, self.lo, self.allp, scale=self.scale)
        return o, lse, dq, dk, dv

    def oracle_grads(self, q_heads=None):
        """Oracle gradients of this rank's loss sum_i dO_i . O_i over its rows:
        dq for its rows, dk and dv in rank-major (k_all) order.  q_heads
        restricts the check to whole groups of query heads (a slice that starts
        and ends on a group boundary)."""
        q, k, v, do = (t.double().numpy() for t in self.full[:4])
        if q_heads is not None:
            g = self.Hq // self.Hkv
            assert q_heads.start % g == 0 and q_heads.stop % g == 0
            kv = slice(q_heads.start // g, q_heads.stop // g)
            q, do, k, v = q[:, q_heads], do[:, q_heads], k[:, kv], v[:, kv]
        dq, dk, dv = orc.attention_bwd(q, k, v, do[:, :, self.pos], self.scale, cu_seqlens=self.cu, rows=self.pos)
        return dq, dk[:, :, self.allp], dv[:, :, self.allp]

    def oracle(self, rows_idx=None):
        """Oracle O, LSE for this rank's rows (or the subset rows_idx of them)."""
        q, k, v = (t.double().numpy() for t in self.full[:3])
        rows = self.pos if rows_idx is None else self.pos[rows_idx]
        return orc.attention_fwd(q, k, v, self.scale, cu_seqlens=self.cu, rows=rows)


def max_err(gpu, ref):
    g = gpu.detach().double().cpu().numpy()
    both_inf = np.isneginf(g) & np.isneginf(ref)
    g = np.where(both_inf, 0.0, g)
    r = np.where(both_inf, 0.0, ref)
    return float(np.abs(g - r).max()) if g.size else 0.0


def assert_close(o, lse, O_ref, L_ref, dtype, what=""):
    to, tl = TOL[dtype]
    eo, el = max_err(o, O_ref), max_err(lse, L_ref)
    assert np.isfinite(eo) and eo <= to, f"{what}: O max-abs error {eo:.3e} > {to}"
    assert np.isfinite(el) and el <= tl, f"{what}: LSE max-abs error {el:.3e} > {tl}"
    return eo, el


def pair_error_bounds(q64, k64, v64, do_r, rows, scale, L_ref, dl_ref, dL, ddl, g, u=2.0 ** -8):
    """Per-element error bounds of dV, dK (every key, natural order) and of the
    rows' dQ, for gradients whose dO is zero outside ``rows``.

    The arithmetic of one pair (i, j): P and dS reach the MFMAs as bf16
    (relative error <= u, the unit roundoff of bf16's 8-bit significand; dS
    may be formed from the rounded P), P carries the kernel's LSE error dL,
    dS the error ddl of the kernel's delta, and dP, delta the fp32 error of
    their sums.  The pair errors, weighted by |dO|, |q| or |k|, are doubled.
    q64, k64, v64: [1, H, S, d] fp64; do_r: [1, Hq, len(rows), d]; L_ref,
    dl_ref, dL, ddl: [1, Hq, len(rows)]; g: query heads per kv head."""
    S = k64.shape[2]
    Hq = q64.shape[1]
    tol_dv = np.zeros((1, k64.shape[1], S, k64.shape[3]))
    tol_dk = np.zeros_like(tol_dv)
    tol_dq = np.zeros((1, Hq, len(rows), q64.shape[3]))
    allowed = np.arange(S)[None, :] <= np.asarray(rows)[:, None]
    for h in range(Hq):
        kvh = h // g
        s = scale * (q64[0, h, rows] @ k64[0, kvh].T)
        P = np.where(allowed, np.exp(np.where(allowed, s, 0.0) - L_ref[0, h][:, None]), 0.0)
        dP = do_r[0, h] @ v64[0, kvh].T
        dsd = np.abs(dP - dl_ref[0, h][:, None])
        eps = u + 2.0 * dL[0, h][:, None] + 1e-5  # P as the MFMAs see it
        pair = P * ((eps + u) * dsd + ddl[0, h][:, None] + 1e-5 * (np.abs(dP) + np.abs(dl_ref[0, h])[:, None]))
        tol_dv[0, kvh] += 2.0 * ((eps * P).T @ np.abs(do_r[0, h]))
        tol_dk[0, kvh] += 2.0 * scale * (pair.T @ np.abs(q64[0, h, rows]))
        tol_dq[0, h] = 2.0 * scale * (pair @ np.abs(k64[0, kvh]))
    return tol_dv + 1e-6, tol_dk + 1e-6, tol_dq + 1e-6
