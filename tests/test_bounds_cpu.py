"""CPU check of the per-element error bound that the GPU parity test of the
backward at full size uses (gpu_cases.pair_error_bounds): against an emulation
of the kernels' arithmetic, the bound holds; against the same emulation with a
planted mistake, it fails.

The emulation follows the kernels' precision, not their code: scores and sums
in fp32, P rounded to bf16 for the P V and dV products, dS rounded to bf16 for
the dK and dQ products, the forward's output from bf16 P and an fp32 row sum,
delta = rowsum(dO . O) in fp32.  dO is zero except on sampled rows, as in the
GPU test, so only those rows contribute."""
import math

import numpy as np
import torch

import oracle as orc
import seeded_inputs as si
from gpu_cases import pair_error_bounds


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def _emulate(q, k, v, do_r, rows, scale, g, drop_keys=None):
    """fp32/bf16 emulation of the forward's LSE and O, delta, and the
    backward's dq (rows), dk, dv (every key) for dO given on ``rows`` only.
    drop_keys: keys whose dK/dV contributions are left out (a planted
    mistake)."""
    Hq, S, d = q.shape[1], k.shape[2], q.shape[3]
    f = np.float32
    allowed = np.arange(S)[None, :] <= rows[:, None]
    L = np.zeros((1, Hq, len(rows)))
    dl = np.zeros_like(L)
    dq = np.zeros((1, Hq, len(rows), d))
    dk = np.zeros((1, k.shape[1], S, d), dtype=f)
    dv = np.zeros_like(dk)
    for h in range(Hq):
        kvh = h // g
        s = (q[0, h, rows].astype(f) @ k[0, kvh].astype(f).T) * f(scale)
        s = np.where(allowed, s, -np.inf).astype(f)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m).astype(f)
        lsum = p.sum(axis=1, dtype=f)
        L[0, h] = (m[:, 0] + np.log(lsum)).astype(f)
        o = (_bf16(p) @ v[0, kvh].astype(f)) / lsum[:, None]
        dl[0, h] = (do_r[0, h].astype(f) * o).sum(axis=1, dtype=f)
        P = np.exp(s - L[0, h][:, None].astype(f)).astype(f)
        dP = do_r[0, h].astype(f) @ v[0, kvh].astype(f).T
        dS = _bf16(P * (dP - dl[0, h][:, None].astype(f)))
        P16 = _bf16(P)
        keep = np.ones(S, dtype=bool)
        if drop_keys is not None:
            keep[drop_keys] = False
        dv[0, kvh] += np.where(keep[:, None], P16.T @ do_r[0, h].astype(f), 0)
        dk[0, kvh] += np.where(keep[:, None], f(scale) * (dS.T @ q[0, h, rows].astype(f)), 0)
        dq[0, h] = f(scale) * (dS @ k[0, kvh].astype(f))
    return L, dl, dq, dk, dv


def _case():
    B, Hq, Hkv, S, d, cp, rank = 1, 4, 1, 512, 64, 2, 0
    q, k, v, do = (t.double().numpy() for t in si.make_qkv(B, Hq, Hkv, S, d, "bf16", seed=21, with_dout=True))
    pos = orc.zigzag_positions(S, cp, rank)
    n = len(pos)
    idx = np.unique(np.concatenate([[0, 1, n // 2 - 1, n // 2, n - 1], np.random.default_rng(3).integers(0, n, 4)]))
    rows = pos[idx]
    return q, k, v, do[:, :, rows], rows, 1.0 / math.sqrt(d), Hq // Hkv


def _errors_and_bounds(drop_keys=None):
    q, k, v, do_r, rows, scale, g = _case()
    dq_ref, dk_ref, dv_ref = orc.attention_bwd(q, k, v, do_r, scale, rows=rows)
    O_ref, L_ref = orc.attention_fwd(q, k, v, scale, rows=rows)
    dl_ref = orc.bwd_delta(do_r, O_ref)
    L, dl, dq, dk, dv = _emulate(q, k, v, do_r, rows, scale, g, drop_keys)
    dL, ddl = np.abs(L - L_ref), np.abs(dl - dl_ref)
    tol_dv, tol_dk, tol_dq = pair_error_bounds(q, k, v, do_r, rows, scale, L_ref, dl_ref, dL, ddl, g)
    return [(name, np.abs(got - ref), tol, ref) for name, got, ref, tol in
            (("dv", dv, dv_ref, tol_dv), ("dk", dk, dk_ref, tol_dk), ("dq", dq, dq_ref, tol_dq))]


def test_bound_holds_for_the_kernels_arithmetic():
    for name, err, tol, ref in _errors_and_bounds():
        assert np.all(err <= tol), f"{name}: emulated error {err.max():.3e} above its bound"
        # Not vacuous: the emulated errors reach a sizeable part of the bound
        # somewhere (0.2-0.5 of it on this case).
        assert (err / tol).max() > 0.05, f"{name}: bound {1 / (err / tol).max():.0f}x the worst error"
        assert np.isfinite(ref).all()


def test_bound_catches_a_dropped_key_tile():
    # Keys 64..127 (one 64-key tile) are attended by every sampled row past
    # position 127; leaving their dK/dV out must break the bound.
    out = dict((name, (err, tol)) for name, err, tol, _ in _errors_and_bounds(drop_keys=np.arange(64, 128)))
    for name in ("dv", "dk"):
        err, tol = out[name]
        assert np.any(err > tol), f"{name}: a dropped key tile went unnoticed"
