"""Seeded synthetic inputs for causal context-parallel attention.

Shared by the tests, ``bench.py`` and ``__graft_entry__.smoke()``: the HIP path
and the fp64 oracle both read the tensors made here, and nothing else is
shared between them.  This module holds no attention arithmetic: only random
draws, dtype casts and the workload shapes.

Recipe (one generator for every workload):
* q, k, v (and dO for the backward) are drawn as fp32 ``torch.randn`` from a CPU
  ``torch.Generator`` seeded with ``seed``, in the order q, k, v, dO, then cast to
  the workload dtype (bf16 casts round to nearest even).  fp64 copies of the cast
  values are exact, which is what the oracle sees.  Large-range cases scale the
  fp32 q draw by a constant before the cast.
* Packed-document lengths are lognormal with distribution mean 2048 and log-sd
  1.0 (so the underlying normal has mean ln 2048 - 1/2), rounded to integers,
  clipped to [128, 16384] and drawn in order until the total is reached; the
  last document is cut to the remainder.  ``numpy.random.default_rng(seed)``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "make_qkv", "doc_lengths", "round_doc_lengths", "cu_seqlens_from_lengths",
           "workload_cu_seqlens"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    S: int
    cp: int
    dtype: str          # "f32" or "bf16"
    varlen: bool = False
    backward: bool = False
    doc_multiple: int = 0  # varlen: document lengths rounded down to a multiple of this (0: as drawn)
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def chunk(self) -> int:
        return self.S // (2 * self.cp)

    @property
    def local_rows(self) -> int:
        return self.S // self.cp


WORKLOADS = {
    "c0_f32_s1024_cp2": Workload("c0_f32_s1024_cp2", 1, 1, 1, 64, 1024, 2, "f32",
                                 note="1 head, d=64, S=1024, cp=2, fp32, scale 1/8"),
    "llama8b_s32k_cp8": Workload("llama8b_s32k_cp8", 1, 32, 8, 128, 32768, 8, "bf16",
                                 note="32q/8kv heads, d=128, S=32768, cp=8, bf16"),
    "llama8b_s128k_cp8": Workload("llama8b_s128k_cp8", 1, 32, 8, 128, 131072, 8, "bf16",
                                  note="32q/8kv heads, d=128, S=131072, cp=8, bf16"),
    "varlen_s64k_cp4": Workload("varlen_s64k_cp4", 1, 32, 8, 128, 65536, 4, "bf16", varlen=True,
                                note="packed lognormal documents, 65536 tokens, cp=4"),
    "varlen8_s64k_cp4": Workload("varlen8_s64k_cp4", 1, 32, 8, 128, 65536, 4, "bf16", varlen=True, doc_multiple=8,
                                 note="the 65536-token documents with lengths rounded down to multiples of 2cp = 8, "
                                      "so both the stream and the per-document deal apply"),
    "bwd_s32k_cp8": Workload("bwd_s32k_cp8", 1, 32, 8, 128, 32768, 8, "bf16", backward=True,
                             note="backward on the 32768-token shapes, dO ~ N(0,1) bf16"),
}


def _torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make_qkv(B: int, Hq: int, Hkv: int, S: int, d: int, dtype: str = "bf16", seed: int = 0,
             with_dout: bool = False, q_scale: float = 1.0):
    """CPU tensors q [B,Hq,S,d], k, v [B,Hkv,S,d] (and dO [B,Hq,S,d]) drawn as
    fp32 N(0,1) in the order q, k, v, dO from one seeded generator, then cast.
    q_scale multiplies the fp32 q draw before the cast (q ~ N(0, q_scale^2)):
    scores then span q_scale times their usual range."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    q = torch.randn(B, Hq, S, d, generator=g, dtype=torch.float32)
    if q_scale != 1.0:
        q = q * q_scale
    k = torch.randn(B, Hkv, S, d, generator=g, dtype=torch.float32)
    v = torch.randn(B, Hkv, S, d, generator=g, dtype=torch.float32)
    out = [q, k, v]
    if with_dout:
        out.append(torch.randn(B, Hq, S, d, generator=g, dtype=torch.float32))
    dt = _torch_dtype(dtype)
    return tuple(t.to(dt) for t in out)


def doc_lengths(total: int = 65536, mean: float = 2048.0, sigma: float = 1.0,
                lo: int = 128, hi: int = 16384, seed: int = 0) -> np.ndarray:
    """Lengths of packed documents summing exactly to ``total``."""
    rng = np.random.default_rng(seed)
    mu = math.log(mean) - 0.5 * sigma * sigma
    out = []
    acc = 0
    while acc < total:
        n = int(np.clip(np.rint(rng.lognormal(mu, sigma)), lo, hi))
        n = min(n, total - acc)
        out.append(n)
        acc += n
    return np.asarray(out, dtype=np.int64)


def round_doc_lengths(lengths, multiple: int) -> np.ndarray:
    """Each length rounded down to a multiple of ``multiple``; the tokens cut
    off form one last document (a multiple too when the total is), and empty
    documents are dropped."""
    lengths = np.asarray(lengths, dtype=np.int64)
    total = int(lengths.sum())
    out = (lengths // multiple) * multiple
    out = np.append(out, total - out.sum())
    return out[out > 0]


def workload_cu_seqlens(w: "Workload"):
    """Document boundaries of a varlen workload (None for dense ones)."""
    if not w.varlen:
        return None
    L = doc_lengths(total=w.S, seed=w.seed)
    if w.doc_multiple:
        L = round_doc_lengths(L, w.doc_multiple)
    return cu_seqlens_from_lengths(L)


def cu_seqlens_from_lengths(lengths) -> np.ndarray:
    """Document boundaries [0, l0, l0+l1, ..., total] as int32."""
    lengths = np.asarray(lengths, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
