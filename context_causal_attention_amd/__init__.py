"""Python binding of libcpattn.so, the MI355X-native hot path of causal
context-parallel (zigzag ring) attention.

Every function here only marshals arguments (tensor pointers, strides, the
current HIP stream) into the C ABI declared in ``include/cpattn.h`` and turns
error codes into exceptions; all work runs in the library's host index builder
and HIP kernels.  There is no fallback: if the library is not built the calls
raise.  PyTorch provides device memory and streams only.

Names match the C entry points.  Error codes map to exceptions the way the
Accelerate plugin reports bad configuration: invalid arguments and shapes raise
``ValueError``; HIP runtime failures raise ``RuntimeError``.
"""
from __future__ import annotations

import ctypes
import math
import os
from ctypes import c_float, c_int32, c_int64, c_size_t, c_void_p, POINTER

import numpy as np
import torch

__all__ = [
    "CP_OK", "CP_EINVAL", "CP_ESHAPE", "CP_EDTYPE", "CP_EWORKSPACE", "CP_EHIP",
    "CP_F32", "CP_BF16", "CP_STREAM", "CP_PER_DOC", "CP_WHOLE_DOC", "CpShape", "CpError", "LIB_PATH",
    "lib", "cp_version", "cp_last_error", "cp_shard_zigzag", "cp_unshard_zigzag",
    "cp_varlen_index", "cp_ring_source", "cp_pairs", "cp_attn_ring_fwd_workspace", "cp_attn_ring_fwd_noalloc",
    "cp_attn_partial_fwd", "cp_attn_merge", "cp_attn_ring_fwd", "RingFwdPlan", "cp_attn_ring_fwd_stepwise",
    "RingFwdStepwisePlan", "cp_a2a_pack", "cp_a2a_pack_inverse", "cp_a2a_unpack", "cp_a2a_unpack_inverse",
    "cp_attn_bwd_workspace", "cp_attn_bwd_delta", "cp_attn_partial_bwd", "cp_attn_ring_bwd", "RingBwdPlan",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcpattn.so")

CP_OK, CP_EINVAL, CP_ESHAPE, CP_EDTYPE, CP_EWORKSPACE, CP_EHIP = range(6)
CP_F32, CP_BF16 = 0, 1
CP_STREAM, CP_PER_DOC, CP_WHOLE_DOC = 0, 1, 2

_DT = {torch.float32: CP_F32, torch.bfloat16: CP_BF16}
_I32P = POINTER(c_int32)


class CpShape(ctypes.Structure):
    _fields_ = [
        ("b", c_int32), ("hq", c_int32), ("hkv", c_int32), ("d", c_int32),
        ("sq", c_int64), ("sk", c_int64), ("scale", c_float),
        ("in_dtype", c_int32), ("out_dtype", c_int32),
        ("q_str", c_int64 * 3), ("k_str", c_int64 * 3), ("v_str", c_int64 * 3), ("o_str", c_int64 * 3),
    ]


class CpError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"cpattn error {code}: {msg}")
        self.code = code


_lib_handle = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        L.cp_last_error.restype = ctypes.c_char_p
        L.cp_version.restype = c_int32
        L.cp_shard_zigzag.argtypes = [c_int64, c_int32, c_int32, _I32P]
        L.cp_unshard_zigzag.argtypes = [c_int64, c_int32, _I32P]
        L.cp_varlen_index.argtypes = [_I32P, c_int32, c_int32, c_int32, c_int32, _I32P, _I32P]
        L.cp_ring_source.argtypes = [c_int32, c_int32, c_int32]
        L.cp_pairs.argtypes = [_I32P, _I32P, c_int64, _I32P, c_int64]
        L.cp_pairs.restype = c_int64
        L.cp_attn_ring_fwd_workspace.argtypes = [POINTER(CpShape), c_int32]
        L.cp_attn_ring_fwd_workspace.restype = c_size_t
        L.cp_attn_partial_fwd.argtypes = [POINTER(CpShape)] + [c_void_p] * 6 + [c_void_p, c_void_p, c_void_p,
                                                                                c_size_t, c_void_p]
        L.cp_attn_merge.argtypes = [c_int64, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
        L.cp_attn_ring_fwd.argtypes = [POINTER(CpShape), c_int32, c_int32] + [c_void_p] * 6 + \
            [c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
        L.cp_attn_ring_fwd_noalloc.argtypes = [POINTER(CpShape), c_int32, c_int32] + [c_void_p] * 6 + \
            [c_void_p, c_void_p, c_void_p]
        L.cp_attn_ring_fwd_stepwise_workspace.argtypes = [POINTER(CpShape), c_int32]
        L.cp_attn_ring_fwd_stepwise_workspace.restype = c_size_t
        L.cp_attn_ring_stage_bytes.argtypes = [POINTER(CpShape), c_int32]
        L.cp_attn_ring_stage_bytes.restype = c_size_t
        L.cp_attn_ring_fwd_stepwise.argtypes = [POINTER(CpShape), c_int32, c_int32] + [c_void_p] * 6 + \
            [c_void_p, c_void_p, c_void_p, c_size_t, c_void_p, c_size_t, c_void_p, c_void_p]
        L.cp_a2a_pack.argtypes = [c_int32, c_int32, c_int64, c_int32, c_int32, c_void_p, c_int64, c_void_p,
                                  c_int32, c_void_p]
        L.cp_a2a_unpack.argtypes = [c_int32, c_int32, c_int64, c_int32, c_int32, c_void_p, c_void_p, c_int32,
                                    c_void_p]
        L.cp_attn_bwd_workspace.argtypes = [POINTER(CpShape), c_int32]
        L.cp_attn_bwd_workspace.restype = c_size_t
        L.cp_attn_bwd_delta.argtypes = [POINTER(CpShape), c_void_p, c_void_p, c_void_p, c_void_p]
        L.cp_attn_partial_bwd.argtypes = [POINTER(CpShape)] + [c_void_p] * 12 + [c_void_p, c_size_t, c_void_p]
        L.cp_attn_ring_bwd.argtypes = [POINTER(CpShape), c_int32, c_int32] + [c_void_p] * 12 + \
            [c_void_p, c_size_t, c_void_p]
        for name in ("cp_shard_zigzag", "cp_unshard_zigzag", "cp_varlen_index", "cp_ring_source",
                     "cp_attn_partial_fwd", "cp_attn_merge", "cp_attn_ring_fwd", "cp_attn_ring_fwd_stepwise",
                     "cp_attn_bwd_delta", "cp_a2a_pack", "cp_a2a_unpack",
                     "cp_attn_partial_bwd", "cp_attn_ring_bwd"):
            getattr(L, name).restype = c_int32
        _lib_handle = L
    return _lib_handle


def cp_version() -> int:
    return int(lib().cp_version())


def cp_last_error() -> str:
    return lib().cp_last_error().decode()


def _check(rc: int):
    if rc == CP_OK:
        return
    msg = cp_last_error()
    if rc == CP_EHIP:
        raise CpError(rc, msg)
    raise ValueError(f"cpattn error {rc}: {msg}")


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_I32P)


# ------------------------------------------------------------------ host index builder
def cp_shard_zigzag(S: int, cp: int, rank: int) -> np.ndarray:
    """Global positions of ``rank``'s rows: chunk rank, then chunk 2cp-1-rank."""
    n = S // cp if cp >= 1 and S >= 0 else 0
    out = np.empty(max(n, 1), dtype=np.int32)
    _check(lib().cp_shard_zigzag(S, cp, rank, _ptr(out)))
    return out[:n]


def cp_unshard_zigzag(S: int, cp: int) -> np.ndarray:
    """Rank-major concatenation of every rank's positions (a permutation of [0, S))."""
    out = np.empty(max(S, 1), dtype=np.int32)
    _check(lib().cp_unshard_zigzag(S, cp, _ptr(out)))
    return out[:S]


def cp_varlen_index(cu_seqlens, cp: int, rank: int, mode: int = CP_STREAM):
    """(pos, lo) of ``rank``'s rows for packed documents with boundaries ``cu_seqlens``."""
    cu = _i32(cu_seqlens)
    n_docs = len(cu) - 1
    S = int(cu[-1]) if len(cu) else 0
    n = S // cp if cp >= 1 and S >= 0 else 0
    pos = np.empty(max(n, 1), dtype=np.int32)
    lo = np.empty(max(n, 1), dtype=np.int32)
    _check(lib().cp_varlen_index(_ptr(cu), n_docs, cp, rank, mode, _ptr(pos), _ptr(lo)))
    return pos[:n], lo[:n]


def cp_ring_source(cp: int, rank: int, step: int) -> int:
    """Rank whose shard ``rank`` attends at ring step ``step``."""
    r = int(lib().cp_ring_source(cp, rank, step))
    if r < 0:
        raise ValueError(cp_last_error())
    return r


def cp_pairs(q_pos, q_lo, k_pos) -> int:
    """Exact count of allowed (query, key) pairs; ``q_lo`` may be None."""
    qp, kp = _i32(q_pos), _i32(k_pos)
    ql = None if q_lo is None else _i32(q_lo)
    n = lib().cp_pairs(_ptr(qp), None if ql is None else _ptr(ql), len(qp), _ptr(kp), len(kp))
    if n < 0:
        raise ValueError(cp_last_error())
    return int(n)


# ------------------------------------------------------------------ device calls
def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _strides(t: torch.Tensor):
    if t.dim() != 4 or t.stride(-1) != 1:
        raise ValueError("tensors must be [B, H, rows, D] with a contiguous last dimension")
    return (ctypes.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))


def _shape(q, k, v, o_strides, scale, out_dtype) -> CpShape:
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError(f"q, k, v must share a dtype among float32/bfloat16 (got {q.dtype}, {k.dtype}, {v.dtype})")
    B, Hq, Sq, D = q.shape
    if k.shape[0] != B or v.shape != k.shape or k.shape[3] != D:
        raise ValueError(f"inconsistent shapes q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    s = CpShape()
    s.b, s.hq, s.hkv, s.d = B, Hq, k.shape[1], D
    s.sq, s.sk = Sq, k.shape[2]
    s.scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    s.in_dtype = _DT[q.dtype]
    s.out_dtype = _DT[out_dtype]
    s.q_str, s.k_str, s.v_str = _strides(q), _strides(k), _strides(v)
    s.o_str = o_strides
    return s


def _dev_i32(a, device) -> torch.Tensor:
    if isinstance(a, torch.Tensor):
        if a.dtype != torch.int32 or a.device != device or not a.is_contiguous():
            a = a.to(device=device, dtype=torch.int32).contiguous()
        return a
    return torch.from_numpy(_i32(a)).to(device)


def cp_attn_ring_fwd_workspace(q, k, v, cp: int = 1) -> int:
    s = _shape(q, k, v, (ctypes.c_int64 * 3)(0, 0, 0), None, torch.float32)
    n = int(lib().cp_attn_ring_fwd_workspace(ctypes.byref(s), cp))
    if n == 0:
        raise ValueError(cp_last_error() or "invalid shape")
    return n


def _workspace(nbytes, device, ws):
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.numel() < nbytes or ws.data_ptr() % 256:
        raise ValueError("workspace too small or not 256-byte aligned")
    return ws


def cp_attn_partial_fwd(q, k, v, q_pos, q_lo, k_pos, scale=None, out=None, lse=None, workspace=None):
    """One ring step: partial (O fp32, LSE fp32) of q against the allowed keys of k/v."""
    dev = q.device
    B, Hq, Sq, D = q.shape
    out = torch.empty(B, Hq, Sq, D, dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty(B, Hq, Sq, dtype=torch.float32, device=dev) if lse is None else lse
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, Hq, Sq):
        raise ValueError("lse must be contiguous float32 [B, Hq, Sq]")
    s = _shape(q, k, v, _strides(out), scale, torch.float32)
    qp, kp = _dev_i32(q_pos, dev), _dev_i32(k_pos, dev)
    ql = None if q_lo is None else _dev_i32(q_lo, dev)
    ws = _workspace(int(lib().cp_attn_ring_fwd_workspace(ctypes.byref(s), 1)) or 256, dev, workspace)
    _check(lib().cp_attn_partial_fwd(ctypes.byref(s), q.data_ptr(), k.data_ptr(), v.data_ptr(), qp.data_ptr(),
                                     None if ql is None else ql.data_ptr(), kp.data_ptr(), out.data_ptr(),
                                     lse.data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev)))
    return out, lse


def cp_attn_merge(o_acc, lse_acc, o_p, lse_p):
    """In place: (o_acc, lse_acc) <- (o_acc, lse_acc) (+) (o_p, lse_p)."""
    for t in (o_acc, lse_acc, o_p, lse_p):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("merge operands must be contiguous float32")
    d = o_acc.shape[-1]
    rows = o_acc.numel() // d
    if o_p.numel() != o_acc.numel() or lse_acc.numel() != rows or lse_p.numel() != rows:
        raise ValueError("merge operands disagree in size")
    _check(lib().cp_attn_merge(rows, d, o_acc.data_ptr(), lse_acc.data_ptr(), o_p.data_ptr(), lse_p.data_ptr(),
                               _stream(o_acc.device)))
    return o_acc, lse_acc


class RingFwdPlan:
    """A validated cp_attn_ring_fwd call with its workspace, replayable with no
    Python-side allocation (used by the bench to time the call alone)."""

    def __init__(self, q_loc, k_all, v_all, cp, rank, q_pos, q_lo, k_pos_all, scale=None, out_dtype=None,
                 out=None, lse=None, workspace=None):
        dev = q_loc.device
        B, Hq, Sq, D = q_loc.shape
        out_dtype = torch.float32 if out_dtype is None else out_dtype
        self.out = torch.empty(B, Hq, Sq, D, dtype=out_dtype, device=dev) if out is None else out
        self.lse = torch.empty(B, Hq, Sq, dtype=torch.float32, device=dev) if lse is None else lse
        if self.out.dtype != out_dtype:
            raise ValueError("out dtype disagrees with out_dtype")
        self.shape = _shape(q_loc, k_all, v_all, _strides(self.out), scale, out_dtype)
        self.qp = _dev_i32(q_pos, dev)
        self.ql = None if q_lo is None else _dev_i32(q_lo, dev)
        self.kp = _dev_i32(k_pos_all, dev)
        nws = int(lib().cp_attn_ring_fwd_workspace(ctypes.byref(self.shape), cp))
        self.ws = _workspace(nws or 256, dev, workspace)
        self.keep = (q_loc, k_all, v_all)
        self.args = (ctypes.byref(self.shape), cp, rank, q_loc.data_ptr(), k_all.data_ptr(), v_all.data_ptr(),
                     self.qp.data_ptr(), None if self.ql is None else self.ql.data_ptr(), self.kp.data_ptr(),
                     self.out.data_ptr(), self.lse.data_ptr(), self.ws.data_ptr(), self.ws.numel())
        self.device = dev

    def run(self, stream=None):
        st = _stream(self.device) if stream is None else stream
        _check(lib().cp_attn_ring_fwd(*self.args, st))
        return self.out, self.lse


def cp_attn_ring_fwd(q_loc, k_all, v_all, cp, rank, q_pos, q_lo, k_pos_all, scale=None, out_dtype=None,
                     out=None, lse=None, workspace=None):
    """A virtual rank's whole ring with every K/V shard resident: final (O, LSE)."""
    return RingFwdPlan(q_loc, k_all, v_all, cp, rank, q_pos, q_lo, k_pos_all, scale, out_dtype, out, lse,
                       workspace).run()


def cp_attn_ring_fwd_noalloc(q_loc, k_all, v_all, cp, rank, q_pos, q_lo, k_pos_all, out, lse, scale=None,
                             q_pos_dev=None, q_lo_dev=None, k_pos_dev=None):
    """cp_attn_ring_fwd without a workspace (the library's static per-device
    scratch holds the tile tables).  out and lse are caller-provided; positions
    may be given already on the device (q_pos_dev, ...) so that the call itself
    allocates nothing."""
    dev = q_loc.device
    shape = _shape(q_loc, k_all, v_all, _strides(out), scale, out.dtype)
    qp = q_pos_dev if q_pos_dev is not None else _dev_i32(q_pos, dev)
    ql = q_lo_dev if q_lo_dev is not None else (None if q_lo is None else _dev_i32(q_lo, dev))
    kp = k_pos_dev if k_pos_dev is not None else _dev_i32(k_pos_all, dev)
    _check(lib().cp_attn_ring_fwd_noalloc(ctypes.byref(shape), cp, rank, q_loc.data_ptr(), k_all.data_ptr(),
                                          v_all.data_ptr(), qp.data_ptr(), None if ql is None else ql.data_ptr(),
                                          kp.data_ptr(), out.data_ptr(), lse.data_ptr(), _stream(dev)))
    return out, lse


class RingFwdStepwisePlan:
    """A validated cp_attn_ring_fwd_stepwise call: one partial forward per ring
    step, each later step merging into (O, LSE) in its epilogue.  staged=True copies each step's K/V shard into a
    two-slot staging buffer on copy_stream (a torch.cuda.Stream, or None for a
    new one) first, overlapped with the previous step, as a rotation ring
    receives the shards; staged=False reads every shard in place.  O is fp32."""

    def __init__(self, q_loc, k_all, v_all, cp, rank, q_pos, q_lo, k_pos_all, scale=None, staged=True,
                 copy_stream=None, out=None, lse=None, workspace=None, stage=None):
        dev = q_loc.device
        B, Hq, Sq, D = q_loc.shape
        self.out = torch.empty(B, Hq, Sq, D, dtype=torch.float32, device=dev) if out is None else out
        self.lse = torch.empty(B, Hq, Sq, dtype=torch.float32, device=dev) if lse is None else lse
        self.shape = _shape(q_loc, k_all, v_all, _strides(self.out), scale, torch.float32)
        self.qp = _dev_i32(q_pos, dev)
        self.ql = None if q_lo is None else _dev_i32(q_lo, dev)
        self.kp = _dev_i32(k_pos_all, dev)
        nws = int(lib().cp_attn_ring_fwd_stepwise_workspace(ctypes.byref(self.shape), cp))
        self.ws = _workspace(nws or 256, dev, workspace)
        self.stage = None
        self.copy_stream = None
        if staged:
            nst = int(lib().cp_attn_ring_stage_bytes(ctypes.byref(self.shape), cp))
            self.stage = _workspace(nst or 256, dev, stage)
            self.copy_stream = torch.cuda.Stream(device=dev) if copy_stream is None else copy_stream
        self.keep = (q_loc, k_all, v_all)
        self.args = (ctypes.byref(self.shape), cp, rank, q_loc.data_ptr(), k_all.data_ptr(), v_all.data_ptr(),
                     self.qp.data_ptr(), None if self.ql is None else self.ql.data_ptr(), self.kp.data_ptr(),
                     self.out.data_ptr(), self.lse.data_ptr(), self.ws.data_ptr(), self.ws.numel(),
                     None if self.stage is None else self.stage.data_ptr(),
                     0 if self.stage is None else self.stage.numel())
        self.device = dev

    def run(self, stream=None):
        st = _stream(self.device) if stream is None else stream
        cst = st if self.copy_stream is None else self.copy_stream.cuda_stream
        _check(lib().cp_attn_ring_fwd_stepwise(*self.args, st, cst))
        return self.out, self.lse


def cp_attn_ring_fwd_stepwise(q_loc, k_all, v_all, cp, rank, q_pos, q_lo, k_pos_all, scale=None, staged=True,
                              copy_stream=None, out=None, lse=None, workspace=None, stage=None):
    """A virtual rank's ring as separate steps (a partial forward per step,
    merged into the running (O, LSE) in the kernel's epilogue), optionally with
    rotating K/V copies: final fp32 (O, LSE)."""
    return RingFwdStepwisePlan(q_loc, k_all, v_all, cp, rank, q_pos, q_lo, k_pos_all, scale, staged,
                               copy_stream, out, lse, workspace, stage).run()


# ------------------------------------------------------------------ head exchange (all-to-all level)
def _a2a_dtype(t):
    if t.dtype not in _DT:
        raise ValueError("head exchange tensors must be float32 or bfloat16")
    return _DT[t.dtype]


def _a2a_packed(t, g, H, rows, d, dtype, what):
    if t.dtype != dtype or not t.is_contiguous() or tuple(t.shape) != (g, H // g, rows, d):
        raise ValueError(f"{what} must be contiguous {dtype} [{g}, {H // g}, {rows}, {d}]")
    return t


def _a2a_shard(x, what):
    if x.dim() != 3 or x.stride(2) != 1 or x.stride(1) != x.shape[2]:
        raise ValueError(f"{what} must be [rows, heads, d] with heads contiguous within a row")
    return x


def cp_a2a_pack(x, g, send=None):
    """Sequence shard x [rows, H, d] -> send buffer [g, H/g, rows, d]."""
    _a2a_shard(x, "x")
    rows, H, d = x.shape
    send = torch.empty(g, H // max(g, 1), rows, d, dtype=x.dtype, device=x.device) if send is None else send
    _a2a_packed(send, g, H, rows, d, x.dtype, "send")
    _check(lib().cp_a2a_pack(g, H, rows, d, _a2a_dtype(x), x.data_ptr(), x.stride(0), send.data_ptr(), 0,
                             _stream(x.device)))
    return send


def cp_a2a_pack_inverse(send, x):
    """Send buffer [g, H/g, rows, d] -> the sequence shard x [rows, H, d] (written in place)."""
    _a2a_shard(x, "x")
    rows, H, d = x.shape
    g = send.shape[0]
    _a2a_packed(send, g, H, rows, d, x.dtype, "send")
    _check(lib().cp_a2a_pack(g, H, rows, d, _a2a_dtype(x), x.data_ptr(), x.stride(0), send.data_ptr(), 1,
                             _stream(x.device)))
    return x


def cp_a2a_unpack(recv, y=None):
    """Received blocks [g, H/g, rows, d] -> [H/g, g*rows, d] (heads, the group's rows in source order)."""
    g, Hg, rows, d = recv.shape
    _a2a_packed(recv, g, g * Hg, rows, d, recv.dtype, "recv")
    y = torch.empty(Hg, g * rows, d, dtype=recv.dtype, device=recv.device) if y is None else y
    if y.dtype != recv.dtype or not y.is_contiguous() or tuple(y.shape) != (Hg, g * rows, d):
        raise ValueError(f"y must be contiguous [{Hg}, {g * rows}, {d}]")
    _check(lib().cp_a2a_unpack(g, g * Hg, rows, d, _a2a_dtype(recv), recv.data_ptr(), y.data_ptr(), 0,
                               _stream(recv.device)))
    return y


def cp_a2a_unpack_inverse(y, g, recv=None):
    """[H/g, g*rows, d] -> the blocks [g, H/g, rows, d] that the reverse exchange sends back."""
    Hg, n, d = y.shape
    if g < 1 or n % g != 0:
        raise ValueError("the row count of y must be a multiple of g")
    rows = n // g
    if y.dtype not in _DT or not y.is_contiguous():
        raise ValueError("y must be contiguous float32 or bfloat16")
    recv = torch.empty(g, Hg, rows, d, dtype=y.dtype, device=y.device) if recv is None else recv
    _a2a_packed(recv, g, g * Hg, rows, d, y.dtype, "recv")
    _check(lib().cp_a2a_unpack(g, g * Hg, rows, d, _a2a_dtype(y), recv.data_ptr(), y.data_ptr(), 1,
                               _stream(y.device)))
    return recv


# ------------------------------------------------------------------ backward
def _bwd_shape(q, k, v, dout, scale) -> CpShape:
    if dout.dtype != q.dtype or dout.shape != q.shape or dout.stride() != q.stride():
        raise ValueError("dout must match q in dtype, shape and strides")
    return _shape(q, k, v, (ctypes.c_int64 * 3)(0, 0, 0), scale, torch.float32)


def _grad_buf(t, shape, device, what):
    if t is None:
        return torch.zeros(*shape, dtype=torch.float32, device=device)
    if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} must be contiguous float32 {tuple(shape)}")
    return t


def _rows_f32(t, shape, what):
    if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} must be contiguous float32 {tuple(shape)}")
    return t


def cp_attn_bwd_workspace(q, k, v, cp: int = 1) -> int:
    s = _shape(q, k, v, (ctypes.c_int64 * 3)(0, 0, 0), None, torch.float32)
    n = int(lib().cp_attn_bwd_workspace(ctypes.byref(s), cp))
    if n == 0:
        raise ValueError(cp_last_error() or "invalid shape")
    return n


def cp_attn_bwd_delta(dout, o, delta=None):
    """delta = rowsum(dO * O) as contiguous float32 [B, Hq, rows]."""
    if o.dtype not in _DT or tuple(o.shape) != tuple(dout.shape):
        raise ValueError("o must be float32 or bfloat16 with dout's shape")
    B, Hq, Sq, D = dout.shape
    delta = torch.empty(B, Hq, Sq, dtype=torch.float32, device=dout.device) if delta is None else delta
    _rows_f32(delta, (B, Hq, Sq), "delta")
    s = CpShape()
    s.b, s.hq, s.hkv, s.d = B, Hq, Hq, D
    s.sq, s.sk, s.scale = Sq, 0, 1.0
    s.in_dtype = _DT.get(dout.dtype, -1)
    s.out_dtype = _DT[o.dtype]
    s.q_str, s.o_str = _strides(dout), _strides(o)
    s.k_str = s.v_str = (ctypes.c_int64 * 3)(0, 0, 0)
    _check(lib().cp_attn_bwd_delta(ctypes.byref(s), dout.data_ptr(), o.data_ptr(), delta.data_ptr(),
                                   _stream(dout.device)))
    return delta


def cp_attn_partial_bwd(q, k, v, dout, lse, delta, q_pos, q_lo, k_pos, dq=None, dk=None, dv=None, scale=None,
                        workspace=None):
    """Backward of one ring step; adds into (and returns) fp32 dq, dk, dv."""
    dev = q.device
    B, Hq, Sq, D = q.shape
    s = _bwd_shape(q, k, v, dout, scale)
    _rows_f32(lse, (B, Hq, Sq), "lse")
    _rows_f32(delta, (B, Hq, Sq), "delta")
    dq = _grad_buf(dq, q.shape, dev, "dq")
    dk = _grad_buf(dk, k.shape, dev, "dk")
    dv = _grad_buf(dv, v.shape, dev, "dv")
    qp, kp = _dev_i32(q_pos, dev), _dev_i32(k_pos, dev)
    ql = None if q_lo is None else _dev_i32(q_lo, dev)
    ws = _workspace(int(lib().cp_attn_bwd_workspace(ctypes.byref(s), 1)) or 256, dev, workspace)
    _check(lib().cp_attn_partial_bwd(ctypes.byref(s), q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(),
                                     lse.data_ptr(), delta.data_ptr(), qp.data_ptr(),
                                     None if ql is None else ql.data_ptr(), kp.data_ptr(), dq.data_ptr(),
                                     dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev)))
    return dq, dk, dv


class RingBwdPlan:
    """A validated cp_attn_ring_bwd call with its workspace and fp32 gradient
    buffers, replayable with no Python-side allocation.  Each run() adds into
    the buffers; zero them (``zero_()``) to start over."""

    def __init__(self, q_loc, k_all, v_all, dout, lse, delta, cp, rank, q_pos, q_lo, k_pos_all, scale=None,
                 dq=None, dk=None, dv=None, workspace=None):
        dev = q_loc.device
        B, Hq, Sq, D = q_loc.shape
        self.shape = _bwd_shape(q_loc, k_all, v_all, dout, scale)
        _rows_f32(lse, (B, Hq, Sq), "lse")
        _rows_f32(delta, (B, Hq, Sq), "delta")
        self.dq = _grad_buf(dq, q_loc.shape, dev, "dq")
        self.dk = _grad_buf(dk, k_all.shape, dev, "dk")
        self.dv = _grad_buf(dv, v_all.shape, dev, "dv")
        self.qp = _dev_i32(q_pos, dev)
        self.ql = None if q_lo is None else _dev_i32(q_lo, dev)
        self.kp = _dev_i32(k_pos_all, dev)
        nws = int(lib().cp_attn_bwd_workspace(ctypes.byref(self.shape), cp))
        self.ws = _workspace(nws or 256, dev, workspace)
        self.keep = (q_loc, k_all, v_all, dout, lse, delta)
        self.args = (ctypes.byref(self.shape), cp, rank, q_loc.data_ptr(), k_all.data_ptr(), v_all.data_ptr(),
                     dout.data_ptr(), lse.data_ptr(), delta.data_ptr(), self.qp.data_ptr(),
                     None if self.ql is None else self.ql.data_ptr(), self.kp.data_ptr(), self.dq.data_ptr(),
                     self.dk.data_ptr(), self.dv.data_ptr(), self.ws.data_ptr(), self.ws.numel())
        self.device = dev

    def run(self, stream=None):
        st = _stream(self.device) if stream is None else stream
        _check(lib().cp_attn_ring_bwd(*self.args, st))
        return self.dq, self.dk, self.dv


def cp_attn_ring_bwd(q_loc, k_all, v_all, dout, lse, delta, cp, rank, q_pos, q_lo, k_pos_all, scale=None,
                     dq=None, dk=None, dv=None, workspace=None):
    """A virtual rank's whole ring backward: adds into (and returns) fp32
    dq [B,Hq,rows,D] and dk, dv [B,Hkv,S,D] (rank-major rows like k_all)."""
    return RingBwdPlan(q_loc, k_all, v_all, dout, lse, delta, cp, rank, q_pos, q_lo, k_pos_all, scale, dq, dk, dv,
                       workspace).run()
