"""Python binding of libgdpa.so (MI355X / gfx950 GDPA kernels).

Argument marshalling only: every step of the computation runs in the HIP
library.  torch is used for device memory and the current stream.  There is no
fallback: if the shared library is missing or a call fails, an exception is
raised.

    o, lse = fwd(q, offsets, k, v, phi="softmax")
    dq, dk, dv = bwd(q, offsets, k, v, o, lse, do, phi="softmax")
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# GDPA_LIB names another build of the same library (e.g. the host-sanitized copy that
# `python -m context_cross_attention_amd.build --sanitize` writes for CPU-only tests).
LIB_PATH = os.environ.get("GDPA_LIB") or os.path.join(_HERE, "libgdpa.so")

PHI = {"softmax": 0, "silu": 1, "relu": 2, "gelu": 3, "identity": 4}
DTYPE = {torch.float32: 0, torch.bfloat16: 1}
FWD_RESIDUAL = 0x1
BWD_ACCUM_DQ = 0x2
BWD_RESIDUAL = 0x4

STATUS = {0: "GDPA_OK", 1: "GDPA_ERR_INVALID_ARGUMENT", 2: "GDPA_ERR_UNSUPPORTED",
          3: "GDPA_ERR_WORKSPACE_TOO_SMALL", 4: "GDPA_ERR_HIP"}


class GdpaProblem(ctypes.Structure):
    """Mirror of gdpa_problem in include/gdpa.h."""
    _fields_ = [("batch", ctypes.c_int32), ("total_tokens", ctypes.c_int32),
                ("max_seqlen", ctypes.c_int32), ("n_kv", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("phi", ctypes.c_int32), ("scale", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class GdpaGroup(ctypes.Structure):
    """Mirror of gdpa_group in include/gdpa.h."""
    _fields_ = [("problem", GdpaProblem), ("offsets", ctypes.c_void_p), ("kv_offsets", ctypes.c_void_p),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("residual", ctypes.c_void_p), ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("d_o", ctypes.c_void_p), ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p),
                ("dv", ctypes.c_void_p)]


class SwaProblem(ctypes.Structure):
    """Mirror of gdpa_swa_problem in include/gdpa.h."""
    _fields_ = [("batch", ctypes.c_int32), ("total_tokens", ctypes.c_int32),
                ("max_seqlen", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("window", ctypes.c_int32),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class PmaProblem(ctypes.Structure):
    """Mirror of gdpa_pma_problem in include/gdpa.h."""
    _fields_ = [("batch", ctypes.c_int32), ("total_tokens", ctypes.c_int32),
                ("max_seqlen", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("seeds", ctypes.c_int32),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class GdpaError(RuntimeError):
    def __init__(self, status: int, where: str, hip_error: int = 0):
        msg = f"{where}: {STATUS.get(status, status)}"
        if status == 4:
            msg += f" (hipError_t {hip_error})"
        super().__init__(msg)
        self.status = status


_lib = None

EXPORTS = ("gdpa_workspace_bytes", "gdpa_fwd", "gdpa_bwd", "gdpa_weightgen_fwd",
           "gdpa_weightgen_bwd_w", "gdpa_swa_workspace_bytes", "gdpa_swa_fwd", "gdpa_swa_bwd",
           "gdpa_pma_workspace_bytes", "gdpa_pma_fwd", "gdpa_pma_bwd",
           "gdpa_fwd_jagged_kv", "gdpa_bwd_jagged_kv", "gdpa_check_kv_offsets", "gdpa_add_bf16",
           "gdpa_fwd_biased", "gdpa_bwd_biased", "gdpa_biased_workspace_bytes",
           "gdpa_grouped_workspace_bytes", "gdpa_fwd_grouped", "gdpa_bwd_grouped",
           "gdpa_swa_block_fwd", "gdpa_swa_block_bwd", "gdpa_bwd_noalloc", "gdpa_fwd_block",
           "gdpa_check_offsets", "gdpa_status_str", "gdpa_last_hip_error")


def load(path: str = LIB_PATH):
    """Load libgdpa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it with `python -m context_cross_attention_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(GdpaProblem)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.gdpa_workspace_bytes.argtypes = [P, ctypes.c_int]
    lib.gdpa_workspace_bytes.restype = sz
    lib.gdpa_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdpa_fwd.restype = ctypes.c_int
    lib.gdpa_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdpa_bwd.restype = ctypes.c_int
    lib.gdpa_bwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdpa_bwd_noalloc.restype = ctypes.c_int
    lib.gdpa_fwd_block.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdpa_fwd_block.restype = ctypes.c_int
    lib.gdpa_weightgen_fwd.argtypes = [i32, i32, i64, vp, vp, vp, vp]
    lib.gdpa_weightgen_fwd.restype = ctypes.c_int
    lib.gdpa_weightgen_bwd_w.argtypes = [i32, i32, i64, vp, vp, vp, vp]
    lib.gdpa_weightgen_bwd_w.restype = ctypes.c_int
    SP = ctypes.POINTER(SwaProblem)
    lib.gdpa_swa_workspace_bytes.argtypes = [SP, ctypes.c_int]
    lib.gdpa_swa_workspace_bytes.restype = sz
    lib.gdpa_swa_fwd.argtypes = [SP, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdpa_swa_fwd.restype = ctypes.c_int
    lib.gdpa_swa_bwd.argtypes = [SP, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdpa_swa_bwd.restype = ctypes.c_int
    PP = ctypes.POINTER(PmaProblem)
    lib.gdpa_pma_workspace_bytes.argtypes = [PP, ctypes.c_int]
    lib.gdpa_pma_workspace_bytes.restype = sz
    lib.gdpa_pma_fwd.argtypes = [PP, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdpa_pma_fwd.restype = ctypes.c_int
    lib.gdpa_pma_bwd.argtypes = [PP, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdpa_pma_bwd.restype = ctypes.c_int
    lib.gdpa_fwd_jagged_kv.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdpa_fwd_jagged_kv.restype = ctypes.c_int
    lib.gdpa_bwd_jagged_kv.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdpa_bwd_jagged_kv.restype = ctypes.c_int
    GP = ctypes.POINTER(GdpaGroup)
    lib.gdpa_grouped_workspace_bytes.argtypes = [ctypes.c_int32, GP, ctypes.c_int]
    lib.gdpa_grouped_workspace_bytes.restype = sz
    for name in ("gdpa_fwd_grouped", "gdpa_bwd_grouped"):
        getattr(lib, name).argtypes = [ctypes.c_int32, GP, vp, sz, vp]
        getattr(lib, name).restype = ctypes.c_int
    SP = ctypes.POINTER(SwaProblem)
    lib.gdpa_swa_block_fwd.argtypes = [SP, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdpa_swa_block_fwd.restype = ctypes.c_int
    lib.gdpa_swa_block_bwd.argtypes = [SP, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdpa_swa_block_bwd.restype = ctypes.c_int
    lib.gdpa_biased_workspace_bytes.argtypes = [P, ctypes.c_int, ctypes.c_int]
    lib.gdpa_biased_workspace_bytes.restype = sz
    lib.gdpa_fwd_biased.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdpa_fwd_biased.restype = ctypes.c_int
    lib.gdpa_bwd_biased.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdpa_bwd_biased.restype = ctypes.c_int
    lib.gdpa_add_bf16.argtypes = [i64, vp, vp, vp, vp, vp, vp]
    lib.gdpa_add_bf16.restype = ctypes.c_int
    lib.gdpa_check_kv_offsets.argtypes = [vp, i32, i32]
    lib.gdpa_check_kv_offsets.restype = ctypes.c_int
    lib.gdpa_check_offsets.argtypes = [vp, i32, i32, i32]
    lib.gdpa_check_offsets.restype = ctypes.c_int
    lib.gdpa_status_str.argtypes = [ctypes.c_int]
    lib.gdpa_status_str.restype = ctypes.c_char_p
    lib.gdpa_last_hip_error.argtypes = []
    lib.gdpa_last_hip_error.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != 0:
        raise GdpaError(status, where, _lib.gdpa_last_hip_error() if status == 4 else 0)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def default_scale(phi: str, d: int) -> float:
    """1/sqrt(d) for softmax, 1 for the elementwise maps (the plain FFN form)."""
    return 1.0 / math.sqrt(d) if phi == "softmax" else 1.0


def make_problem(q: torch.Tensor, offsets: torch.Tensor, k: torch.Tensor, phi: str,
                 scale: Optional[float], flags: int = 0, max_seqlen: Optional[int] = None,
                 total_tokens: Optional[int] = None) -> GdpaProblem:
    B, n, H, d = k.shape
    T = q.shape[0] if total_tokens is None else total_tokens
    if phi not in PHI:
        raise ValueError(f"phi must be one of {tuple(PHI)}")
    if q.dtype not in DTYPE:
        raise TypeError(f"unsupported dtype {q.dtype}")
    return GdpaProblem(B, T, T if max_seqlen is None else max_seqlen, n, H, d, PHI[phi],
                       default_scale(phi, d) if scale is None else float(scale), DTYPE[q.dtype], flags)


def _require(t: torch.Tensor, name: str, shape, dtype, device):
    if t.shape != torch.Size(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def workspace_bytes(prob: GdpaProblem, backward: bool) -> int:
    return int(load().gdpa_workspace_bytes(ctypes.byref(prob), 1 if backward else 0))


def _sized_workspace(need: int, device, workspace: Optional[torch.Tensor]):
    if workspace is not None and workspace.numel() >= need:
        return workspace
    return torch.empty(max(need, 1), dtype=torch.uint8, device=device)


def _workspace(prob: GdpaProblem, backward: bool, device, workspace: Optional[torch.Tensor]):
    return _sized_workspace(workspace_bytes(prob, backward), device, workspace)


def fwd(q: torch.Tensor, offsets: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
        phi: str = "softmax", scale: Optional[float] = None, residual: Optional[torch.Tensor] = None,
        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
        want_lse: bool = True, workspace: Optional[torch.Tensor] = None
        ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """GDPA forward.  q [T,H,d], offsets int32 [B+1], k, v [B,n,H,d] (same dtype, device).

    Returns (o [T,H,d], lse [T,H] float32 for softmax when want_lse, else None).
    With `residual` ([T,H,d]), o = residual + GDPA(q, k, v).
    """
    lib = load()
    B, n, H, d = k.shape
    T = q.shape[0]
    dev = q.device
    _require(q, "q", (T, H, d), q.dtype, dev)
    _require(k, "k", (B, n, H, d), q.dtype, dev)
    _require(v, "v", (B, n, H, d), q.dtype, dev)
    _require(offsets, "offsets", (B + 1,), torch.int32, dev)
    flags = 0
    if residual is not None:
        _require(residual, "residual", (T, H, d), q.dtype, dev)
        flags |= FWD_RESIDUAL
    if out is None:
        out = torch.empty_like(q)
    _require(out, "out", (T, H, d), q.dtype, dev)
    if phi == "softmax" and want_lse and lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    if phi != "softmax":
        lse = None
    if lse is not None:
        _require(lse, "lse", (T, H), torch.float32, dev)
    prob = make_problem(q, offsets, k, phi, scale, flags)
    ws = _workspace(prob, False, dev, workspace)
    st = lib.gdpa_fwd(ctypes.byref(prob), _ptr(offsets), _ptr(q), _ptr(k), _ptr(v), _ptr(residual),
                      _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream())
    _check(st, "gdpa_fwd")
    return out, lse


def bwd_reads_o(dtype, head_dim: int, n_kv: int) -> bool:
    """Whether the softmax backward reads the forward's output O for its row term.

    The backward that holds a sample's whole context in one work-group (bf16,
    head_dim 128, n_kv <= 256) sums the row term from P and dP itself and reads no O
    (the rule of gdpa_bwd in include/gdpa.h)."""
    return not (dtype == torch.bfloat16 and head_dim == 128 and n_kv <= 256)


def bwd(q: torch.Tensor, offsets: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
        o: Optional[torch.Tensor], lse: Optional[torch.Tensor], do: torch.Tensor,
        phi: str = "softmax", scale: Optional[float] = None, dq: Optional[torch.Tensor] = None,
        accumulate_dq: bool = False, residual: bool = False, dk: Optional[torch.Tensor] = None,
        dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """GDPA backward of sum(O * dO).  Returns (dq, dk, dv).

    For softmax, o and lse are the forward's outputs (o may be None where
    bwd_reads_o() is False); for the elementwise maps they are unused.
    With accumulate_dq, dq (which may be `do` itself) receives dq + dQ.
    With residual, dq receives do + dQ: the gradient of O = Q + GDPA(Q).
    """
    lib = load()
    B, n, H, d = k.shape
    T = q.shape[0]
    dev = q.device
    for name, t in (("q", q), ("do", do)):
        _require(t, name, (T, H, d), q.dtype, dev)
    for name, t in (("k", k), ("v", v)):
        _require(t, name, (B, n, H, d), q.dtype, dev)
    _require(offsets, "offsets", (B + 1,), torch.int32, dev)
    if phi == "softmax":
        if o is not None or bwd_reads_o(q.dtype, d, n):
            _require(o, "o", (T, H, d), q.dtype, dev)
        _require(lse, "lse", (T, H), torch.float32, dev)
    else:
        o, lse = None, None
    flags = 0
    if accumulate_dq:
        if dq is None:
            raise ValueError("accumulate_dq needs dq")
        flags |= BWD_ACCUM_DQ
    if residual:
        flags |= BWD_RESIDUAL
    if dq is None:
        dq = torch.empty_like(q)
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _require(dq, "dq", (T, H, d), q.dtype, dev)
    _require(dk, "dk", (B, n, H, d), q.dtype, dev)
    _require(dv, "dv", (B, n, H, d), q.dtype, dev)
    prob = make_problem(q, offsets, k, phi, scale, flags)
    ws = _workspace(prob, True, dev, workspace)
    st = lib.gdpa_bwd(ctypes.byref(prob), _ptr(offsets), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                      _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(),
                      _stream())
    _check(st, "gdpa_bwd")
    return dq, dk, dv


def fwd_block(x: torch.Tensor, offsets: torch.Tensor, k: torch.Tensor, v: torch.Tensor, phi: str = "softmax",
              scale: Optional[float] = None, o: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
              lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Residual layer block: o = GDPA(x; k, v) and y = x + o in one pass (x [T,H,d] is
    the queries).  Returns (o, y, lse for softmax else None)."""
    lib = load()
    B, n, H, d = k.shape
    T = x.shape[0]
    dev = x.device
    _require(x, "x", (T, H, d), x.dtype, dev)
    _require(k, "k", (B, n, H, d), x.dtype, dev)
    _require(v, "v", (B, n, H, d), x.dtype, dev)
    _require(offsets, "offsets", (B + 1,), torch.int32, dev)
    o = torch.empty_like(x) if o is None else o
    y = torch.empty_like(x) if y is None else y
    _require(o, "o", (T, H, d), x.dtype, dev)
    _require(y, "y", (T, H, d), x.dtype, dev)
    if phi == "softmax":
        lse = torch.empty((T, H), dtype=torch.float32, device=dev) if lse is None else lse
        _require(lse, "lse", (T, H), torch.float32, dev)
    else:
        lse = None
    prob = make_problem(x, offsets, k, phi, scale, 0)
    ws = _workspace(prob, False, dev, workspace)
    _check(lib.gdpa_fwd_block(ctypes.byref(prob), _ptr(offsets), _ptr(x), _ptr(k), _ptr(v), _ptr(o), _ptr(y),
                              _ptr(lse), _ptr(ws), ws.numel(), _stream()), "gdpa_fwd_block")
    return o, y, lse


NOALLOC_SCRATCH_BYTES = 64 << 20  # GDPA_NOALLOC_SCRATCH_BYTES of include/gdpa.h


def bwd_noalloc(q: torch.Tensor, offsets: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                o: Optional[torch.Tensor], lse: Optional[torch.Tensor], do: torch.Tensor, dq: torch.Tensor,
                dk: torch.Tensor, dv: torch.Tensor, phi: str = "softmax", scale: Optional[float] = None,
                accumulate_dq: bool = False, residual: bool = False):
    """gdpa_bwd_noalloc: bwd() into caller-given dq, dk, dv with the library's per-GPU
    scratch as workspace; allocates nothing (calls on one GPU must not overlap)."""
    lib = load()
    B, n, H, d = k.shape
    T = q.shape[0]
    dev = q.device
    for name, t in (("q", q), ("do", do), ("dq", dq)):
        _require(t, name, (T, H, d), q.dtype, dev)
    for name, t in (("k", k), ("v", v), ("dk", dk), ("dv", dv)):
        _require(t, name, (B, n, H, d), q.dtype, dev)
    _require(offsets, "offsets", (B + 1,), torch.int32, dev)
    if phi == "softmax":
        if o is not None or bwd_reads_o(q.dtype, d, n):
            _require(o, "o", (T, H, d), q.dtype, dev)
        _require(lse, "lse", (T, H), torch.float32, dev)
    else:
        o, lse = None, None
    flags = (BWD_ACCUM_DQ if accumulate_dq else 0) | (BWD_RESIDUAL if residual else 0)
    prob = make_problem(q, offsets, k, phi, scale, flags)
    st = lib.gdpa_bwd_noalloc(ctypes.byref(prob), _ptr(offsets), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                              _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), _stream())
    _check(st, "gdpa_bwd_noalloc")
    return dq, dk, dv


def _jagged_problem(q, offsets, k, n_kv: int, phi: str, scale: Optional[float], flags: int) -> GdpaProblem:
    T, H, d = q.shape
    if phi not in PHI:
        raise ValueError(f"phi must be one of {tuple(PHI)}")
    if q.dtype not in DTYPE:
        raise TypeError(f"unsupported dtype {q.dtype}")
    return GdpaProblem(offsets.shape[0] - 1, T, T, int(n_kv), H, d, PHI[phi],
                       default_scale(phi, d) if scale is None else float(scale), DTYPE[q.dtype], flags)


def jagged_kv_workspace_bytes(q: torch.Tensor, offsets: torch.Tensor, k: torch.Tensor, n_kv: int,
                              phi: str, backward: bool) -> int:
    """Workspace bytes of fwd_jagged_kv (backward=False) or bwd_jagged_kv (backward=True)."""
    prob = _jagged_problem(q, offsets, k, n_kv, phi, None, 0)
    return int(load().gdpa_workspace_bytes(ctypes.byref(prob), 1 if backward else 0))


def fwd_jagged_kv(q: torch.Tensor, offsets: torch.Tensor, kv_offsets: torch.Tensor, k: torch.Tensor,
                  v: torch.Tensor, n_kv: int, phi: str = "softmax", scale: Optional[float] = None,
                  residual: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                  lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """GDPA forward with a jagged context: sample b owns rows kv_offsets[b] .. kv_offsets[b+1]-1
    of k, v [rows,H,d]; n_kv is the largest per-sample count (1 <= count <= n_kv).
    Returns (o [T,H,d], lse [T,H] for softmax else None)."""
    lib = load()
    T, H, d = q.shape
    B = offsets.shape[0] - 1
    dev = q.device
    _require(q, "q", (T, H, d), q.dtype, dev)
    _require(offsets, "offsets", (B + 1,), torch.int32, dev)
    _require(kv_offsets, "kv_offsets", (B + 1,), torch.int32, dev)
    for name, t in (("k", k), ("v", v)):
        _require(t, name, (k.shape[0], H, d), q.dtype, dev)
    flags = 0
    if residual is not None:
        _require(residual, "residual", (T, H, d), q.dtype, dev)
        flags |= FWD_RESIDUAL
    out = torch.empty_like(q) if out is None else out
    _require(out, "out", (T, H, d), q.dtype, dev)
    if phi == "softmax":
        lse = torch.empty((T, H), dtype=torch.float32, device=dev) if lse is None else lse
        _require(lse, "lse", (T, H), torch.float32, dev)
    else:
        lse = None
    prob = _jagged_problem(q, offsets, k, n_kv, phi, scale, flags)
    ws = _workspace(prob, False, dev, workspace)
    _check(lib.gdpa_fwd_jagged_kv(ctypes.byref(prob), _ptr(offsets), _ptr(kv_offsets), _ptr(q), _ptr(k),
                                  _ptr(v), _ptr(residual), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                                  _stream()), "gdpa_fwd_jagged_kv")
    return out, lse


def bwd_jagged_kv(q: torch.Tensor, offsets: torch.Tensor, kv_offsets: torch.Tensor, k: torch.Tensor,
                  v: torch.Tensor, n_kv: int, o: Optional[torch.Tensor], lse: Optional[torch.Tensor],
                  do: torch.Tensor, phi: str = "softmax", scale: Optional[float] = None,
                  dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                  dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Backward of fwd_jagged_kv: returns (dq [T,H,d], dk, dv [rows,H,d])."""
    lib = load()
    T, H, d = q.shape
    B = offsets.shape[0] - 1
    dev = q.device
    _require(q, "q", (T, H, d), q.dtype, dev)
    _require(offsets, "offsets", (B + 1,), torch.int32, dev)
    _require(kv_offsets, "kv_offsets", (B + 1,), torch.int32, dev)
    for name, t in (("k", k), ("v", v)):
        _require(t, name, (k.shape[0], H, d), q.dtype, dev)
    _require(do, "do", (T, H, d), q.dtype, dev)
    if phi == "softmax":
        _require(o, "o", (T, H, d), q.dtype, dev)
        _require(lse, "lse", (T, H), torch.float32, dev)
    else:
        o, lse = None, None
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _require(dq, "dq", (T, H, d), q.dtype, dev)
    _require(dk, "dk", (k.shape[0], H, d), q.dtype, dev)
    _require(dv, "dv", (k.shape[0], H, d), q.dtype, dev)
    prob = _jagged_problem(q, offsets, k, n_kv, phi, scale, 0)
    ws = _workspace(prob, True, dev, workspace)
    _check(lib.gdpa_bwd_jagged_kv(ctypes.byref(prob), _ptr(offsets), _ptr(kv_offsets), _ptr(q), _ptr(k),
                                  _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv),
                                  _ptr(ws), ws.numel(), _stream()), "gdpa_bwd_jagged_kv")
    return dq, dk, dv


def add_bf16(out: torch.Tensor, x0: torch.Tensor, x1: torch.Tensor, x2: Optional[torch.Tensor] = None,
             x3: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out = x0 + x1 (+ x2) (+ x3), bf16 tensors of one size (out may alias an input)."""
    for name, t in (("x0", x0), ("x1", x1), ("x2", x2), ("x3", x3)):
        if t is not None:
            _require(t, name, out.shape, torch.bfloat16, out.device)
    _require(out, "out", out.shape, torch.bfloat16, out.device)
    _check(load().gdpa_add_bf16(out.numel(), _ptr(out), _ptr(x0), _ptr(x1), _ptr(x2), _ptr(x3), _stream()),
           "gdpa_add_bf16")
    return out


def _biased_shapes(q, offsets, k, kv_offsets, n_kv):
    T, H, d = q.shape
    B = offsets.shape[0] - 1
    if kv_offsets is None:
        n = k.shape[1]
        return B, n, (B, n, H, d), (B, n, H)
    if n_kv is None:
        raise ValueError("a jagged context needs n_kv, the largest per-sample row count")
    return B, int(n_kv), (k.shape[0], H, d), (k.shape[0], H)


def biased_workspace_bytes(q: torch.Tensor, offsets: torch.Tensor, k: torch.Tensor, phi: str, backward: bool,
                           out_bias: bool, kv_offsets: Optional[torch.Tensor] = None,
                           n_kv: Optional[int] = None) -> int:
    """Workspace bytes of fwd_biased / bwd_biased (out_bias: an output bias is given)."""
    _, n, _, _ = _biased_shapes(q, offsets, k, kv_offsets, n_kv)
    prob = _jagged_problem(q, offsets, k, n, phi, None, 0)
    return int(load().gdpa_biased_workspace_bytes(ctypes.byref(prob), int(backward), int(out_bias)))


def fwd_biased(q: torch.Tensor, offsets: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
               score_bias: Optional[torch.Tensor], out_bias: Optional[torch.Tensor], phi: str = "softmax",
               scale: Optional[float] = None, kv_offsets: Optional[torch.Tensor] = None,
               n_kv: Optional[int] = None, out: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """GDPA forward with FFN biases: O = phi(scale Q K^T + score_bias) V + out_bias.
    score_bias float32 [B,n,H] (or [rows,H] with kv_offsets), out_bias float32 [B,H,d];
    either may be None.  Returns (o, lse for softmax else None)."""
    lib = load()
    T, H, d = q.shape
    dev = q.device
    _require(q, "q", (T, H, d), q.dtype, dev)
    B, n, kshape, sbshape = _biased_shapes(q, offsets, k, kv_offsets, n_kv)
    _require(offsets, "offsets", (B + 1,), torch.int32, dev)
    for name, t in (("k", k), ("v", v)):
        _require(t, name, kshape, q.dtype, dev)
    if kv_offsets is not None:
        _require(kv_offsets, "kv_offsets", (B + 1,), torch.int32, dev)
    if score_bias is not None:
        _require(score_bias, "score_bias", sbshape, torch.float32, dev)
    if out_bias is not None:
        _require(out_bias, "out_bias", (B, H, d), torch.float32, dev)
    out = torch.empty_like(q) if out is None else out
    _require(out, "out", (T, H, d), q.dtype, dev)
    lse = (torch.empty((T, H), dtype=torch.float32, device=dev) if lse is None else lse) if phi == "softmax" else None
    if lse is not None:
        _require(lse, "lse", (T, H), torch.float32, dev)
    prob = _jagged_problem(q, offsets, k, n, phi, scale, 0)
    ws = _workspace(prob, False, dev, workspace)
    _check(lib.gdpa_fwd_biased(ctypes.byref(prob), _ptr(offsets), _ptr(kv_offsets), _ptr(q), _ptr(k), _ptr(v),
                               _ptr(score_bias), _ptr(out_bias), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                               _stream()), "gdpa_fwd_biased")
    return out, lse


def bwd_biased(q: torch.Tensor, offsets: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
               score_bias: Optional[torch.Tensor], out_bias: Optional[torch.Tensor], o: Optional[torch.Tensor],
               lse: Optional[torch.Tensor], do: torch.Tensor, phi: str = "softmax", scale: Optional[float] = None,
               kv_offsets: Optional[torch.Tensor] = None, n_kv: Optional[int] = None,
               workspace: Optional[torch.Tensor] = None, dq: Optional[torch.Tensor] = None,
               dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
               d_score_bias: Optional[torch.Tensor] = None, d_out_bias: Optional[torch.Tensor] = None):
    """Backward of fwd_biased: returns (dq, dk, dv, d_score_bias, d_out_bias)."""
    lib = load()
    T, H, d = q.shape
    dev = q.device
    _require(q, "q", (T, H, d), q.dtype, dev)
    B, n, kshape, sbshape = _biased_shapes(q, offsets, k, kv_offsets, n_kv)
    _require(offsets, "offsets", (B + 1,), torch.int32, dev)
    for name, t in (("k", k), ("v", v)):
        _require(t, name, kshape, q.dtype, dev)
    _require(do, "do", (T, H, d), q.dtype, dev)
    if phi == "softmax":
        _require(o, "o", (T, H, d), q.dtype, dev)
        _require(lse, "lse", (T, H), torch.float32, dev)
    else:
        o, lse = None, None
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, shape in (("dq", dq, (T, H, d)), ("dk", dk, kshape), ("dv", dv, kshape)):
        _require(t, name, shape, q.dtype, dev)
    dsb = torch.empty(sbshape, dtype=torch.float32, device=dev) if d_score_bias is None else d_score_bias
    dob = torch.empty((B, H, d), dtype=torch.float32, device=dev) if d_out_bias is None else d_out_bias
    _require(dsb, "d_score_bias", sbshape, torch.float32, dev)
    _require(dob, "d_out_bias", (B, H, d), torch.float32, dev)
    prob = _jagged_problem(q, offsets, k, n, phi, scale, 0)
    need = lib.gdpa_biased_workspace_bytes(ctypes.byref(prob), 1, int(out_bias is not None))
    ws = _sized_workspace(need, dev, workspace)
    _check(lib.gdpa_bwd_biased(ctypes.byref(prob), _ptr(offsets), _ptr(kv_offsets), _ptr(q), _ptr(k), _ptr(v),
                               _ptr(score_bias), _ptr(out_bias), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk),
                               _ptr(dv), _ptr(dsb), _ptr(dob), _ptr(ws), ws.numel(), _stream()), "gdpa_bwd_biased")
    return dq, dk, dv, dsb, dob


@dataclass
class GroupSpec:
    """One problem of a grouped call: q [T,H,d], offsets int32 [B+1], k, v [B,n,H,d]
    (or [rows,H,d] with kv_offsets and n_kv), its own score map and scale."""
    q: torch.Tensor
    offsets: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    phi: str = "softmax"
    scale: Optional[float] = None
    kv_offsets: Optional[torch.Tensor] = None
    n_kv: Optional[int] = None

    def problem(self) -> GdpaProblem:
        T, H, d = self.q.shape
        dev = self.q.device
        _require(self.q, "q", (T, H, d), self.q.dtype, dev)
        B = self.offsets.shape[0] - 1
        _require(self.offsets, "offsets", (B + 1,), torch.int32, dev)
        if self.kv_offsets is None:
            n = self.k.shape[1]
            kshape = (B, n, H, d)
        else:
            if self.n_kv is None:
                raise ValueError("a jagged context needs n_kv")
            _require(self.kv_offsets, "kv_offsets", (B + 1,), torch.int32, dev)
            n, kshape = int(self.n_kv), (self.k.shape[0], H, d)
        _require(self.k, "k", kshape, self.q.dtype, dev)
        _require(self.v, "v", kshape, self.q.dtype, dev)
        return _jagged_problem(self.q, self.offsets, self.k, n, self.phi, self.scale, 0)


def _groups(specs: Sequence[GroupSpec]):
    arr = (GdpaGroup * len(specs))()
    for i, sp in enumerate(specs):
        g = arr[i]
        g.problem = sp.problem()
        g.offsets, g.kv_offsets = sp.offsets.data_ptr(), _addr(sp.kv_offsets)
        g.q, g.k, g.v = sp.q.data_ptr(), sp.k.data_ptr(), sp.v.data_ptr()
    return arr


def _addr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def grouped_workspace_bytes(specs: Sequence[GroupSpec], backward: bool) -> int:
    arr = _groups(specs)
    return int(load().gdpa_grouped_workspace_bytes(len(specs), arr, int(backward)))


def fwd_grouped(specs: Sequence[GroupSpec], outs: Optional[Sequence[Tuple[torch.Tensor, Optional[torch.Tensor]]]] = None,
                workspace: Optional[torch.Tensor] = None):
    """Forward of several independent GDPA problems in one call (they run
    concurrently).  Returns [(o, lse or None)] per group."""
    lib = load()
    arr = _groups(specs)
    res = []
    for i, sp in enumerate(specs):
        T, H, d = sp.q.shape
        o, lse = (None, None) if outs is None else outs[i]
        o = torch.empty_like(sp.q) if o is None else o
        _require(o, "o", (T, H, d), sp.q.dtype, sp.q.device)
        if sp.phi == "softmax":
            lse = torch.empty((T, H), dtype=torch.float32, device=sp.q.device) if lse is None else lse
            _require(lse, "lse", (T, H), torch.float32, sp.q.device)
        else:
            lse = None
        arr[i].o, arr[i].lse = o.data_ptr(), _addr(lse)
        res.append((o, lse))
    need = lib.gdpa_grouped_workspace_bytes(len(specs), arr, 0)
    ws = _sized_workspace(need, specs[0].q.device, workspace)
    _check(lib.gdpa_fwd_grouped(len(specs), arr, _ptr(ws), ws.numel(), _stream()), "gdpa_fwd_grouped")
    return res


def bwd_grouped(specs: Sequence[GroupSpec], fwd_outs: Sequence[Tuple[Optional[torch.Tensor], Optional[torch.Tensor]]],
                dos: Sequence[torch.Tensor], grads: Optional[Sequence[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]]] = None,
                workspace: Optional[torch.Tensor] = None):
    """Backward of fwd_grouped: fwd_outs[i] = (o, lse) (softmax groups), dos[i] = dO.
    Returns [(dq, dk, dv)] per group."""
    lib = load()
    arr = _groups(specs)
    res = []
    for i, sp in enumerate(specs):
        T, H, d = sp.q.shape
        dev = sp.q.device
        _require(dos[i], "do", (T, H, d), sp.q.dtype, dev)
        o, lse = fwd_outs[i]
        if sp.phi == "softmax":
            _require(o, "o", (T, H, d), sp.q.dtype, dev)
            _require(lse, "lse", (T, H), torch.float32, dev)
        else:
            o, lse = None, None
        dq, dk, dv = (None, None, None) if grads is None else grads[i]
        dq = torch.empty_like(sp.q) if dq is None else dq
        dk = torch.empty_like(sp.k) if dk is None else dk
        dv = torch.empty_like(sp.v) if dv is None else dv
        _require(dq, "dq", (T, H, d), sp.q.dtype, dev)
        _require(dk, "dk", tuple(sp.k.shape), sp.q.dtype, dev)
        _require(dv, "dv", tuple(sp.v.shape), sp.q.dtype, dev)
        g = arr[i]
        g.o, g.lse, g.d_o = _addr(o), _addr(lse), dos[i].data_ptr()
        g.dq, g.dk, g.dv = dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
        res.append((dq, dk, dv))
    need = lib.gdpa_grouped_workspace_bytes(len(specs), arr, 1)
    ws = _sized_workspace(need, specs[0].q.device, workspace)
    _check(lib.gdpa_bwd_grouped(len(specs), arr, _ptr(ws), ws.numel(), _stream()), "gdpa_bwd_grouped")
    return res


def check_kv_offsets(kv_offsets, n_kv: int) -> bool:
    """Host-side check of a kv_offsets array (list / numpy / CPU tensor)."""
    t = torch.as_tensor(kv_offsets, dtype=torch.int32).contiguous().cpu()
    return load().gdpa_check_kv_offsets(ctypes.c_void_p(t.data_ptr()), t.numel() - 1, int(n_kv)) == 0


def _swa_problem(q: torch.Tensor, offsets: torch.Tensor, window: int, scale: Optional[float]):
    T, H, d = q.shape
    if q.dtype not in DTYPE:
        raise TypeError(f"unsupported dtype {q.dtype}")
    return SwaProblem(offsets.shape[0] - 1, T, T, H, d, int(window),
                      1.0 / math.sqrt(d) if scale is None else float(scale), DTYPE[q.dtype], 0)


def swa_workspace_bytes(q: torch.Tensor, offsets: torch.Tensor, window: int, backward: bool) -> int:
    """Workspace bytes of swa_fwd (backward=False) or swa_bwd (backward=True)."""
    prob = _swa_problem(q, offsets, window, None)
    return int(load().gdpa_swa_workspace_bytes(ctypes.byref(prob), 1 if backward else 0))


def _swa_workspace(prob: SwaProblem, backward: bool, device, workspace: Optional[torch.Tensor]):
    need = int(load().gdpa_swa_workspace_bytes(ctypes.byref(prob), 1 if backward else 0))
    if workspace is not None and workspace.numel() >= need:
        return workspace
    return torch.empty(max(need, 1), dtype=torch.uint8, device=device)


def swa_fwd(q: torch.Tensor, offsets: torch.Tensor, k: torch.Tensor, v: torch.Tensor, window: int,
            scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Sliding-window self-attention forward over the jagged batch: q, k, v [T,H,d] bf16,
    token i of a sample attends to its tokens j with i - window < j <= i.  Returns (o, lse)."""
    lib = load()
    T, H, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require(t, name, (T, H, d), q.dtype, dev)
    _require(offsets, "offsets", (offsets.shape[0],), torch.int32, dev)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((T, H), dtype=torch.float32, device=dev) if lse is None else lse
    _require(out, "out", (T, H, d), q.dtype, dev)
    _require(lse, "lse", (T, H), torch.float32, dev)
    prob = _swa_problem(q, offsets, window, scale)
    ws = _swa_workspace(prob, False, dev, workspace)
    _check(lib.gdpa_swa_fwd(ctypes.byref(prob), _ptr(offsets), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                            _ptr(lse), _ptr(ws), ws.numel(), _stream()), "gdpa_swa_fwd")
    return out, lse


def swa_bwd(q: torch.Tensor, offsets: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
            o: torch.Tensor, lse: torch.Tensor, do: torch.Tensor, window: int,
            scale: Optional[float] = None, dq: Optional[torch.Tensor] = None,
            dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None):
    """Sliding-window self-attention backward of sum(O * dO).  Returns (dq, dk, dv)."""
    lib = load()
    T, H, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _require(t, name, (T, H, d), q.dtype, dev)
    _require(lse, "lse", (T, H), torch.float32, dev)
    _require(offsets, "offsets", (offsets.shape[0],), torch.int32, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _require(t, name, (T, H, d), q.dtype, dev)
    prob = _swa_problem(q, offsets, window, scale)
    ws = _swa_workspace(prob, True, dev, workspace)
    _check(lib.gdpa_swa_bwd(ctypes.byref(prob), _ptr(offsets), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                            _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(),
                            _stream()), "gdpa_swa_bwd")
    return dq, dk, dv


def swa_block_fwd(x: torch.Tensor, offsets: torch.Tensor, window: int, scale: Optional[float] = None,
                  o: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                  lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Self-attention block with its residual: y = x + SWA(x, x, x).  Returns (y, o, lse);
    o and lse are what swa_block_bwd needs."""
    lib = load()
    T, H, d = x.shape
    dev = x.device
    _require(x, "x", (T, H, d), x.dtype, dev)
    _require(offsets, "offsets", (offsets.shape[0],), torch.int32, dev)
    o = torch.empty_like(x) if o is None else o
    y = torch.empty_like(x) if y is None else y
    lse = torch.empty((T, H), dtype=torch.float32, device=dev) if lse is None else lse
    for name, t in (("o", o), ("y", y)):
        _require(t, name, (T, H, d), x.dtype, dev)
    _require(lse, "lse", (T, H), torch.float32, dev)
    prob = _swa_problem(x, offsets, window, scale)
    ws = _swa_workspace(prob, False, dev, workspace)
    _check(lib.gdpa_swa_block_fwd(ctypes.byref(prob), _ptr(offsets), _ptr(x), _ptr(o), _ptr(y), _ptr(lse),
                                  _ptr(ws), ws.numel(), _stream()), "gdpa_swa_block_fwd")
    return y, o, lse


def swa_block_bwd(x: torch.Tensor, offsets: torch.Tensor, o: torch.Tensor, lse: torch.Tensor, dy: torch.Tensor,
                  window: int, scale: Optional[float] = None, dx: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None):
    """Backward of swa_block_fwd: dx = dy + dQ + dK + dV.  Returns dx."""
    lib = load()
    T, H, d = x.shape
    dev = x.device
    for name, t in (("x", x), ("o", o), ("dy", dy)):
        _require(t, name, (T, H, d), x.dtype, dev)
    _require(lse, "lse", (T, H), torch.float32, dev)
    _require(offsets, "offsets", (offsets.shape[0],), torch.int32, dev)
    dx = torch.empty_like(x) if dx is None else dx
    _require(dx, "dx", (T, H, d), x.dtype, dev)
    prob = _swa_problem(x, offsets, window, scale)
    ws = _swa_workspace(prob, True, dev, workspace)
    _check(lib.gdpa_swa_block_bwd(ctypes.byref(prob), _ptr(offsets), _ptr(x), _ptr(o), _ptr(lse), _ptr(dy),
                                  _ptr(dx), _ptr(ws), ws.numel(), _stream()), "gdpa_swa_block_bwd")
    return dx


def _pma_problem(seeds: torch.Tensor, offsets: torch.Tensor, k: torch.Tensor, scale: Optional[float]):
    m, H, d = seeds.shape
    if seeds.dtype not in DTYPE:
        raise TypeError(f"unsupported dtype {seeds.dtype}")
    return PmaProblem(offsets.shape[0] - 1, k.shape[0], k.shape[0], H, d, m,
                      1.0 / math.sqrt(d) if scale is None else float(scale), DTYPE[seeds.dtype], 0)


def pma_workspace_bytes(seeds: torch.Tensor, offsets: torch.Tensor, k: torch.Tensor, backward: bool) -> int:
    """Workspace bytes of pma_fwd (backward=False) or pma_bwd (backward=True)."""
    prob = _pma_problem(seeds, offsets, k, None)
    return int(load().gdpa_pma_workspace_bytes(ctypes.byref(prob), 1 if backward else 0))


def _pma_workspace(prob: PmaProblem, backward: bool, device, workspace: Optional[torch.Tensor]):
    need = int(load().gdpa_pma_workspace_bytes(ctypes.byref(prob), 1 if backward else 0))
    if workspace is not None and workspace.numel() >= need:
        return workspace
    return torch.empty(max(need, 1), dtype=torch.uint8, device=device)


def pma_fwd(seeds: torch.Tensor, offsets: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
            scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Seed pooling attention forward: seeds [m,H,d], k, v [T,H,d] bf16 over the jagged
    batch; returns (o [B,m,H,d], lse [B,m,H] float32)."""
    lib = load()
    m, H, d = seeds.shape
    T = k.shape[0]
    B = offsets.shape[0] - 1
    dev = seeds.device
    for name, t in (("k", k), ("v", v)):
        _require(t, name, (T, H, d), seeds.dtype, dev)
    _require(seeds, "seeds", (m, H, d), seeds.dtype, dev)
    _require(offsets, "offsets", (B + 1,), torch.int32, dev)
    out = torch.empty((B, m, H, d), dtype=seeds.dtype, device=dev) if out is None else out
    lse = torch.empty((B, m, H), dtype=torch.float32, device=dev) if lse is None else lse
    _require(out, "out", (B, m, H, d), seeds.dtype, dev)
    _require(lse, "lse", (B, m, H), torch.float32, dev)
    prob = _pma_problem(seeds, offsets, k, scale)
    ws = _pma_workspace(prob, False, dev, workspace)
    _check(lib.gdpa_pma_fwd(ctypes.byref(prob), _ptr(offsets), _ptr(seeds), _ptr(k), _ptr(v), _ptr(out),
                            _ptr(lse), _ptr(ws), ws.numel(), _stream()), "gdpa_pma_fwd")
    return out, lse


PMA_BWD_KV_SUM = 0x1  # gdpa_pma_bwd: dk receives dK + dV


def pma_bwd(seeds: torch.Tensor, offsets: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
            o: torch.Tensor, lse: torch.Tensor, do: torch.Tensor, scale: Optional[float] = None,
            d_seeds: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
            dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
            kv_sum: bool = False):
    """Seed pooling attention backward of sum(O * dO).  Returns (d_seeds [m,H,d], dk, dv);
    with kv_sum (a sequence pooled with itself, k is v) dk holds dK + dV and dv is None."""
    lib = load()
    m, H, d = seeds.shape
    T = k.shape[0]
    B = offsets.shape[0] - 1
    dev = seeds.device
    for name, t in (("k", k), ("v", v)):
        _require(t, name, (T, H, d), seeds.dtype, dev)
    for name, t in (("o", o), ("do", do)):
        _require(t, name, (B, m, H, d), seeds.dtype, dev)
    _require(seeds, "seeds", (m, H, d), seeds.dtype, dev)
    _require(lse, "lse", (B, m, H), torch.float32, dev)
    _require(offsets, "offsets", (B + 1,), torch.int32, dev)
    d_seeds = torch.empty_like(seeds) if d_seeds is None else d_seeds
    dk = torch.empty_like(k) if dk is None else dk
    dv = None if kv_sum else (torch.empty_like(v) if dv is None else dv)
    _require(d_seeds, "d_seeds", (m, H, d), seeds.dtype, dev)
    for name, t in (("dk", dk), ("dv", dv)):
        if t is not None:
            _require(t, name, (T, H, d), seeds.dtype, dev)
    prob = _pma_problem(seeds, offsets, k, scale)
    if kv_sum:
        prob.flags = PMA_BWD_KV_SUM
    ws = _pma_workspace(prob, True, dev, workspace)
    _check(lib.gdpa_pma_bwd(ctypes.byref(prob), _ptr(offsets), _ptr(seeds), _ptr(k), _ptr(v), _ptr(o),
                            _ptr(lse), _ptr(do), _ptr(d_seeds), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(),
                            _stream()), "gdpa_pma_bwd")
    return d_seeds, dk, dv


def weightgen_fwd(ctx: torch.Tensor, w: torch.Tensor, out: Optional[torch.Tensor] = None):
    """out[B, cols] = ctx[B, c] @ w[cols, c]^T (bf16, fp32 accumulation)."""
    lib = load()
    B, c = ctx.shape
    cols = w.shape[0]
    _require(ctx, "ctx", (B, c), torch.bfloat16, ctx.device)
    _require(w, "w", (cols, c), torch.bfloat16, ctx.device)
    if out is None:
        out = torch.empty((B, cols), dtype=torch.bfloat16, device=ctx.device)
    _require(out, "out", (B, cols), torch.bfloat16, ctx.device)
    _check(lib.gdpa_weightgen_fwd(B, c, cols, _ptr(ctx), _ptr(w), _ptr(out), _stream()),
           "gdpa_weightgen_fwd")
    return out


def weightgen_bwd_w(ctx: torch.Tensor, d_out: torch.Tensor, d_w: Optional[torch.Tensor] = None):
    """d_w[cols, c] = d_out[B, cols]^T @ ctx[B, c] (bf16, fp32 accumulation)."""
    lib = load()
    B, c = ctx.shape
    cols = d_out.shape[1]
    _require(ctx, "ctx", (B, c), torch.bfloat16, ctx.device)
    _require(d_out, "d_out", (B, cols), torch.bfloat16, ctx.device)
    if d_w is None:
        d_w = torch.empty((cols, c), dtype=torch.bfloat16, device=ctx.device)
    _require(d_w, "d_w", (cols, c), torch.bfloat16, ctx.device)
    _check(lib.gdpa_weightgen_bwd_w(B, c, cols, _ptr(ctx), _ptr(d_out), _ptr(d_w), _stream()),
           "gdpa_weightgen_bwd_w")
    return d_w


def check_offsets(offsets_host, total_tokens: int, max_seqlen: int) -> bool:
    """Host-side offsets check (gdpa_check_offsets) on a CPU int32 tensor."""
    lib = load()
    t = torch.as_tensor(offsets_host, dtype=torch.int32).contiguous()
    return lib.gdpa_check_offsets(ctypes.c_void_p(t.data_ptr()), t.numel() - 1, total_tokens,
                                  max_seqlen) == 0
