"""Exact, IO-aware tiled softmax attention for AMD Instinct MI355X (gfx950).

Thin Python binding of ``libfa.so`` (C ABI in ``include/fa.h``).  Every
function here only marshals arguments: it checks tensor dtype, device and
shape, allocates outputs with torch when the caller passes none, and hands raw
device pointers plus the current HIP stream to the library.  All arithmetic
runs in the library's HIP kernels; there is no CPU or PyTorch fallback, and a
missing library raises.  Tensors are bfloat16 or float16 (all 16-bit
tensors of a call share q's type; float16 calls go to the *_f16 entry points).
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["load", "build", "FaError", "fa_fwd", "fa_fwd_qk", "fa_fwd_splitkv",
           "fa_fwd_splitkv_workspace_size", "fa_fwd_varlen", "fa_bwd", "fa_bwd_varlen",
           "fa_bwd_workspace_size", "fa_bwd_noalloc", "fa_status_string", "LIB_PATH"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")
_lib = None

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float


class FaError(RuntimeError):
    """A non-zero fa_status returned by the library."""

    def __init__(self, status: int, where: str):
        self.status = int(status)
        super().__init__("%s: %s" % (where, fa_status_string(status)))


def build() -> str:
    """Compile libfa.so for gfx950 (always recompiles)."""
    from . import buildlib
    return buildlib.build()


def load() -> ctypes.CDLL:
    """Load libfa.so (building it first if it is absent) and declare the ABI."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    lib.fa_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp]
    lib.fa_fwd.restype = _i
    lib.fa_fwd_qk.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp]
    lib.fa_fwd_qk.restype = _i
    lib.fa_fwd_splitkv_workspace_size.argtypes = [_i, _i, _i, _i, _i, _i]
    lib.fa_fwd_splitkv_workspace_size.restype = ctypes.c_size_t
    lib.fa_fwd_splitkv.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _i, _i,
                                   _i, _i, _i, _f, _i, _i, _vp]
    lib.fa_fwd_splitkv.restype = _i
    lib.fa_fwd_varlen.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i,
                                  _i, _f, _i, _vp]
    lib.fa_fwd_varlen.restype = _i
    lib.fa_bwd_workspace_size.argtypes = [_i, _i, _i, _i]
    lib.fa_bwd_workspace_size.restype = ctypes.c_size_t
    lib.fa_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                           ctypes.c_size_t, _i, _i, _i, _i, _f, _i, _vp]
    lib.fa_bwd.restype = _i
    lib.fa_bwd_varlen.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i,
                                  _i, _vp, ctypes.c_size_t, _i, _i, _f, _i, _vp]
    lib.fa_bwd_varlen.restype = _i
    lib.fa_bwd_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i,
                                   _i, _f, _i, _vp]
    lib.fa_bwd_noalloc.restype = _i
    lib.fa_status_string.argtypes = [_i]
    lib.fa_status_string.restype = ctypes.c_char_p
    _u64 = ctypes.c_uint64
    lib.fa_fwd_dropout.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _f, _u64,
                                   _u64, _vp]
    lib.fa_fwd_dropout.restype = _i
    lib.fa_bwd_dropout.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                   ctypes.c_size_t, _i, _i, _i, _i, _f, _i, _f, _u64, _u64,
                                   _vp]
    lib.fa_bwd_dropout.restype = _i
    lib.fa_fwd_varlen_dropout.argtypes = lib.fa_fwd_varlen.argtypes[:-1] + [_f, _u64, _u64,
                                                                            _vp]
    lib.fa_fwd_varlen_dropout.restype = _i
    lib.fa_bwd_varlen_dropout.argtypes = lib.fa_bwd_varlen.argtypes[:-1] + [_f, _u64, _u64,
                                                                            _vp]
    lib.fa_bwd_varlen_dropout.restype = _i
    for name in ("fa_fwd", "fa_fwd_qk", "fa_fwd_splitkv", "fa_fwd_varlen", "fa_bwd",
                 "fa_bwd_varlen", "fa_fwd_dropout", "fa_bwd_dropout", "fa_fwd_varlen_dropout",
                 "fa_bwd_varlen_dropout"):
        f16 = getattr(lib, name + "_f16")  # the fp16 twin: same arguments
        f16.argtypes = getattr(lib, name).argtypes
        f16.restype = _i
    _lib = lib
    return lib


def fa_status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def fa_bwd_workspace_size(B: int, H: int, N: int, D: int) -> int:
    return int(load().fa_bwd_workspace_size(B, H, N, D))


# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _check(t, name, shape=None, dtype=None):
    """GPU, contiguous, 16-bit (bf16 or fp16; ``dtype`` when given: the
    tensors of one call share q's element type), optionally of ``shape``."""
    torch = _torch()
    if dtype is None and t.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("%s must be bfloat16 or float16, got %s" % (name, t.dtype))
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s like q, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape),
                                                         tuple(shape)))


def _check_lse(lse, shape, device):
    """A caller-supplied L buffer: contiguous float32 of ``shape`` on the
    GPU of q (a host tensor would hand the kernels a host address)."""
    torch = _torch()
    if lse is None:
        return
    if (lse.dtype != torch.float32 or tuple(lse.shape) != tuple(shape)
            or not lse.is_contiguous()):
        raise ValueError("lse must be contiguous float32 %s" % (list(shape),))
    if not lse.is_cuda or lse.device != device:
        raise ValueError("lse must be on %s like q" % (device,))


def _check_workspace(ws, device):
    """A caller-supplied workspace: contiguous, on the GPU of q."""
    if ws is None:
        return
    if not ws.is_cuda or ws.device != device:
        raise ValueError("workspace must be a GPU tensor on %s like q" % (device,))
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")


def _same_device(q, *named):
    for t, name in named:
        if t.device != q.device:
            raise ValueError("%s is on %s, q on %s" % (name, t.device, q.device))


def _fn(name, q):
    """The entry point for q's element type (the _f16 twin for float16)."""
    return getattr(load(), name + ("_f16" if q.dtype == _torch().float16 else ""))


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _scale(scale, D):
    return 1.0 / math.sqrt(D) if scale is None else float(scale)


def fa_fwd(q, k, v, softmax_scale=None, causal=False, out=None, lse=None,
           return_lse=True, stream=None, dropout_p=0.0, seed=0, offset=0):
    """Forward pass.  q, k, v: bf16 or fp16 [B, H, N, D] on the GPU.

    Returns (o, lse): o [B, H, N, D] in q's type and lse fp32 [B, H, N]
    (natural-log row log-sum-exp of the scaled scores), or (o, None) with
    ``return_lse=False``.  ``softmax_scale`` defaults to 1/sqrt(D).  With
    ``dropout_p`` > 0 the weights are dropped by fa_fwd_dropout's rule, the
    decisions fixed by (``seed``, ``offset``): pass the same to fa_bwd.
    """
    torch = _torch()
    _check(q, "q")
    B, H, N, D = q.shape
    _check(k, "k", q.shape, q.dtype)
    _check(v, "v", q.shape, q.dtype)
    o = torch.empty_like(q) if out is None else out
    _check(o, "out", q.shape, q.dtype)
    _same_device(q, (k, "k"), (v, "v"), (o, "out"))
    if lse is None and return_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_lse(lse, (B, H, N), q.device)
    if dropout_p:
        rc = _fn("fa_fwd_dropout", q)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N,
                                      D, _scale(softmax_scale, D), int(bool(causal)),
                                      float(dropout_p), int(seed), int(offset),
                                      _stream(stream))
    else:
        rc = _fn("fa_fwd", q)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, D,
                              _scale(softmax_scale, D), int(bool(causal)), _stream(stream))
    if rc != 0:
        raise FaError(rc, "fa_fwd")
    return o, lse


def fa_fwd_qk(q, k, v, softmax_scale=None, causal=False, out=None, lse=None,
              return_lse=True, stream=None):
    """Forward pass with Nq queries against Nk keys.  q: bf16 [B, H, Nq, D];
    k, v: bf16 [B, H, Nk, D].  Under ``causal`` query i reads keys
    j <= i + Nk - Nq (the queries are the last Nq positions).

    Returns (o [B, H, Nq, D] bf16, lse [B, H, Nq] fp32 or None).
    """
    torch = _torch()
    _check(q, "q")
    B, H, Nq, D = q.shape
    if k.dim() != 4:
        raise ValueError("k must be [B, H, Nk, D]")
    Nk = k.shape[2]
    _check(k, "k", (B, H, Nk, D), q.dtype)
    _check(v, "v", (B, H, Nk, D), q.dtype)
    o = torch.empty_like(q) if out is None else out
    _check(o, "out", q.shape, q.dtype)
    _same_device(q, (k, "k"), (v, "v"), (o, "out"))
    if lse is None and return_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check_lse(lse, (B, H, Nq), q.device)
    rc = _fn("fa_fwd_qk", q)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk,
                          D, _scale(softmax_scale, D), int(bool(causal)), _stream(stream))
    if rc != 0:
        raise FaError(rc, "fa_fwd_qk")
    return o, lse


def fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, D, num_splits=0) -> int:
    return int(load().fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, D, num_splits))


def fa_fwd_splitkv(q, k, v, softmax_scale=None, causal=False, num_splits=0, out=None,
                   lse=None, return_lse=True, workspace=None, stream=None):
    """Decoding-shaped forward: q bf16 [B, H, Nq, D] against k, v bf16
    [B, H, Nk, D], keys split across workgroups (``num_splits`` 0 = automatic)
    and merged exactly.  Same result as fa_fwd_qk up to rounding.  A
    workspace (uint8 GPU tensor) is allocated when not given.

    Returns (o [B, H, Nq, D] bf16, lse [B, H, Nq] fp32 or None).
    """
    torch = _torch()
    _check(q, "q")
    B, H, Nq, D = q.shape
    if k.dim() != 4:
        raise ValueError("k must be [B, H, Nk, D]")
    Nk = k.shape[2]
    _check(k, "k", (B, H, Nk, D), q.dtype)
    _check(v, "v", (B, H, Nk, D), q.dtype)
    o = torch.empty_like(q) if out is None else out
    _check(o, "out", q.shape, q.dtype)
    _same_device(q, (k, "k"), (v, "v"), (o, "out"))
    if lse is None and return_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check_lse(lse, (B, H, Nq), q.device)
    need = fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, D, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = _fn("fa_fwd_splitkv", q)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                               _ptr(workspace), ws_bytes, B, H, Nq, Nk, D,
                               _scale(softmax_scale, D), int(bool(causal)), int(num_splits),
                               _stream(stream))
    if rc != 0:
        raise FaError(rc, "fa_fwd_splitkv")
    return o, lse


def fa_fwd_varlen(q, k, v, cu_seqlens, max_seqlen, softmax_scale=None,
                  causal=False, out=None, lse=None, return_lse=True, stream=None,
                  dropout_p=0.0, seed=0, offset=0):
    """Packed forward.  q, k, v: bf16 [H, total, D]; cu_seqlens: int32 GPU
    tensor [nseq + 1]; max_seqlen: host int >= the longest sequence.  With
    ``dropout_p`` > 0 the weights are dropped by fa_fwd_varlen_dropout's rule
    (pass the same ``seed`` and ``offset`` to fa_bwd_varlen).

    Returns (o [H, total, D] bf16, lse [H, total] fp32 or None).
    """
    torch = _torch()
    _check(q, "q")
    H, total, D = q.shape
    _check(k, "k", q.shape, q.dtype)
    _check(v, "v", q.shape, q.dtype)
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be a 1-D int32 GPU tensor")
    if not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be contiguous")
    nseq = cu_seqlens.shape[0] - 1
    o = torch.empty_like(q) if out is None else out
    _check(o, "out", q.shape, q.dtype)
    _same_device(q, (k, "k"), (v, "v"), (o, "out"), (cu_seqlens, "cu_seqlens"))
    if lse is None and return_lse:
        lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
    _check_lse(lse, (H, total), q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens), nseq, total,
            int(max_seqlen), H, D, _scale(softmax_scale, D), int(bool(causal)))
    if dropout_p:
        rc = _fn("fa_fwd_varlen_dropout", q)(*args, float(dropout_p), int(seed), int(offset),
                                             _stream(stream))
    else:
        rc = _fn("fa_fwd_varlen", q)(*args, _stream(stream))
    if rc != 0:
        raise FaError(rc, "fa_fwd_varlen")
    return o, lse


def fa_bwd(q, k, v, o, lse, dout, softmax_scale=None, causal=False, dq=None,
           dk=None, dv=None, workspace=None, stream=None, dropout_p=0.0, seed=0, offset=0):
    """Backward pass.  o and lse must come from fa_fwd on the same inputs (and
    the same ``dropout_p``, ``seed`` and ``offset``, whose decisions are
    replayed).

    Returns (dq, dk, dv) [B, H, N, D] in q's element type.  ``workspace`` (uint8 GPU tensor
    of at least fa_bwd_workspace_size bytes) is allocated when not given.
    """
    torch = _torch()
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _check(t, name, q.shape, q.dtype)
    B, H, N, D = q.shape
    if lse is None:
        raise ValueError("lse from fa_fwd is required")
    _check_lse(lse, (B, H, N), q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check(t, name, q.shape, q.dtype)
    _same_device(q, (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"), (dk, "dk"),
                 (dv, "dv"))
    ws_bytes = fa_bwd_workspace_size(B, H, N, D)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, q.device)
    if dropout_p:
        rc = _fn("fa_bwd_dropout", q)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                      _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                      _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), B, H,
                                      N, D,
                                      _scale(softmax_scale, D), int(bool(causal)),
                                      float(dropout_p), int(seed), int(offset),
                                      _stream(stream))
    else:
        rc = _fn("fa_bwd", q)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                              _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), B, H, N, D,
                              _scale(softmax_scale, D), int(bool(causal)), _stream(stream))
    if rc != 0:
        raise FaError(rc, "fa_bwd")
    return dq, dk, dv


def fa_bwd_noalloc(q, k, v, o, lse, dout, softmax_scale=None, causal=False, dq=None,
                   dk=None, dv=None, stream=None):
    """fa_bwd without a workspace: the library's static device scratch holds
    it (bf16 only; B * H * N <= 2**21 rows).  With dq, dk and dv given the
    call allocates nothing; calls that overlap on one GPU race.

    Returns (dq, dk, dv) [B, H, N, D] bf16.
    """
    torch = _torch()
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _check(t, name, q.shape, q.dtype)
    B, H, N, D = q.shape
    if lse is None:
        raise ValueError("lse from fa_fwd is required")
    _check_lse(lse, (B, H, N), q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check(t, name, q.shape, q.dtype)
    _same_device(q, (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"), (dk, "dk"),
                 (dv, "dv"))
    if q.dtype != torch.bfloat16:
        raise ValueError("fa_bwd_noalloc takes bfloat16 tensors")
    rc = load().fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                               _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, D,
                               _scale(softmax_scale, D), int(bool(causal)), _stream(stream))
    if rc != 0:
        raise FaError(rc, "fa_bwd_noalloc")
    return dq, dk, dv


def fa_bwd_varlen(q, k, v, o, lse, dout, cu_seqlens, max_seqlen, softmax_scale=None,
                  causal=False, dq=None, dk=None, dv=None, workspace=None, stream=None,
                  dropout_p=0.0, seed=0, offset=0):
    """Backward pass of fa_fwd_varlen.  q, k, v, o, dout: bf16 or fp16
    [H, total, D]; lse: fp32 [H, total] from fa_fwd_varlen on the same
    inputs; cu_seqlens: int32 GPU tensor [nseq + 1]; max_seqlen: host int >=
    the longest sequence.

    Returns (dq, dk, dv) [H, total, D] in q's element type.  ``workspace``
    (GPU tensor of at least fa_bwd_workspace_size(1, H, total, D) bytes) is
    allocated when not given.  ``dropout_p``, ``seed`` and ``offset`` must be
    those of the forward pass, whose decisions are replayed.
    """
    torch = _torch()
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _check(t, name, q.shape, q.dtype)
    H, total, D = q.shape
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be a 1-D int32 GPU tensor")
    if not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be contiguous")
    nseq = cu_seqlens.shape[0] - 1
    if lse is None:
        raise ValueError("lse from fa_fwd_varlen is required")
    _check_lse(lse, (H, total), q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check(t, name, q.shape, q.dtype)
    _same_device(q, (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"), (dk, "dk"),
                 (dv, "dv"), (cu_seqlens, "cu_seqlens"))
    ws_bytes = fa_bwd_workspace_size(1, H, total, D)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
            _ptr(dv), _ptr(cu_seqlens), nseq, total, int(max_seqlen), _ptr(workspace),
            workspace.numel() * workspace.element_size(), H, D, _scale(softmax_scale, D),
            int(bool(causal)))
    if dropout_p:
        rc = _fn("fa_bwd_varlen_dropout", q)(*args, float(dropout_p), int(seed), int(offset),
                                             _stream(stream))
    else:
        rc = _fn("fa_bwd_varlen", q)(*args, _stream(stream))
    if rc != 0:
        raise FaError(rc, "fa_bwd_varlen")
    return dq, dk, dv
