"""fp64 CPU attention oracle -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it, and it
imports nothing from the GPU package: the two share only the seeded input
generators (``attn_inputs``), which hold none of the method's arithmetic.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over rows); this
module builds it with gcc and marshals arrays.  Every function takes tensors or
arrays of any float dtype (bf16 widens to fp64 exactly) and returns float64
numpy arrays.

What it computes is the plain definition of softmax attention (scores, stable
softmax, weighted sum of values, L = m + ln l) and its exact gradient; the
sources on the FlashAttention pages are cited in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.POINTER(ctypes.c_int64)
_I32 = ctypes.POINTER(ctypes.c_int32)
_i64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
             "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"],
            check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_attn_fwd.argtypes = [_D, _D, _D, _D, _D, _i64, _i64, _i64,
                                    _i64, ctypes.c_double, ctypes.c_int]
    lib.oracle_attn_fwd_rows.argtypes = [_D, _D, _D, _I64, _I64, _i64, _D, _D,
                                         _i64, _i64, _i64, _i64,
                                         ctypes.c_double, ctypes.c_int]
    lib.oracle_attn_fwd_varlen.argtypes = [_D, _D, _D, _D, _D, _I32, _i64,
                                           _i64, _i64, _i64, ctypes.c_double,
                                           ctypes.c_int]
    lib.oracle_attn_fwd_varlen_rows.argtypes = [
        _D, _D, _D, _I32, _i64, _i64, _i64, _i64, ctypes.c_double,
        ctypes.c_int, _I64, _I64, _i64, _D, _D]
    lib.oracle_attn_fwd_qk.argtypes = [_D, _D, _D, _D, _D, _i64, _i64, _i64,
                                       _i64, _i64, ctypes.c_double, ctypes.c_int]
    lib.oracle_attn_fwd_qk_rows.argtypes = [_D, _D, _D, _I64, _I64, _i64, _D, _D,
                                            _i64, _i64, _i64, _i64, _i64,
                                            ctypes.c_double, ctypes.c_int]
    _u32p = ctypes.POINTER(ctypes.c_uint32)
    _u64 = ctypes.c_uint64
    lib.oracle_philox4x32_10.argtypes = [_u32p, _u32p, _u32p]
    lib.oracle_philox4x32_10.restype = None
    lib.oracle_dropout_threshold.argtypes = [ctypes.c_double]
    lib.oracle_dropout_threshold.restype = ctypes.c_int
    lib.oracle_dropout_mask.argtypes = [ctypes.POINTER(ctypes.c_uint8), _i64, _i64, _i64,
                                        ctypes.c_double, _u64, _u64]
    lib.oracle_attn_fwd_dropout.argtypes = [_D, _D, _D, _D, _D, _i64, _i64, _i64, _i64,
                                            ctypes.c_double, ctypes.c_int, ctypes.c_double,
                                            _u64, _u64]
    lib.oracle_attn_bwd_dropout.argtypes = [_D, _D, _D, _D, _D, _D, _D, _i64, _i64, _i64,
                                            _i64, ctypes.c_double, ctypes.c_int,
                                            ctypes.c_double, _u64, _u64]
    lib.oracle_attn_fwd_dropout_bh.argtypes = lib.oracle_attn_fwd_dropout.argtypes + [_i64]
    lib.oracle_attn_bwd_dropout_bh.argtypes = lib.oracle_attn_bwd_dropout.argtypes + [_i64]
    for f in (lib.oracle_dropout_mask, lib.oracle_attn_fwd_dropout,
              lib.oracle_attn_bwd_dropout, lib.oracle_attn_fwd_dropout_bh,
              lib.oracle_attn_bwd_dropout_bh):
        f.restype = ctypes.c_int
    lib.oracle_attn_bwd.argtypes = [_D, _D, _D, _D, _D, _D, _D, _i64, _i64,
                                    _i64, _i64, ctypes.c_double, ctypes.c_int]
    for f in (lib.oracle_attn_fwd, lib.oracle_attn_fwd_rows,
              lib.oracle_attn_fwd_qk, lib.oracle_attn_fwd_qk_rows,
              lib.oracle_attn_fwd_varlen, lib.oracle_attn_fwd_varlen_rows,
              lib.oracle_attn_bwd):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use (OMP_NUM_THREADS or all cores)."""
    return int(_load().oracle_num_threads())


def _f64(x) -> np.ndarray:
    """Any tensor/array -> C-contiguous float64 numpy (bf16 widens exactly)."""
    if hasattr(x, "detach"):  # torch tensor, possibly on a GPU
        import torch
        x = x.detach().to(device="cpu", dtype=torch.float64).contiguous().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _p(a: np.ndarray, t=_D):
    return a.ctypes.data_as(t)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError("oracle %s failed with code %d" % (what, rc))


def fwd(q, k, v, scale: float, causal: bool):
    """Dense forward.  q, k, v: [B, H, N, D].  Returns (O [B,H,N,D], L [B,H,N])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, D = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    o = np.empty_like(q)
    lse = np.empty((B, H, N), dtype=np.float64)
    _check(_load().oracle_attn_fwd(_p(q), _p(k), _p(v), _p(o), _p(lse), B, H,
                                   N, D, float(scale), int(bool(causal))),
           "fwd")
    return o, lse


def fwd_rows(q, k, v, scale: float, causal: bool, bh, rows):
    """Selected rows of the dense forward.

    bh[t] is the flattened head index b*H + h, rows[t] the query row.
    Returns (O_rows [n, D], L_rows [n]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, D = q.shape
    bh = np.ascontiguousarray(bh, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    n = bh.shape[0]
    o = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    _check(_load().oracle_attn_fwd_rows(_p(q), _p(k), _p(v), _p(bh, _I64),
                                        _p(rows, _I64), n, _p(o), _p(lse), B,
                                        H, N, D, float(scale),
                                        int(bool(causal))), "fwd_rows")
    return o, lse


def fwd_qk(q, k, v, scale: float, causal: bool):
    """Nq queries against Nk keys.  q: [B, H, Nq, D]; k, v: [B, H, Nk, D].

    Under the causal mask query i reads keys j <= i + Nk - Nq (bottom-right
    alignment).  Returns (O [B,H,Nq,D], L [B,H,Nq]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    assert k.shape == (B, H, Nk, D) and v.shape == k.shape
    o = np.empty_like(q)
    lse = np.empty((B, H, Nq), dtype=np.float64)
    _check(_load().oracle_attn_fwd_qk(_p(q), _p(k), _p(v), _p(o), _p(lse), B, H,
                                      Nq, Nk, D, float(scale), int(bool(causal))),
           "fwd_qk")
    return o, lse


def fwd_qk_rows(q, k, v, scale: float, causal: bool, bh, rows):
    """Selected rows of fwd_qk (bh[t] = b*H + h, rows[t] the query row)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    bh = np.ascontiguousarray(bh, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    n = bh.shape[0]
    o = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    _check(_load().oracle_attn_fwd_qk_rows(_p(q), _p(k), _p(v), _p(bh, _I64),
                                           _p(rows, _I64), n, _p(o), _p(lse), B, H,
                                           Nq, Nk, D, float(scale), int(bool(causal))),
           "fwd_qk_rows")
    return o, lse


def fwd_varlen(q, k, v, cu_seqlens, scale: float, causal: bool):
    """Packed forward.  q, k, v: [H, total, D]; cu_seqlens int [nseq+1].

    Returns (O [H, total, D], L [H, total]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    H, total, D = q.shape
    cu = np.ascontiguousarray(_i32(cu_seqlens))
    o = np.empty_like(q)
    lse = np.empty((H, total), dtype=np.float64)
    _check(_load().oracle_attn_fwd_varlen(_p(q), _p(k), _p(v), _p(o), _p(lse),
                                          _p(cu, _I32), cu.shape[0] - 1, H,
                                          total, D, float(scale),
                                          int(bool(causal))), "fwd_varlen")
    return o, lse


def fwd_varlen_rows(q, k, v, cu_seqlens, scale: float, causal: bool, heads,
                    tokens):
    """Selected rows of the packed forward: (heads[t], packed token tokens[t])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    H, total, D = q.shape
    cu = np.ascontiguousarray(_i32(cu_seqlens))
    heads = np.ascontiguousarray(heads, dtype=np.int64)
    tokens = np.ascontiguousarray(tokens, dtype=np.int64)
    n = heads.shape[0]
    o = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    _check(_load().oracle_attn_fwd_varlen_rows(
        _p(q), _p(k), _p(v), _p(cu, _I32), cu.shape[0] - 1, H, total, D,
        float(scale), int(bool(causal)), _p(heads, _I64), _p(tokens, _I64), n,
        _p(o), _p(lse)), "fwd_varlen_rows")
    return o, lse


def bwd(q, k, v, dout, scale: float, causal: bool):
    """Dense backward: gradients of <dout, O> w.r.t. q, k, v ([B,H,N,D] each)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, D = q.shape
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    _check(_load().oracle_attn_bwd(_p(q), _p(k), _p(v), _p(dout), _p(dq),
                                   _p(dk), _p(dv), B, H, N, D, float(scale),
                                   int(bool(causal))), "bwd")
    return dq, dk, dv


def bwd_varlen(q, k, v, dout, cu_seqlens, scale: float, causal: bool):
    """Packed backward: gradients of <dout, O> for the packed forward
    (``fwd_varlen``).  q, k, v, dout: [H, total, D]; cu_seqlens int [nseq+1].

    The packed forward applies the plain definition inside each segment
    [cu[b], cu[b+1]) and reads nothing outside it, so its Jacobian is block
    diagonal over the segments: each segment's gradients are the dense
    gradients (``bwd``) of that segment alone.  Tokens of no segment get
    zero gradients.  Returns (dQ, dK, dV), each [H, total, D].
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    H, total, D = q.shape
    cu = _i32(cu_seqlens)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(q), np.zeros_like(q)
    for b in range(cu.shape[0] - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        if e <= s:
            continue
        seg = [x[None, :, s:e] for x in (q, k, v, dout)]
        g = bwd(*seg, scale, causal)
        for out, gi in zip((dq, dk, dv), g):
            out[:, s:e] = gi[0]
    return dq, dk, dv


def _i32(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.asarray(x, dtype=np.int32)


# ---------------------------------------------------------------------------
# Dropout
# ---------------------------------------------------------------------------
def philox4x32_10(counter, key):
    """One Philox4x32-10 call: four uint32 counter words, two key words."""
    c = np.ascontiguousarray(counter, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.empty(4, dtype=np.uint32)
    u32 = ctypes.POINTER(ctypes.c_uint32)
    _load().oracle_philox4x32_10(c.ctypes.data_as(u32), k.ctypes.data_as(u32),
                                 out.ctypes.data_as(u32))
    return out


def dropout_threshold(p: float) -> int:
    """T with keep iff decision byte >= T (dropout probability T / 256)."""
    return int(_load().oracle_dropout_threshold(float(p)))


def dropout_mask(bh: int, nq: int, nk: int, p: float, seed: int, offset: int):
    """Keep mask (bool [nq, nk]) of flattened head bh."""
    keep = np.empty((nq, nk), dtype=np.uint8)
    _check(_load().oracle_dropout_mask(keep.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                                       bh, nq, nk, float(p), int(seed), int(offset)),
           "dropout_mask")
    return keep.astype(bool)


def fwd_dropout(q, k, v, scale: float, causal: bool, p: float, seed: int, offset: int):
    """Dense forward with attention dropout.  Returns (O, L)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, D = q.shape
    o = np.empty_like(q)
    lse = np.empty((B, H, N), dtype=np.float64)
    _check(_load().oracle_attn_fwd_dropout(_p(q), _p(k), _p(v), _p(o), _p(lse), B, H, N, D,
                                           float(scale), int(bool(causal)), float(p),
                                           int(seed), int(offset)), "fwd_dropout")
    return o, lse


def bwd_dropout(q, k, v, dout, scale: float, causal: bool, p: float, seed: int,
                offset: int):
    """Dense backward with attention dropout (same decisions as fwd_dropout)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, D = q.shape
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    _check(_load().oracle_attn_bwd_dropout(_p(q), _p(k), _p(v), _p(dout), _p(dq), _p(dk),
                                           _p(dv), B, H, N, D, float(scale),
                                           int(bool(causal)), float(p), int(seed),
                                           int(offset)), "bwd_dropout")
    return dq, dk, dv


def _segments(cu_seqlens):
    cu = _i32(cu_seqlens)
    return [(b, int(cu[b]), int(cu[b + 1])) for b in range(cu.shape[0] - 1)
            if int(cu[b + 1]) > int(cu[b])]


def fwd_varlen_dropout(q, k, v, cu_seqlens, scale: float, causal: bool, p: float, seed: int,
                       offset: int):
    """Packed forward with attention dropout.  q, k, v: [H, total, D].

    Each sequence b of each head h is the dense dropout forward (``fwd_dropout``'s
    arithmetic) of that segment alone, its decisions drawn as head b * H + h with
    positions counted from the sequence start.  Returns (O [H, total, D],
    L [H, total]); tokens of no sequence get O = 0, L = -inf.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    H, total, D = q.shape
    o = np.zeros_like(q)
    lse = np.full((H, total), -np.inf)
    for b, s, e in _segments(cu_seqlens):
        for h in range(H):
            qs, ks, vs = (np.ascontiguousarray(x[h, s:e]) for x in (q, k, v))
            os_ = np.empty_like(qs)
            ls = np.empty((e - s,), dtype=np.float64)
            _check(_load().oracle_attn_fwd_dropout_bh(
                _p(qs), _p(ks), _p(vs), _p(os_), _p(ls), 1, 1, e - s, D, float(scale),
                int(bool(causal)), float(p), int(seed), int(offset), b * H + h),
                "fwd_varlen_dropout")
            o[h, s:e], lse[h, s:e] = os_, ls
    return o, lse


def bwd_varlen_dropout(q, k, v, dout, cu_seqlens, scale: float, causal: bool, p: float,
                       seed: int, offset: int):
    """Packed backward with attention dropout, the same decisions as
    ``fwd_varlen_dropout``: per sequence and head, ``bwd_dropout``'s exact
    gradients of that segment alone.  Returns (dQ, dK, dV), each [H, total, D]."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    H, total, D = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(q), np.zeros_like(q)
    for b, s, e in _segments(cu_seqlens):
        for h in range(H):
            qs, ks, vs, ds = (np.ascontiguousarray(x[h, s:e]) for x in (q, k, v, dout))
            g = [np.empty_like(qs) for _ in range(3)]
            _check(_load().oracle_attn_bwd_dropout_bh(
                _p(qs), _p(ks), _p(vs), _p(ds), _p(g[0]), _p(g[1]), _p(g[2]), 1, 1, e - s,
                D, float(scale), int(bool(causal)), float(p), int(seed), int(offset),
                b * H + h), "bwd_varlen_dropout")
            dq[h, s:e], dk[h, s:e], dv[h, s:e] = g
    return dq, dk, dv
