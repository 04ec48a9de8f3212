"""Shared helpers for the GPU parity tests: tolerances, comparisons, and
oracle calls on sampled rows or heads (one (batch, head) slice at a time, so
the fp64 copies stay small even for the 65536-token workload)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

# Tolerances fixed for this path: O max-abs and mean-abs, L abs, and the
# relative L2 error of each gradient tensor.
O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
L_ABS = 1e-3
GRAD_REL_L2 = 1e-2


def say(*a):
    """Print and flush, so a GPU failure still shows which case was running."""
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def dropout_scale(p: float) -> float:
    """The factor 1 / (1 - p') that attention dropout puts on every kept
    weight (p' = T / 256, T the byte threshold of the generator rule)."""
    return 256.0 / (256 - oracle.dropout_threshold(p))


def check_fwd(o_gpu, lse_gpu, o_ref, lse_ref, what="", scale=1.0):
    """Element-wise comparison of O (bf16 GPU vs fp64 oracle) and L.

    The O bounds hold for attention outputs, weighted means of V rows.  Under
    dropout the kept weights carry the factor 1 / (1 - p') (tensortonic
    section 7), so O is that factor times such a mean and so are its bf16
    rounding and its error: pass ``scale`` = dropout_scale(p) and the O
    errors are measured in units of the undropped output (divided by it).
    L, the log-sum-exp of all allowed scores, does not depend on dropout."""
    o_gpu = f64(o_gpu) if isinstance(o_gpu, torch.Tensor) else o_gpu
    lse_gpu = f64(lse_gpu) if isinstance(lse_gpu, torch.Tensor) else lse_gpu
    assert np.isfinite(o_gpu).all(), what + ": non-finite O"
    assert np.isfinite(lse_gpu).all(), what + ": non-finite L"
    err = np.abs(o_gpu - o_ref) / scale
    lerr = np.abs(lse_gpu - lse_ref)
    stats = dict(o_max=float(err.max()), o_mean=float(err.mean()),
                 l_max=float(lerr.max()))
    say("  %s: O max %.3e mean %.3e | L max %.3e" % (what, stats["o_max"],
                                                     stats["o_mean"], stats["l_max"]))
    assert stats["o_max"] <= O_MAX_ABS, (what, stats)
    assert stats["o_mean"] <= O_MEAN_ABS, (what, stats)
    assert stats["l_max"] <= L_ABS, (what, stats)
    return stats


def rel_l2(got, ref) -> float:
    """Relative L2 error; where the exact gradient is identically zero (one
    key per row: every weight is 1 and the score gradient vanishes) it is the
    absolute L2 norm of the result instead."""
    got = f64(got) if isinstance(got, torch.Tensor) else got
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    return float(num / den) if den > 0 else float(num)


# Rows per block of the blockwise gradient check: the kernels' query stage
# and key-tile granularity, so one bad stage or ragged row cannot hide in the
# norm of a whole (batch, head) slice.
GRAD_BLOCK_ROWS = 64


def check_grad(got, ref, what="", cu=None, block_rows=GRAD_BLOCK_ROWS):
    """Relative L2 error of a gradient tensor, over the whole tensor and over
    every block of ``block_rows`` consecutive rows of each leading index
    (rows are the second-to-last axis).  With packed offsets ``cu`` the blocks
    start at each sequence's first row and stop at its end.  Each must be
    <= GRAD_REL_L2; returns (whole, worst block).

    A block's error is measured against the larger of its own reference norm
    and the norm that a block of its rows would have at the tensor's mean row
    norm.  A block far smaller than that is ill-conditioned: its gradient is
    the difference dP - D of nearly equal terms (one dominant weight), and D
    comes from the stored 16-bit O, whose rounding (relative 2^-9) is then
    magnified (seen: 1.5 % in a 2-token slice whose kept weight was 0.85).  A
    wrong stage still shows: its error is of the order of the gradient
    itself."""
    got = f64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), what + ": non-finite gradient"
    whole = rel_l2(got, ref)
    n, d = ref.shape[-2], ref.shape[-1]
    g2 = got.reshape(-1, n, d)
    r2 = ref.reshape(-1, n, d)
    if cu is None:
        segs = [(0, n)]
    else:
        c = [int(x) for x in cu]
        segs = [(a, b) for a, b in zip(c[:-1], c[1:]) if b > a]
    rows_total = sum(b - a for a, b in segs) * r2.shape[0]
    row_norm = float(np.sqrt(sum(float(np.sum(r2[:, a:b] ** 2)) for a, b in segs) /
                             max(rows_total, 1)))
    worst, at = 0.0, None
    for s in range(r2.shape[0]):
        for a, b in segs:
            for r0 in range(a, b, block_rows):
                r1 = min(b, r0 + block_rows)
                den = max(float(np.linalg.norm(r2[s, r0:r1])), row_norm * np.sqrt(r1 - r0))
                num = float(np.linalg.norm(g2[s, r0:r1] - r2[s, r0:r1]))
                e = num / den if den > 0 else num
                if e > worst:
                    worst, at = e, (s, r0)
    assert whole <= GRAD_REL_L2, (what, "whole", whole)
    assert worst <= GRAD_REL_L2, (what, "block (slice, row0)", at, worst)
    return whole, worst


def oracle_rows_dense(q, k, v, scale, causal, bh, rows):
    """Oracle O and L for flattened heads bh[t] = b*H + h and rows rows[t].

    q, k, v are CPU bf16 [B, H, N, D]; each needed (b, h) slice is widened to
    fp64 on its own.
    """
    B, H, N, D = q.shape
    bh = np.asarray(bh, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    o = np.empty((len(bh), D))
    lse = np.empty(len(bh))
    qf, kf, vf = (x.reshape(B * H, N, D) for x in (q, k, v))
    for head in np.unique(bh):
        sel = np.nonzero(bh == head)[0]
        oh, lh = oracle.fwd_rows(qf[head][None, None], kf[head][None, None],
                                 vf[head][None, None], scale, causal,
                                 np.zeros(len(sel), dtype=np.int64), rows[sel])
        o[sel], lse[sel] = oh, lh
    return o, lse


def oracle_rows_varlen(q, k, v, cu, scale, causal, heads, toks):
    """Oracle O and L for packed rows (heads[t], token toks[t]); q, k, v are
    CPU bf16 [H, total, D], widened one head at a time."""
    H, total, D = q.shape
    heads = np.asarray(heads, dtype=np.int64)
    toks = np.asarray(toks, dtype=np.int64)
    o = np.empty((len(heads), D))
    lse = np.empty(len(heads))
    for h in np.unique(heads):
        sel = np.nonzero(heads == h)[0]
        oh, lh = oracle.fwd_varlen_rows(q[h][None], k[h][None], v[h][None], cu,
                                        scale, causal,
                                        np.zeros(len(sel), dtype=np.int64),
                                        toks[sel])
        o[sel], lse[sel] = oh, lh
    return o, lse
