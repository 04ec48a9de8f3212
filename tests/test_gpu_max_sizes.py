"""Parity at the largest sizes the entry points accept.

Every kernel addresses one (batch, head) slice with 32-bit byte offsets, and
the entry points accept a slice of N rows while (N + 256) * D * 2 bytes stay
below 2 GiB.  These cases take the largest N accepted at D = 128 (8388351
rows: a ragged key count, and a packed token axis of that length), so byte
offsets inside a slice come within 64 KiB of 2^31, and tensors above 4 GiB
across slices (B8 H64 N32768 D128).  Inputs are drawn on the GPU from a
seeded generator; the slices that are checked are copied back, so the oracle
sees the same bits.  The dense backward at that size is compared bit for bit
with the same slice run alone (its result depends only on the slice's data),
the other cases against the oracle.
"""
import numpy as np
import pytest
import torch

import attn_inputs as ai
import oracle
from _parity import check_fwd, check_grad, f64, say

pytestmark = pytest.mark.gpu

D = 128
MAX_ROWS = (1 << 31) // (D * 2) - 257   # largest slice the entry points accept at D = 128


def _release():
    """Return the cached blocks of the test that just ran (several GiB)."""
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_keys_near_slice_limit(gpu):
    """Nq queries against the largest accepted key count (ragged): fa_fwd_qk
    (forward tiles), fa_fwd_splitkv with 40 queries (forward tiles over key
    ranges) and with one query (decoding kernel)."""
    Nq, Nk = 40, MAX_ROWS
    say("case keys near the slice limit", (Nq, Nk, D))
    q = ai.randn_bf16_device((1, 1, Nq, D), 7100)
    k = ai.randn_bf16_device((1, 1, Nk, D), 7101)
    v = ai.randn_bf16_device((1, 1, Nk, D), 7102)
    scale = ai.default_scale(D)
    rows = np.array([0, 1, 17, 31, 32, Nq - 1])
    o_ref, l_ref = oracle.fwd_qk_rows(q.cpu(), k.cpu(), v.cpu(), scale, True,
                                      np.zeros_like(rows), rows)
    o, lse = gpu.fa_fwd_qk(q, k, v, causal=True)
    check_fwd(o[0, 0, rows], lse[0, 0, rows], o_ref, l_ref, "fa_fwd_qk Nk %d" % Nk)
    o, lse = gpu.fa_fwd_splitkv(q, k, v, causal=True)
    check_fwd(o[0, 0, rows], lse[0, 0, rows], o_ref, l_ref, "fa_fwd_splitkv Nq 40")
    # one query at the last position: the last row of the 40-query case
    q1 = q[:, :, Nq - 1:].contiguous()
    o1, l1 = gpu.fa_fwd_splitkv(q1, k, v, causal=True)
    check_fwd(o1[0, 0], l1[0, 0], o_ref[-1:], l_ref[-1:], "fa_fwd_splitkv Nq 1")
    del q, k, v, o, lse, q1, o1, l1
    _release()


def test_dense_forward_beyond_4gib(gpu):
    """B8 H64 N32768 D128 causal: 4 GiB per tensor, so slice offsets pass
    2^32 bytes; sampled rows of the first, a middle and the last slice."""
    B, H, N = 8, 64, 32768
    say("case dense forward", (B, H, N, D))
    q, k, v = (ai.randn_bf16_device((B, H, N, D), 7200 + i) for i in range(3))
    o, lse = gpu.fa_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    scale = ai.default_scale(D)
    rows = np.array([0, 1, 127, 128, 4095, 16383, 16384, N - 2, N - 1])
    for b, h in ((0, 0), (3, 17), (B - 1, H - 1)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        o_ref, l_ref = oracle.fwd_rows(q[sl].cpu(), k[sl].cpu(), v[sl].cpu(), scale, True,
                                       np.zeros_like(rows), rows)
        check_fwd(o[b, h, rows], lse[b, h, rows], o_ref, l_ref, "slice (%d, %d)" % (b, h))
    del q, k, v, o, lse
    _release()


def test_varlen_near_slice_limit(gpu):
    """H2 packed axis of the largest accepted length: 32766 sequences of 256
    tokens and one of 255, causal, forward and backward; the first, a middle
    and the last two sequences of both heads against the oracle."""
    H = 2
    lengths = [256] * 32766 + [255]
    total = sum(lengths)
    assert total == MAX_ROWS
    say("case varlen near the slice limit", (H, total, D))
    cu = ai.cu_seqlens(lengths)
    cuc = cu.cuda()
    q, k, v, do = (ai.randn_bf16_device((H, total, D), 7300 + i) for i in range(4))
    o, lse = gpu.fa_fwd_varlen(q, k, v, cuc, 256, causal=True)
    dq, dk, dv = gpu.fa_bwd_varlen(q, k, v, o, lse, do, cuc, 256, causal=True)
    torch.cuda.synchronize()
    scale = ai.default_scale(D)
    c = [int(x) for x in cu]
    for i in (0, 16384, len(lengths) - 2, len(lengths) - 1):
        a, e = c[i], c[i + 1]
        for h in range(H):
            qs, ks, vs, dos = (t[h:h + 1, a:e].cpu()[None] for t in (q, k, v, do))
            o_ref, l_ref = oracle.fwd(qs, ks, vs, scale, True)
            check_fwd(o[h, a:e], lse[h, a:e], o_ref[0, 0], l_ref[0, 0],
                      "sequence %d head %d fwd" % (i, h))
            refs = oracle.bwd(qs, ks, vs, dos, scale, True)
            for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
                check_grad(g[h, a:e], r[0, 0], "sequence %d head %d %s" % (i, h, name))
    del q, k, v, do, o, lse, dq, dk, dv
    _release()


def test_dense_backward_beyond_4gib(gpu):
    """B8 H64 N32768 D128 causal backward (4 GiB per tensor): the first and
    the last slice equal, bit for bit, the same slice run alone."""
    B, H, N = 8, 64, 32768
    say("case dense backward", (B, H, N, D))
    q, k, v, do = (ai.randn_bf16_device((B, H, N, D), 7400 + i) for i in range(4))
    o, lse = gpu.fa_fwd(q, k, v, causal=True)
    dq, dk, dv = gpu.fa_bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (B - 1, H - 1)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        one = [t[sl].contiguous() for t in (q, k, v, o, lse, do)]
        g1 = gpu.fa_bwd(*one, causal=True)
        torch.cuda.synchronize()
        for name, big, small in zip(("dq", "dk", "dv"), (dq, dk, dv), g1):
            same = torch.equal(big[sl], small)
            say("  slice (%d, %d) %s bitwise equal: %s" % (b, h, name, same))
            assert same, (b, h, name)
        del one, g1
    del q, k, v, do, o, lse, dq, dk, dv
    _release()
