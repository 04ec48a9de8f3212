"""GPU parity on seeded random shapes: every entry point against the fp64
oracle on sizes drawn from fixed seeds (odd lengths, ragged tiles,
single rows, empty varlen sequences, more queries than keys), so that cases
between the hand-picked ones are covered too."""
import numpy as np
import pytest
import torch

import attn_inputs as ai
import oracle
from _parity import check_fwd, check_grad, dropout_scale, f64, say

pytestmark = pytest.mark.gpu

def _cases(seed):
    """The three case lists drawn from one seeded generator."""
    rng = np.random.default_rng(seed)

    def draw(n, lo, hi):
        return [int(x) for x in rng.integers(lo, hi + 1, size=n)]

    # (B, H, N, D, causal) for the dense forward and backward
    dense = [(int(b), int(h), int(n), int(d), bool(c)) for b, h, n, d, c in zip(
        draw(12, 1, 2), draw(12, 1, 3), draw(12, 1, 700), rng.choice([64, 128], 12),
        rng.integers(0, 2, 12))]
    # (B, H, Nq, Nk, D, causal, num_splits) for the unequal-length and split
    # paths (half the query counts fall in the decoding kernel's range, at
    # most 32; some key counts are smaller than the query counts)
    qk = [(int(b), int(h), int(nq), int(nk), int(d), bool(c), int(s))
          for b, h, nq, nk, d, c, s in zip(
              draw(12, 1, 2), draw(12, 1, 2), draw(6, 1, 32) + draw(6, 33, 300),
              draw(4, 1, 1500) + draw(2, 1, 40) + draw(4, 1, 1500) + draw(2, 1, 40),
              rng.choice([64, 128], 12), rng.integers(0, 2, 12), draw(12, 0, 9))]
    # varlen: sequence lengths (zeros allowed), heads, width, causal
    varlen = [([int(x) for x in rng.integers(0, 400, size=int(ns))], int(h), int(d), bool(c))
              for ns, h, d, c in zip(draw(6, 1, 7), draw(6, 1, 3), rng.choice([64, 128], 6),
                                     rng.integers(0, 2, 6))]
    varlen[0] = ([0] + varlen[0][0] + [0], *varlen[0][1:])  # empty sequences at both ends
    return dense, qk, varlen


def _dropout_cases(seed):
    """Dropout cases from a generator of their own: (B, H, N, D, causal, p,
    seed, offset) dense and (lengths, H, D, causal, p, seed, offset) packed,
    with 64-bit seeds and offsets anywhere in [0, 2^32)."""
    rng = np.random.default_rng(seed)
    dense = [(int(rng.integers(1, 3)), int(rng.integers(1, 3)), int(rng.integers(1, 600)),
              int(rng.choice([64, 128])), bool(rng.integers(0, 2)),
              round(float(rng.uniform(0.05, 0.6)), 3), int(rng.integers(0, 2**63)),
              int(rng.integers(0, 2**32))) for _ in range(12)]
    packed = [([int(x) for x in rng.integers(0, 300, size=int(rng.integers(1, 6)))],
               int(rng.integers(1, 3)), int(rng.choice([64, 128])), bool(rng.integers(0, 2)),
               round(float(rng.uniform(0.05, 0.6)), 3), int(rng.integers(0, 2**63)),
               int(rng.integers(0, 2**32))) for _ in range(4)]
    return dense, packed


DENSE, QK, VARLEN, DENSE_BWD = [], [], [], []
for _seed in (20260, 777, 4242):
    _d, _q, _v = _cases(_seed)
    DENSE += _d
    QK += _q
    VARLEN += _v
    DENSE_BWD += _d[:8]
DROP_DENSE, DROP_PACKED = _dropout_cases(9090)


@pytest.mark.parametrize("case", DENSE, ids=lambda c: "B%dH%dN%dD%dc%d" % c)
def test_dense_forward(gpu, case):
    B, H, N, D, causal = case
    say("case", case)
    q, k, v = ai.qkv(B, H, N, D, 3000 + N)
    scale = ai.default_scale(D)
    o, lse = gpu.fa_fwd(q.cuda(), k.cuda(), v.cuda(), softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.fwd(q, k, v, scale, causal)
    check_fwd(o, lse, o_ref, l_ref, str(case))


@pytest.mark.parametrize("case", DENSE_BWD, ids=lambda c: "B%dH%dN%dD%dc%d" % c)
def test_dense_backward(gpu, case):
    B, H, N, D, causal = case
    say("case", case)
    q, k, v = ai.qkv(B, H, N, D, 4000 + N)
    do = ai.randn_bf16((B, H, N, D), 4100 + N)
    scale = ai.default_scale(D)
    qc, kc, vc, doc = (x.cuda() for x in (q, k, v, do))
    o, lse = gpu.fa_fwd(qc, kc, vc, softmax_scale=scale, causal=causal)
    grads = gpu.fa_bwd(qc, kc, vc, o, lse, doc, softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    refs = oracle.bwd(q, k, v, do, scale, causal)
    for name, g, r in zip(("dQ", "dK", "dV"), grads, refs):
        say("  %s rel-L2 whole %.3e, worst 64-row block %.3e"
            % (name, *check_grad(g, r, "%s %s" % (case, name))))


@pytest.mark.parametrize("case", QK, ids=lambda c: "B%dH%dNq%dNk%dD%dc%ds%d" % c)
def test_unequal_and_split(gpu, case):
    B, H, Nq, Nk, D, causal, ns = case
    say("case", case)
    q = ai.randn_bf16((B, H, Nq, D), 5000 + Nq)
    k = ai.randn_bf16((B, H, Nk, D), 5001 + Nk)
    v = ai.randn_bf16((B, H, Nk, D), 5002 + Nk)
    scale = ai.default_scale(D)
    o_ref, l_ref = oracle.fwd_qk(q, k, v, scale, causal)
    dead = np.isneginf(l_ref)  # queries before the first key (causal, Nq > Nk)
    for name, fn, kw in (("qk", gpu.fa_fwd_qk, {}),
                         ("splitkv", gpu.fa_fwd_splitkv, dict(num_splits=ns))):
        o, lse = fn(q.cuda(), k.cuda(), v.cuda(), softmax_scale=scale, causal=causal, **kw)
        torch.cuda.synchronize()
        og, lg = f64(o), f64(lse)
        assert (og[dead] == 0).all() and np.isneginf(lg[dead]).all(), (case, name)
        check_fwd(og[~dead], lg[~dead], o_ref[~dead], l_ref[~dead], "%s %s" % (name, case))


@pytest.mark.parametrize("case", VARLEN, ids=lambda c: "n%dH%dD%dc%d" % (len(c[0]), c[1], c[2], c[3]))
def test_varlen(gpu, case):
    lengths, H, D, causal = case
    say("case", case)
    total = sum(lengths)
    if total == 0:
        lengths = lengths[:-1] + [1]
        total = 1
    cu = ai.cu_seqlens(lengths)
    g = ai.generator(6000 + total)
    q, k, v = (ai.randn_bf16((H, total, D), g) for _ in range(3))
    scale = ai.default_scale(D)
    o, lse = gpu.fa_fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cu.cuda(), max(max(lengths), 1),
                               softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.fwd_varlen(q, k, v, cu, scale, causal)
    check_fwd(o, lse, o_ref, l_ref, str(case))


@pytest.mark.parametrize("case", DROP_DENSE, ids=lambda c: "B%dH%dN%dD%dc%d_p%s" % c[:6])
def test_dropout_forward_backward(gpu, case):
    B, H, N, D, causal, p, seed, offset = case
    say("case", case)
    q, k, v = ai.qkv(B, H, N, D, 7000 + N)
    do = ai.randn_bf16((B, H, N, D), 7100 + N)
    scale = ai.default_scale(D)
    qc, kc, vc, doc = (x.cuda() for x in (q, k, v, do))
    kw = dict(softmax_scale=scale, causal=causal, dropout_p=p, seed=seed, offset=offset)
    o, lse = gpu.fa_fwd(qc, kc, vc, **kw)
    grads = gpu.fa_bwd(qc, kc, vc, o, lse, doc, **kw)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.fwd_dropout(q, k, v, scale, causal, p, seed, offset)
    check_fwd(o, lse, o_ref, l_ref, str(case), scale=dropout_scale(p))
    refs = oracle.bwd_dropout(q, k, v, do, scale, causal, p, seed, offset)
    for name, g, r in zip(("dQ", "dK", "dV"), grads, refs):
        say("  %s rel-L2 whole %.3e, worst 64-row block %.3e"
            % (name, *check_grad(g, r, "%s %s" % (case, name))))


@pytest.mark.parametrize("case", DROP_PACKED,
                         ids=lambda c: "n%dH%dD%dc%d_p%s" % (len(c[0]), c[1], c[2], c[3], c[4]))
def test_dropout_packed_forward_backward(gpu, case):
    lengths, H, D, causal, p, seed, offset = case
    say("case", case)
    if sum(lengths) == 0:
        lengths = lengths[:-1] + [1]
    cu = ai.cu_seqlens(lengths)
    total = int(cu[-1])
    g = ai.generator(7200 + total)
    q, k, v, do = (ai.randn_bf16((H, total, D), g) for _ in range(4))
    scale = ai.default_scale(D)
    qc, kc, vc, doc, cuc = (x.cuda() for x in (q, k, v, do, cu))
    kw = dict(softmax_scale=scale, causal=causal, dropout_p=p, seed=seed, offset=offset)
    o, lse = gpu.fa_fwd_varlen(qc, kc, vc, cuc, max(lengths), **kw)
    grads = gpu.fa_bwd_varlen(qc, kc, vc, o, lse, doc, cuc, max(lengths), **kw)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.fwd_varlen_dropout(q, k, v, cu, scale, causal, p, seed, offset)
    check_fwd(o.cpu(), lse.cpu(), o_ref, l_ref, str(case), scale=dropout_scale(p))
    refs = oracle.bwd_varlen_dropout(q, k, v, do, cu, scale, causal, p, seed, offset)
    for name, got, want in zip(("dQ", "dK", "dV"), grads, refs):
        say("  %s rel-L2 whole %.3e, worst 64-row block %.3e"
            % (name, *check_grad(got.cpu(), want, "%s %s" % (case, name), cu=cu)))
