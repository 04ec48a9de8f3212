"""GPU parity of the packed variable-length backward pass (fa_bwd_varlen)."""
import pytest
import torch

import attn_inputs as ai
import oracle
from _parity import check_grad, say

pytestmark = pytest.mark.gpu

LENGTH_SETS = [
    [1],
    [5, 0, 17, 1],                 # an empty sequence in the middle
    [64, 128, 63, 65, 129, 1],     # tile-edge lengths
    [0, 300, 0, 257, 0],           # leading / trailing empties
    [1000, 37, 513],               # several 64-query stages per key tile
]


def _grads(fa, q, k, v, do, cu, max_seqlen, scale, causal):
    qc, kc, vc, doc, cuc = (x.cuda() for x in (q, k, v, do, cu))
    o, lse = fa.fa_fwd_varlen(qc, kc, vc, cuc, max_seqlen, softmax_scale=scale,
                              causal=causal)
    grads = fa.fa_bwd_varlen(qc, kc, vc, o, lse, doc, cuc, max_seqlen,
                             softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    return [g.cpu() for g in grads]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lengths", LENGTH_SETS, ids=lambda L: "x".join(map(str, L)))
def test_small_full_oracle(gpu, lengths, causal, D):
    H = 2
    say("case varlen bwd", lengths, "causal", causal, "D", D)
    cu = ai.cu_seqlens(lengths)
    total = int(cu[-1])
    g = ai.generator(600 + total + D)
    q, k, v, do = (ai.randn_bf16((H, total, D), g) for _ in range(4))
    scale = ai.default_scale(D)
    got = _grads(gpu, q, k, v, do, cu, max(lengths), scale, causal)
    refs = oracle.bwd_varlen(q, k, v, do, cu, scale, causal)
    for name, g_, r in zip(("dQ", "dK", "dV"), got, refs):
        say("  %s rel-L2 whole %.3e, worst 64-row block %.3e"
            % (name, *check_grad(g_, r, "%s %s %s" % (lengths, causal, name), cu=cu)))


def test_packed_equals_separate_runs_bitwise(gpu):
    """Each packed sequence gives bit-for-bit the dense backward of that
    sequence alone (tiles are aligned to each sequence's start)."""
    lengths = [300, 1, 129, 64, 700, 0]
    H, D = 2, 128
    cu = ai.cu_seqlens(lengths)
    total = int(cu[-1])
    g = ai.generator(37)
    q, k, v, do = (ai.randn_bf16((H, total, D), g) for _ in range(4))
    scale = ai.default_scale(D)
    for causal in (False, True):
        dq, dk, dv = _grads(gpu, q, k, v, do, cu, max(lengths), scale, causal)
        for b, n in enumerate(lengths):
            if n == 0:
                continue
            sl = slice(int(cu[b]), int(cu[b + 1]))
            seg = [x[None, :, sl].contiguous().cuda() for x in (q, k, v, do)]
            o, lse = gpu.fa_fwd(*seg[:3], softmax_scale=scale, causal=causal)
            gd = gpu.fa_bwd(*seg[:3], o, lse, seg[3], softmax_scale=scale, causal=causal)
            torch.cuda.synchronize()
            for name, packed, dense in zip(("dQ", "dK", "dV"), (dq, dk, dv), gd):
                assert torch.equal(packed[:, sl], dense[0].cpu()), (b, n, causal, name)


def test_fp16(gpu):
    lengths = [200, 0, 131]
    H, D = 2, 64
    cu = ai.cu_seqlens(lengths)
    total = int(cu[-1])
    g = ai.generator(38)
    q, k, v, do = (ai.randn_bf16((H, total, D), g).to(torch.float16) for _ in range(4))
    scale = ai.default_scale(D)
    got = _grads(gpu, q, k, v, do, cu, max(lengths), scale, True)
    assert all(x.dtype == torch.float16 for x in got)
    refs = oracle.bwd_varlen(q, k, v, do, cu, scale, True)
    for name, g_, r in zip(("dQ", "dK", "dV"), got, refs):
        say("  fp16 %s rel-L2 whole %.3e, worst 64-row block %.3e"
            % (name, *check_grad(g_, r, "fp16 " + name, cu=cu)))


def test_varlen_workload_full_size_sampled_heads(gpu):
    """16 sequences with lengths ~ U[128, 8192] (seeded), H32 D128, causal,
    all heads on the GPU; one seeded head against the oracle's exact
    gradients, every sequence of that head (about 10 s of fp64 work)."""
    q, k, v, cu, lengths = ai.varlen_inputs()
    H, total, D = q.shape
    say("case varlen bwd full size, total", total)
    do = ai.randn_bf16((H, total, D), ai.generator(ai.VARLEN_DATA_SEED + 100))
    scale = ai.default_scale(D)
    got = _grads(gpu, q, k, v, do, cu, max(lengths), scale, True)
    g = ai.generator(51)
    heads = [int(x) for x in torch.randperm(H, generator=g)[:1]]
    for h in heads:
        sl = slice(h, h + 1)
        refs = oracle.bwd_varlen(q[sl], k[sl], v[sl], do[sl], cu, scale, True)
        for name, g_, r in zip(("dQ", "dK", "dV"), got, refs):
            say("  head %d %s rel-L2 whole %.3e, worst 64-row block %.3e"
                % (h, name, *check_grad(g_[sl], r, "head %d %s" % (h, name), cu=cu)))
