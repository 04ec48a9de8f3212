"""GPU parity of the packed variable-length forward pass (fa_fwd_varlen)."""
import pytest
import torch

import attn_inputs as ai
import oracle
from _parity import check_fwd, say

pytestmark = pytest.mark.gpu


def _run(fa, q, k, v, cu, max_seqlen, scale, causal):
    o, lse = fa.fa_fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cu.cuda(), max_seqlen,
                              softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


LENGTH_SETS = [
    [1],
    [5, 0, 17, 1],                 # an empty sequence in the middle
    [64, 128, 63, 65, 129, 1],     # tile-edge lengths
    [0, 300, 0, 257, 0],           # leading / trailing empties
    [1000, 37, 513],
]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lengths", LENGTH_SETS, ids=lambda L: "x".join(map(str, L)))
def test_small_full_oracle(gpu, lengths, causal, D):
    H = 3
    say("case varlen", lengths, "causal", causal, "D", D)
    cu = ai.cu_seqlens(lengths)
    total = int(cu[-1])
    g = ai.generator(200 + total + D)
    q, k, v = (ai.randn_bf16((H, total, D), g) for _ in range(3))
    scale = ai.default_scale(D)
    o, lse = _run(gpu, q, k, v, cu, max(lengths), scale, causal)
    o_ref, l_ref = oracle.fwd_varlen(q, k, v, cu, scale, causal)
    check_fwd(o, lse, o_ref, l_ref, "varlen %s" % lengths)


def test_packed_equals_separate_runs_bitwise(gpu):
    """Each packed sequence gives bit-for-bit the dense result on that
    sequence alone (tiles are aligned to each sequence's start)."""
    lengths = [300, 1, 129, 64, 700]
    H, D = 2, 128
    cu = ai.cu_seqlens(lengths)
    total = int(cu[-1])
    g = ai.generator(31)
    q, k, v = (ai.randn_bf16((H, total, D), g) for _ in range(3))
    for causal in (False, True):
        o, lse = _run(gpu, q, k, v, cu, max(lengths), ai.default_scale(D), causal)
        for b, n in enumerate(lengths):
            sl = slice(int(cu[b]), int(cu[b + 1]))
            od, ld = gpu.fa_fwd(q[None, :, sl].contiguous().cuda(),
                                k[None, :, sl].contiguous().cuda(),
                                v[None, :, sl].contiguous().cuda(),
                                softmax_scale=ai.default_scale(D), causal=causal)
            torch.cuda.synchronize()
            assert torch.equal(o[:, sl], od[0].cpu()), (b, n, causal)
            assert torch.equal(lse[:, sl], ld[0].cpu()), (b, n, causal)


def test_varlen_workload_full_oracle(gpu):
    """16 sequences with lengths ~ U[128, 8192] (seeded), H32 D128, causal:
    every element of O and every row of L against the oracle, eight heads at
    a time (about 2.9e12 fp64 flops in all)."""
    q, k, v, cu, lengths = ai.varlen_inputs()
    H, total, D = q.shape
    say("case", ai.VARLEN_NAME, "total", total)
    scale = ai.default_scale(D)
    o, lse = _run(gpu, q, k, v, cu, max(lengths), scale, True)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    for h0 in range(0, H, 8):
        sl = slice(h0, h0 + 8)
        o_ref, l_ref = oracle.fwd_varlen(q[sl], k[sl], v[sl], cu, scale, True)
        check_fwd(o[sl], lse[sl], o_ref, l_ref, "%s heads %d-%d" % (ai.VARLEN_NAME, h0, h0 + 7))
