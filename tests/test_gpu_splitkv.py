"""GPU parity of the decoding-shaped forward (fa_fwd_splitkv: keys split
across workgroups, partials merged by log-sum-exp) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import attn_inputs as ai
import oracle
from _parity import check_fwd, f64, say

pytestmark = pytest.mark.gpu


def _inputs(B, H, Nq, Nk, D, seed):
    return (ai.randn_bf16((B, H, Nq, D), seed), ai.randn_bf16((B, H, Nk, D), seed + 1),
            ai.randn_bf16((B, H, Nk, D), seed + 2))


CASES = [  # (B, H, Nq, Nk, D, num_splits): single key, ragged ranges, many ranges
    (2, 2, 1, 1, 128, 0), (2, 3, 1, 64, 128, 0), (1, 2, 1, 65, 64, 2),
    (2, 2, 1, 1000, 128, 0), (1, 4, 1, 4097, 128, 7), (1, 2, 1, 4097, 64, 64),
    (2, 2, 4, 3000, 128, 0), (1, 2, 16, 2048, 64, 5), (1, 2, 130, 70, 128, 2),
    (1, 1, 200, 5000, 128, 0), (1, 2, 3, 640, 128, 1),
    # decoding kernel limits: 32 queries (largest) and 33 (forward tiles),
    # fewer keys than queries (dead rows under the causal mask), fewer
    # blocks than waves, a ragged range end with several ranges
    (1, 2, 32, 700, 128, 0), (1, 2, 33, 700, 128, 0), (1, 3, 16, 5, 64, 0),
    (2, 1, 2, 70, 128, 1), (2, 2, 7, 100, 128, 3),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%dNq%dNk%dD%ds%d" % c)
def test_cases_full_oracle(gpu, case, causal):
    B, H, Nq, Nk, D, ns = case
    say("case", case, "causal", causal)
    q, k, v = _inputs(B, H, Nq, Nk, D, 700 + Nq + Nk + D + ns)
    scale = ai.default_scale(D)
    o, lse = gpu.fa_fwd_splitkv(q.cuda(), k.cuda(), v.cuda(), softmax_scale=scale,
                                causal=causal, num_splits=ns)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.fwd_qk(q, k, v, scale, causal)
    og, lg = f64(o), f64(lse)
    dead = np.isneginf(l_ref)  # more queries than keys under the causal mask
    assert (og[dead] == 0).all() and np.isneginf(lg[dead]).all()
    check_fwd(og[~dead], lg[~dead], o_ref[~dead], l_ref[~dead], str(case))


def test_workspace_is_used_and_reused(gpu):
    """A caller-provided workspace of exactly the reported size; two calls in a
    row on different inputs give the same results as fresh calls."""
    B, H, Nq, Nk, D = 2, 4, 2, 3000, 128
    need = gpu.fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, D)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    outs = []
    for seed in (800, 810):
        q, k, v = (x.cuda() for x in _inputs(B, H, Nq, Nk, D, seed))
        a = gpu.fa_fwd_splitkv(q, k, v, causal=True, workspace=ws)
        b = gpu.fa_fwd_splitkv(q, k, v, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
        outs.append(a[0].clone())
    assert not torch.equal(outs[0], outs[1])


def test_decode_workload_full_oracle(gpu):
    """One new query per sequence against a 16384-token cache, B8 H32 D128."""
    B, H, Nq, Nk, D = 8, 32, 1, 16384, 128
    say("case decode", (B, H, Nq, Nk, D))
    q, k, v = _inputs(B, H, Nq, Nk, D, 900)
    scale = ai.default_scale(D)
    o, lse = gpu.fa_fwd_splitkv(q.cuda(), k.cuda(), v.cuda(), softmax_scale=scale,
                                causal=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.fwd_qk(q, k, v, scale, True)
    check_fwd(o, lse, o_ref, l_ref, "decode B8 H32 Nk16384")
