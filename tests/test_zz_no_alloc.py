"""fa_bwd_noalloc, the backward entry point that allocates nothing, against
fa_bwd: bit for bit, on two calls in a row whose second input is smaller
(the static scratch keeps the first call's contents), each also against the
oracle's exact gradients."""
import pytest
import torch

import attn_inputs as ai
import oracle
from _parity import check_grad, say

pytestmark = pytest.mark.gpu


def test_noalloc_backward_matches_fa_bwd(gpu):
    cases = [((2, 4, 1000, 128), True, 6100), ((1, 2, 300, 64), False, 6200)]
    for (B, H, N, D), causal, seed in cases:
        say("noalloc backward", (B, H, N, D), "causal", causal)
        q, k, v, do = ai.backward_inputs(B, H, N, D, seed=seed)
        qc, kc, vc, doc = (x.cuda() for x in (q, k, v, do))
        o, lse = gpu.fa_fwd(qc, kc, vc, causal=causal)
        ref = gpu.fa_bwd(qc, kc, vc, o, lse, doc, causal=causal)
        outs = [torch.full_like(qc, float("nan")) for _ in range(3)]
        got = gpu.fa_bwd_noalloc(qc, kc, vc, o, lse, doc, causal=causal, dq=outs[0],
                                 dk=outs[1], dv=outs[2])
        torch.cuda.synchronize()
        for name, g, r in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(g, r), (name, (B, H, N, D), causal)
        exact = oracle.bwd(q, k, v, do, ai.default_scale(D), causal)
        for name, g, r in zip(("dq", "dk", "dv"), got, exact):
            check_grad(g, r, "noalloc %s %s" % (name, (B, H, N, D)))
