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


def test_noalloc_at_the_scratch_limit(gpu):
    """B2 H32 N32768 D128 causal: 2^21 query rows, the most the static array
    serves; bit for bit against fa_bwd (inputs drawn on the GPU)."""
    B, H, N, D = 2, 32, 32768, 128
    assert B * H * N == 1 << 21
    say("noalloc backward at the scratch limit", (B, H, N, D))
    q, k, v, do = (ai.randn_bf16_device((B, H, N, D), 6300 + i) for i in range(4))
    o, lse = gpu.fa_fwd(q, k, v, causal=True)
    ref = gpu.fa_bwd(q, k, v, o, lse, do, causal=True)
    got = gpu.fa_bwd_noalloc(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(g, r), name
    del q, k, v, do, o, lse, ref, got
    torch.cuda.empty_cache()
