"""GPU parity of the backward pass (fa_bwd) against the fp64 oracle gradients.

O and L come from the library's own forward pass, as the ABI requires."""
import pytest
import torch

import attn_inputs as ai
import oracle
from _parity import check_grad, say

pytestmark = pytest.mark.gpu


def _fwd_bwd(fa, q, k, v, do, scale, causal):
    qc, kc, vc, doc = (x.cuda() for x in (q, k, v, do))
    o, lse = fa.fa_fwd(qc, kc, vc, softmax_scale=scale, causal=causal)
    dq, dk, dv = fa.fa_bwd(qc, kc, vc, o, lse, doc, softmax_scale=scale,
                           causal=causal)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def _check(got, ref, what):
    """Whole-tensor and per-64-row-block relative L2 of dQ, dK and dV."""
    errs = [check_grad(g, r, "%s %s" % (what, name))
            for name, g, r in zip(("dQ", "dK", "dV"), got, ref)]
    say("  %s: rel-L2 (whole / worst 64-row block) dQ %.3e / %.3e  dK %.3e / %.3e"
        "  dV %.3e / %.3e" % (what, *[x for e in errs for x in e]))


# N = 300 and 960 at D = 128 leave an odd number of interior 64-query stages
# for some key tiles in both modes, so the dK/dV loop's one-stage remainder
# after its two-stage trips runs as well as the trips themselves
SHAPES = [(1, 1, 1, 64), (1, 2, 64, 128), (2, 1, 129, 64), (1, 2, 200, 128),
          (1, 1, 333, 64), (2, 2, 384, 128), (1, 2, 300, 128), (1, 1, 960, 128)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dH%dN%dD%d" % s)
def test_shapes_full_oracle(gpu, shape, causal):
    B, H, N, D = shape
    say("case bwd", shape, "causal", causal)
    q, k, v, do = ai.backward_inputs(B, H, N, D, seed=300 + N + D)
    scale = ai.default_scale(D)
    got = _fwd_bwd(gpu, q, k, v, do, scale, causal)
    ref = oracle.bwd(q, k, v, do, scale, causal)
    _check(got, ref, str(shape))


def test_deterministic(gpu):
    B, H, N, D = 1, 2, 500, 128
    q, k, v, do = ai.backward_inputs(B, H, N, D, seed=41)
    a = _fwd_bwd(gpu, q, k, v, do, ai.default_scale(D), True)
    b = _fwd_bwd(gpu, q, k, v, do, ai.default_scale(D), True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_workload_full_oracle(gpu):
    """B2 H32 N4096 D128 causal (the benchmark's launch): every one of the 64
    (batch, head) slices against the oracle's exact gradients, element by
    element, per slice and per 64-row block."""
    w = ai.BACKWARD
    say("case", w.name)
    q, k, v, do = ai.backward_inputs()
    got = _fwd_bwd(gpu, q, k, v, do, w.scale, True)
    for b in range(w.B):
        sl = slice(b, b + 1)
        ref = oracle.bwd(q[sl], k[sl], v[sl], do[sl], w.scale, True)
        _check([x[sl] for x in got], ref, "%s b%d (all %d heads)" % (w.name, b, w.H))


@pytest.mark.parametrize("causal", [False, True])
def test_long_backward_sampled_head(gpu, causal):
    """B1 H4 N8192 D128: many 64-query stages per key tile and 128-query
    tiles per unit; one seeded head against the oracle's exact gradients."""
    B, H, N, D = 1, 4, 8192, 128
    say("case long bwd B%d H%d N%d D%d causal %d" % (B, H, N, D, causal))
    q, k, v = ai.qkv(B, H, N, D, 70 + causal)
    do = ai.randn_bf16((B, H, N, D), 72 + causal)
    scale = ai.default_scale(D)
    got = _fwd_bwd(gpu, q, k, v, do, scale, causal)
    h = int(torch.randint(0, H, (1,), generator=ai.generator(73 + causal)))
    sl = (slice(0, 1), slice(h, h + 1))
    ref = oracle.bwd(q[sl], k[sl], v[sl], do[sl], scale, causal)
    _check([x[sl] for x in got], ref, "long bwd h%d causal %d" % (h, causal))
