"""GPU parity of the fp16 entry points (the *_f16 twins) against the fp64
oracle, on fp16 inputs and at the same tolerances as bf16."""
import numpy as np
import pytest
import torch

import attn_inputs as ai
import oracle
from _parity import check_fwd, check_grad, f64, say

pytestmark = pytest.mark.gpu


def _r(shape, seed):
    return ai.randn_f16(shape, seed)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 200, 128), (2, 2, 129, 64), (1, 1, 513, 64),
                                   (1, 3, 1000, 128)], ids=lambda s: "B%dH%dN%dD%d" % s)
def test_fwd(gpu, shape, causal):
    B, H, N, D = shape
    say("f16 fwd", shape, causal)
    q, k, v = (_r(shape, 1000 + N + D + i) for i in range(3))
    o, lse = gpu.fa_fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal)
    torch.cuda.synchronize()
    assert o.dtype == torch.float16
    o_ref, l_ref = oracle.fwd(q, k, v, ai.default_scale(D), causal)
    check_fwd(o, lse, o_ref, l_ref, "f16 " + str(shape))


def test_fwd_large_scores(gpu):
    """Q * 8 (exact in fp16): raw scores far beyond the range exp can take."""
    q, k, v = (_r((1, 2, 300, 64), 1100 + i) for i in range(3))
    q8 = q * 8
    o, lse = gpu.fa_fwd(q8.cuda(), k.cuda(), v.cuda(), causal=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.fwd(q8, k, v, ai.default_scale(64), True)
    check_fwd(o, lse, o_ref, l_ref, "f16 Q*8")


def test_varlen_qk_splitkv(gpu):
    H, D = 2, 128
    lengths = [1, 130, 77, 300]
    total = sum(lengths)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    q, k, v = (_r((H, total, D), 1200 + i) for i in range(3))
    o, lse = gpu.fa_fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cu.cuda(), max(lengths),
                               causal=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.fwd_varlen(q, k, v, cu, ai.default_scale(D), True)
    check_fwd(o, lse, o_ref, l_ref, "f16 varlen")
    q, k, v = _r((2, 2, 5, D), 1210), _r((2, 2, 3000, D), 1211), _r((2, 2, 3000, D), 1212)
    # fa_fwd_splitkv with 5 queries runs the decoding kernel: several ranges
    # (partials merged), one range (O and L written directly), automatic
    for fn, kw in ((gpu.fa_fwd_qk, {}), (gpu.fa_fwd_splitkv, dict(num_splits=5)),
                   (gpu.fa_fwd_splitkv, dict(num_splits=1)), (gpu.fa_fwd_splitkv, {})):
        o, lse = fn(q.cuda(), k.cuda(), v.cuda(), causal=True, **kw)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.fwd_qk(q, k, v, ai.default_scale(D), True)
        check_fwd(o, lse, o_ref, l_ref, "f16 " + fn.__name__)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 190, 128), (2, 1, 300, 64)],
                         ids=lambda s: "B%dH%dN%dD%d" % s)
def test_bwd(gpu, shape, causal):
    B, H, N, D = shape
    say("f16 bwd", shape, causal)
    q, k, v, do = (_r(shape, 1300 + N + i) for i in range(4))
    scale = ai.default_scale(D)
    qc, kc, vc, doc = (x.cuda() for x in (q, k, v, do))
    o, lse = gpu.fa_fwd(qc, kc, vc, softmax_scale=scale, causal=causal)
    dq, dk, dv = gpu.fa_bwd(qc, kc, vc, o, lse, doc, softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    assert dq.dtype == torch.float16
    ref = oracle.bwd(q, k, v, do, scale, causal)
    for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        say("  %s rel-L2 whole %.3e, worst 64-row block %.3e"
            % (name, *check_grad(got, want, "fp16 %s %s" % (shape, name))))


def test_mixed_dtypes_rejected(gpu):
    q = _r((1, 1, 16, 64), 1400).cuda()
    k = q.to(torch.bfloat16)
    with pytest.raises(TypeError):
        gpu.fa_fwd(q, k, q)
