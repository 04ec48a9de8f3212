"""GPU parity of attention dropout on packed sequences (fa_fwd_varlen_dropout,
fa_bwd_varlen_dropout): sequence b of head h draws its decisions as head
b * H + h, positions counted from the sequence start."""
import numpy as np
import pytest
import torch

import attn_inputs as ai
import oracle
from _parity import check_fwd, check_grad, dropout_scale, f64, say
from test_gpu_dropout import _code_basis, _codes_from_mask

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("causal", [False, True])
def test_packed_forward_mask_is_exact(gpu, causal):
    """q = 0 makes every weight 1/n_i; with each sequence's v the code basis,
    O_i spells out row i's decisions, which must equal the oracle's mask of
    head b * H + h bit for bit (lengths are multiples of D)."""
    lengths = [0, 256, 128, 0, 384]
    H, D = 2, 64
    p, seed, offset = 0.3, 99, 11
    cu = ai.cu_seqlens(lengths)
    total = int(cu[-1])
    say("packed dropout mask", lengths, causal)
    q = torch.zeros(H, total, D, dtype=torch.bfloat16)
    k = ai.randn_bf16((H, total, D), 2100)
    v = torch.zeros(H, total, D, dtype=torch.bfloat16)
    for b, n in enumerate(lengths):
        if n:
            v[:, int(cu[b]):int(cu[b + 1])] = _code_basis(n, D)
    o, _ = gpu.fa_fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cu.cuda(), max(lengths),
                             causal=causal, dropout_p=p, seed=seed, offset=offset)
    torch.cuda.synchronize()
    inv = 256.0 / (256 - oracle.dropout_threshold(p))
    for b, n in enumerate(lengths):
        if not n:
            continue
        s = int(cu[b])
        n_i = (np.arange(n) + 1) if causal else np.full(n, n)
        for h in range(H):
            codes = np.rint(f64(o[h, s:s + n]) * n_i[:, None] / inv).astype(np.int64)
            keep = oracle.dropout_mask(b * H + h, n, n, p, seed, offset)
            if causal:
                keep &= np.tril(np.ones((n, n), dtype=bool))
            assert np.array_equal(codes, _codes_from_mask(keep, D)), (b, h)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_packed_forward_backward_full_oracle(gpu, causal, D):
    lengths = [5, 0, 130, 64, 201]
    H, p, seed, offset = 2, 0.2, 424242, 3
    cu = ai.cu_seqlens(lengths)
    total = int(cu[-1])
    say("packed dropout", lengths, "causal", causal, "D", D)
    g = ai.generator(700 + D)
    q, k, v, do = (ai.randn_bf16((H, total, D), g) for _ in range(4))
    scale = ai.default_scale(D)
    qc, kc, vc, doc, cuc = (x.cuda() for x in (q, k, v, do, cu))
    o, lse = gpu.fa_fwd_varlen(qc, kc, vc, cuc, max(lengths), softmax_scale=scale,
                               causal=causal, dropout_p=p, seed=seed, offset=offset)
    grads = gpu.fa_bwd_varlen(qc, kc, vc, o, lse, doc, cuc, max(lengths), softmax_scale=scale,
                              causal=causal, dropout_p=p, seed=seed, offset=offset)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.fwd_varlen_dropout(q, k, v, cu, scale, causal, p, seed, offset)
    check_fwd(o.cpu(), lse.cpu(), o_ref, l_ref, "packed dropout %s" % lengths,
              scale=dropout_scale(p))
    refs = oracle.bwd_varlen_dropout(q, k, v, do, cu, scale, causal, p, seed, offset)
    for name, got, want in zip(("dQ", "dK", "dV"), grads, refs):
        say("  %s rel-L2 whole %.3e, worst 64-row block %.3e"
            % (name, *check_grad(got.cpu(), want, "packed dropout " + name, cu=cu)))


def test_packed_fp16_dropout(gpu):
    lengths = [70, 0, 129]
    H, D, p, seed, offset = 2, 128, 0.15, 8, 1
    cu = ai.cu_seqlens(lengths)
    total = int(cu[-1])
    g = ai.generator(710)
    q, k, v, do = (ai.randn_bf16((H, total, D), g).to(torch.float16) for _ in range(4))
    scale = ai.default_scale(D)
    qc, kc, vc, doc, cuc = (x.cuda() for x in (q, k, v, do, cu))
    o, lse = gpu.fa_fwd_varlen(qc, kc, vc, cuc, max(lengths), causal=True, dropout_p=p,
                               seed=seed, offset=offset)
    grads = gpu.fa_bwd_varlen(qc, kc, vc, o, lse, doc, cuc, max(lengths), causal=True,
                              dropout_p=p, seed=seed, offset=offset)
    torch.cuda.synchronize()
    assert o.dtype == torch.float16
    o_ref, l_ref = oracle.fwd_varlen_dropout(q, k, v, cu, scale, True, p, seed, offset)
    check_fwd(o.cpu(), lse.cpu(), o_ref, l_ref, "packed fp16 dropout", scale=dropout_scale(p))
    refs = oracle.bwd_varlen_dropout(q, k, v, do, cu, scale, True, p, seed, offset)
    for name, got, want in zip(("dQ", "dK", "dV"), grads, refs):
        check_grad(got.cpu(), want, "packed fp16 dropout " + name, cu=cu)
