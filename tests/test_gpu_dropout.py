"""GPU parity of attention dropout (fa_fwd_dropout / fa_bwd_dropout) against
the fp64 oracle, including bit-exact recovery of the drop decisions in both
passes."""
import numpy as np
import pytest
import torch

import attn_inputs as ai
import oracle
from _parity import check_fwd, check_grad, dropout_scale, f64, say

pytestmark = pytest.mark.gpu


def _code_basis(N, D, dtype=torch.bfloat16):
    """Rows x_j = 2^(j // D) e_(j % D): a weighted sum over all rows j with
    weights w_j in {0, c} gives, in column d, c times the 4-bit code
    sum_t [w_(d + D t) != 0] 2^t (N = 4 D)."""
    x = torch.zeros(N, D, dtype=torch.float32)
    for j in range(N):
        x[j, j % D] = 2.0 ** (j // D)
    return x.to(dtype)


def _codes_from_mask(keep, D):
    """The same codes from a boolean [rows, N] mask."""
    n = keep.shape[1]
    return sum(keep[:, t * D:(t + 1) * D].astype(np.int64) << t for t in range(n // D))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p,seed,offset,D", [(0.25, 1, 0, 128), (0.5, 123456789012345, 7, 128),
                                             (0.1, 5, 4000000000, 128), (0.3, 77, 3, 64),
                                             (0.995, 2**64 - 1, 2**32 - 1, 128)])
def test_forward_mask_is_exact(gpu, causal, p, seed, offset, D):
    """q = 0 makes every weight 1/n_i; with v the code basis, O_i spells out
    row i's decisions, which must equal the oracle's bit for bit."""
    B, H, N = 1, 3, 4 * D
    say("dropout fwd mask", p, seed, offset, causal, D)
    q = torch.zeros(B, H, N, D, dtype=torch.bfloat16)
    k = ai.randn_bf16((B, H, N, D), 2000)
    v = _code_basis(N, D).expand(B, H, N, D).contiguous()
    o, _ = gpu.fa_fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, dropout_p=p,
                      seed=seed, offset=offset)
    torch.cuda.synchronize()
    T = oracle.dropout_threshold(p)
    inv = 256.0 / (256 - T)
    n_i = (np.arange(N) + 1) if causal else np.full(N, N)
    for h in range(H):
        codes = np.rint(f64(o[0, h]) * n_i[:, None] / inv).astype(np.int64)
        keep = oracle.dropout_mask(h, N, N, p, seed, offset)
        if causal:
            keep &= np.tril(np.ones((N, N), dtype=bool))
        assert np.array_equal(codes, _codes_from_mask(keep, D)), h


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [128, 64])
def test_backward_replays_the_mask_exactly(gpu, causal, D):
    """q = 0 again; dO the code basis: dV_j = sum_i P_ij Z_ij dO_i spells out
    column j of the mask as the dK/dV pass replays it."""
    B, H, N = 1, 2, 4 * D
    p, seed, offset = 0.3, 99, 12
    say("dropout bwd mask", causal, D)
    q = torch.zeros(B, H, N, D, dtype=torch.bfloat16).cuda()
    k = ai.randn_bf16((B, H, N, D), 2100).cuda()
    v = ai.randn_bf16((B, H, N, D), 2101).cuda()
    do = _code_basis(N, D).expand(B, H, N, D).contiguous().cuda()
    o, lse = gpu.fa_fwd(q, k, v, causal=causal, dropout_p=p, seed=seed, offset=offset)
    dq, dk, dv = gpu.fa_bwd(q, k, v, o, lse, do, causal=causal, dropout_p=p, seed=seed,
                            offset=offset)
    torch.cuda.synchronize()
    T = oracle.dropout_threshold(p)
    inv = 256.0 / (256 - T)
    for h in range(H):
        keep = oracle.dropout_mask(h, N, N, p, seed, offset)
        if causal:
            keep &= np.tril(np.ones((N, N), dtype=bool))
        # the weight of (i, j) is inv / n_i; element (j, d) of dV sums rows
        # i = d + D t (t = 0..3) with coefficients 2^t, so one flipped decision
        # there moves it by at least the smallest inv / n_i * 2^t among the
        # rows that may read key j
        n_i = (np.arange(N) + 1) if causal else np.full(N, N)
        want = (keep.T.astype(np.float64) * (inv / n_i)[None, :]) @ f64(do[0, h])
        got = f64(dv[0, h])
        rows = np.arange(D)[None, :] + D * np.arange(4)[:, None]          # [t, d]
        flip = inv / n_i[rows] * (2.0 ** np.arange(4))[:, None]           # [t, d]
        j = np.arange(N)[:, None, None]
        live = (rows[None] >= j) if causal else np.ones((N, 4, D), dtype=bool)
        min_flip = np.where(live, flip[None], np.inf).min(axis=1)        # [j, d]
        tol = np.where(np.isinf(min_flip), 1e-6, 0.5 * min_flip)
        # compare where a flip stands clear of bf16 rounding (all but a few
        # large early-row sums under causal masking)
        sharp = np.abs(want) * 2.0 ** -7 < tol
        assert sharp.mean() > 0.99, sharp.mean()
        assert (np.abs(got - want)[sharp] < tol[sharp]).all(), h


SHAPES = [(1, 2, 16, 64), (2, 1, 40, 128), (1, 2, 200, 128), (1, 1, 300, 64)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dH%dN%dD%d" % s)
def test_forward_backward_full_oracle(gpu, shape, causal):
    B, H, N, D = shape
    p, seed, offset = 0.2, 31337, N
    say("dropout", shape, causal)
    q, k, v, do = (ai.randn_bf16(shape, 2200 + N + i) for i in range(4))
    scale = ai.default_scale(D)
    qc, kc, vc, doc = (x.cuda() for x in (q, k, v, do))
    o, lse = gpu.fa_fwd(qc, kc, vc, softmax_scale=scale, causal=causal, dropout_p=p,
                        seed=seed, offset=offset)
    dq, dk, dv = gpu.fa_bwd(qc, kc, vc, o, lse, doc, softmax_scale=scale, causal=causal,
                            dropout_p=p, seed=seed, offset=offset)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.fwd_dropout(q, k, v, scale, causal, p, seed, offset)
    check_fwd(o, lse, o_ref, l_ref, "dropout " + str(shape), scale=dropout_scale(p))
    ref = oracle.bwd_dropout(q, k, v, do, scale, causal, p, seed, offset)
    for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        say("  %s rel-L2 whole %.3e, worst 64-row block %.3e"
            % (name, *check_grad(got, want, "dropout %s %s" % (shape, name))))


def test_f16_and_zero_probability(gpu):
    q, k, v = (ai.randn_f16((1, 2, 130, 128), 2300 + i).cuda() for i in range(3))
    o, lse = gpu.fa_fwd(q, k, v, causal=True, dropout_p=0.4, seed=3, offset=1)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.fwd_dropout(q, k, v, ai.default_scale(128), True, 0.4, 3, 1)
    check_fwd(o, lse, o_ref, l_ref, "f16 dropout", scale=dropout_scale(0.4))
    # a probability below 1/512 rounds to T = 0: plain attention, bit for bit
    a = gpu.fa_fwd(q, k, v, causal=True, dropout_p=1e-3, seed=3, offset=1)
    b = gpu.fa_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
