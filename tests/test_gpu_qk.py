"""GPU parity of the forward pass with Nq queries against Nk keys (fa_fwd_qk,
bottom-right causal mask) against the fp64 oracle."""
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


def _run(fa, q, k, v, scale, causal):
    o, lse = fa.fa_fwd_qk(q.cuda(), k.cuda(), v.cuda(), softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


SHAPES = [  # (B, H, Nq, Nk, D): decode, short chunks, Nq > Nk, ragged tails
    (2, 2, 1, 1, 64), (2, 3, 1, 300, 128), (1, 2, 7, 129, 64), (2, 1, 128, 128, 128),
    (1, 2, 130, 70, 128), (2, 2, 200, 1000, 64), (1, 2, 64, 4100, 128),
    (1, 3, 257, 513, 128), (1, 1, 300, 37, 64),
    # Nk - Nq = 32m + 31: the first row of a pair's light tile (whose keys
    # the kernel walks downwards) has every allowed key in unmasked tiles
    (1, 2, 256, 607, 128), (1, 2, 640, 1311, 64),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dH%dNq%dNk%dD%d" % s)
def test_shapes_full_oracle(gpu, shape, causal):
    B, H, Nq, Nk, D = shape
    say("case", shape, "causal", causal)
    q, k, v = _inputs(B, H, Nq, Nk, D, 300 + Nq + Nk + D)
    scale = ai.default_scale(D)
    o, lse = _run(gpu, q, k, v, scale, causal)
    o_ref, l_ref = oracle.fwd_qk(q, k, v, scale, causal)
    dead = np.isneginf(l_ref)  # rows with no readable key (Nq > Nk, causal)
    assert dead.any() == (causal and Nq > Nk)
    lg = f64(lse)
    og = f64(o)
    assert (og[dead] == 0).all() and np.isneginf(lg[dead]).all()
    check_fwd(og[~dead], lg[~dead], o_ref[~dead], l_ref[~dead], str(shape))


@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_match_fa_fwd_bitwise(gpu, causal):
    q, k, v = ai.qkv(2, 3, 333, 128, seed=41)
    a = gpu.fa_fwd_qk(q.cuda(), k.cuda(), v.cuda(), causal=causal)
    b = gpu.fa_fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_chunked_prefill_sampled(gpu):
    """A 4096-query chunk against a 16384-key sequence (B1 H32 D128, causal):
    256 seeded (head, row) samples plus the first and last rows of head 0."""
    B, H, Nq, Nk, D = 1, 32, 4096, 16384, 128
    q, k, v = _inputs(B, H, Nq, Nk, D, 500)
    scale = ai.default_scale(D)
    say("case chunked prefill", (B, H, Nq, Nk, D))
    o, lse = _run(gpu, q, k, v, scale, True)
    heads, rows = (x.numpy() for x in ai.sample_rows(501, B * H, Nq, count=256,
                                                     extra=[(0, 0), (0, Nq - 1)]))
    o_ref = np.empty((len(heads), D))
    l_ref = np.empty(len(heads))
    qf, kf, vf = (x.reshape(B * H, -1, D) for x in (q, k, v))
    for head in np.unique(heads):
        sel = np.nonzero(heads == head)[0]
        oh, lh = oracle.fwd_qk_rows(qf[head][None, None], kf[head][None, None],
                                    vf[head][None, None], scale, True,
                                    np.zeros(len(sel), dtype=np.int64), rows[sel])
        o_ref[sel], l_ref[sel] = oh, lh
    og = f64(o).reshape(B * H, Nq, D)[heads, rows]
    lg = f64(lse).reshape(B * H, Nq)[heads, rows]
    check_fwd(og, lg, o_ref, l_ref, "chunked prefill sampled")
