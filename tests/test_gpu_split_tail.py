"""GPU parity of the dense causal forward when B*H is a multiple of 8.

Then the launch maps workgroups to heads XCD by XCD and issues the last heads
of each XCD as single query tiles, heaviest first, the rest as pairs of tiles
(one from each end of the causal triangle). These shapes cover both regimes:
every head split into single tiles, and pairs followed by a single-tile tail,
with even and odd tile counts and ragged last tiles. O and L are pre-filled
with NaN so that a tile no workgroup writes fails the finiteness check.
"""
import numpy as np
import pytest
import torch

import attn_inputs as ai
import oracle
from _parity import check_fwd, f64, say

pytestmark = pytest.mark.gpu


def _nan_out(B, H, N, D, dtype):
    o = torch.full((B, H, N, D), float("nan"), dtype=dtype, device="cuda")
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    return o, lse


def _tiles(N):
    return (N + 127) // 128


# (B, H, N, D). Heads per XCD hx = B*H/8; a head has ceil(tiles/2) pair units.
SHAPES = [
    (1, 8, 1, 64),        # one row per head
    (2, 4, 1000, 128),    # hx 1: all single tiles, 8 tiles
    (1, 8, 1100, 128),    # hx 1: 9 tiles (odd), ragged last tile
    (1, 16, 129, 64),     # hx 2: 2 tiles, the second one row
    (4, 8, 700, 64),      # hx 4: all heads as single tiles
    (8, 8, 2500, 128),    # hx 8, 20 tiles: 1 paired head + 7 tail heads per XCD
    (8, 8, 2500, 64),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dH%dN%dD%d" % s)
def test_dense_causal_full_oracle(gpu, shape):
    B, H, N, D = shape
    say("split tail", shape, "tiles", _tiles(N))
    q, k, v = ai.qkv(B, H, N, D, seed=4100 + N + D)
    scale = ai.default_scale(D)
    o, lse = _nan_out(B, H, N, D, torch.bfloat16)
    gpu.fa_fwd(q.cuda(), k.cuda(), v.cuda(), softmax_scale=scale, causal=True,
               out=o, lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.fwd(q, k, v, scale, True)
    check_fwd(o.cpu(), lse.cpu(), o_ref, l_ref, "split tail " + str(shape))


def test_f16_mixed_regime(gpu):
    B, H, N, D = 8, 8, 2500, 128
    say("split tail f16", (B, H, N, D))
    q, k, v = (ai.randn_f16((B, H, N, D), 4200 + i) for i in range(3))
    scale = ai.default_scale(D)
    o, lse = _nan_out(B, H, N, D, torch.float16)
    gpu.fa_fwd(q.cuda(), k.cuda(), v.cuda(), softmax_scale=scale, causal=True,
               out=o, lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.fwd(q, k, v, scale, True)
    check_fwd(o.cpu(), lse.cpu(), o_ref, l_ref, "split tail f16")


@pytest.mark.parametrize("Nq,Nk", [(600, 1000), (1000, 600), (300, 300)])
def test_unequal_lengths_bottom_right(gpu, Nq, Nk):
    """fa_fwd_qk with a causal mask takes the same launch; with Nq > Nk the
    first Nq - Nk query rows see no key."""
    B, H, D = 1, 8, 128
    say("split tail qk", Nq, Nk)
    q = ai.randn_bf16((B, H, Nq, D), 4300)
    k = ai.randn_bf16((B, H, Nk, D), 4301)
    v = ai.randn_bf16((B, H, Nk, D), 4302)
    scale = ai.default_scale(D)
    o, lse = _nan_out(B, H, Nq, D, torch.bfloat16)
    gpu.fa_fwd_qk(q.cuda(), k.cuda(), v.cuda(), softmax_scale=scale, causal=True,
                  out=o, lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.fwd_qk(q, k, v, scale, True)
    og, lg = f64(o), f64(lse)
    dead = np.isneginf(l_ref)  # rows with no readable key get O = 0, L = -inf
    assert dead.any() == (Nq > Nk)
    assert (og[dead] == 0).all() and np.isneginf(lg[dead]).all()
    check_fwd(og[~dead], lg[~dead], o_ref[~dead], l_ref[~dead],
              "split tail qk %d %d" % (Nq, Nk))


def test_dropout_same_mapping(gpu):
    """Dropout's generator is indexed by (head, row, key), not by workgroup,
    so the remapped launch must reproduce the oracle's mask exactly."""
    B, H, N, D = 2, 4, 900, 64
    p, seed, offset = 0.25, 777, 5
    say("split tail dropout", (B, H, N, D))
    q, k, v = ai.qkv(B, H, N, D, seed=4400)
    scale = ai.default_scale(D)
    o, lse = _nan_out(B, H, N, D, torch.bfloat16)
    gpu.fa_fwd(q.cuda(), k.cuda(), v.cuda(), softmax_scale=scale, causal=True,
               out=o, lse=lse, dropout_p=p, seed=seed, offset=offset)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.fwd_dropout(q, k, v, scale, True, p, seed, offset)
    check_fwd(o.cpu(), lse.cpu(), o_ref, l_ref, "split tail dropout")
