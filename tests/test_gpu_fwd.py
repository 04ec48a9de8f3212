"""GPU parity of the dense forward pass (fa_fwd) against the fp64 oracle."""
import pytest
import torch

import attn_inputs as ai
import oracle
from _parity import check_fwd, oracle_rows_dense, say

pytestmark = pytest.mark.gpu


def _run(fa, q, k, v, scale, causal):
    o, lse = fa.fa_fwd(q.cuda(), k.cuda(), v.cuda(), softmax_scale=scale,
                       causal=causal)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def test_tiny_and_stability_variant(gpu):
    """B1 H1 N128 D64, non-causal, scale 1/8; then Q*8 (raw scores > 100)."""
    q, k, v, q8 = ai.tiny_inputs()
    scale = ai.TINY.scale
    for name, qq in (("tiny", q), ("tiny Q*8", q8)):
        say("case", name)
        o, lse = _run(gpu, qq, k, v, scale, False)
        o_ref, l_ref = oracle.fwd(qq, k, v, scale, False)
        check_fwd(o, lse, o_ref, l_ref, name)


@pytest.mark.parametrize("causal", [False, True])
def test_scores_in_the_thousands(gpu, causal):
    """Q*32 (exact in bf16): raw scores of several hundred to a thousand, so
    the running maximum moves by far more than the lazy bound over and over
    and the weights are nearly one-hot; every element against the oracle.
    O is then close to single V rows, so V is halved (also exact) to keep
    |O| below 4, where rounding O to bf16 alone stays within 2^-7."""
    B, H, N, D = 1, 2, 777, 128
    q, k, v = ai.qkv(B, H, N, D, seed=31)
    q32 = (q.float() * 32).to(torch.bfloat16)
    vh = (v.float() * 0.5).to(torch.bfloat16)
    assert torch.equal(q32.float(), q.float() * 32) and torch.equal(vh.float(), v.float() * 0.5)
    scale = ai.default_scale(D)
    say("case Q*32 causal", causal)
    o, lse = _run(gpu, q32, k, vh, scale, causal)
    o_ref, l_ref = oracle.fwd(q32, k, vh, scale, causal)
    check_fwd(o, lse, o_ref, l_ref, "Q*32")


SHAPES = [  # (B, H, N, D): single rows, ragged tails, several tiles
    (1, 1, 1, 64), (1, 2, 1, 128), (2, 1, 63, 64), (1, 3, 64, 128),
    (1, 1, 127, 128), (2, 2, 129, 64), (1, 2, 200, 128), (2, 3, 300, 128),
    (1, 1, 513, 64), (1, 2, 1000, 128),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dH%dN%dD%d" % s)
def test_shapes_full_oracle(gpu, shape, causal):
    B, H, N, D = shape
    say("case", shape, "causal", causal)
    q, k, v = ai.qkv(B, H, N, D, seed=100 + N + D)
    scale = ai.default_scale(D)
    o, lse = _run(gpu, q, k, v, scale, causal)
    o_ref, l_ref = oracle.fwd(q, k, v, scale, causal)
    check_fwd(o, lse, o_ref, l_ref, str(shape))


def test_causal_row0_reads_only_key0(gpu):
    """Row 0 has a single allowed key: its weight is exactly 1, so O_0 = v_0
    bit for bit, and L_0 = the scaled score s_00."""
    B, H, N, D = 2, 4, 300, 128
    q, k, v = ai.qkv(B, H, N, D, seed=7)
    scale = ai.default_scale(D)
    o, lse = _run(gpu, q, k, v, scale, True)
    assert torch.equal(o[:, :, 0], v[:, :, 0])
    s00 = scale * (q[:, :, 0].double() * k[:, :, 0].double()).sum(-1)
    assert (lse[:, :, 0].double() - s00).abs().max() < 1e-4


def test_deterministic_and_fully_written(gpu):
    """Two runs agree bit for bit (no races); NaN-filled outputs are fully
    overwritten; lse may be omitted."""
    B, H, N, D = 2, 3, 777, 128
    q, k, v = (x.cuda() for x in ai.qkv(B, H, N, D, seed=8))
    for causal in (False, True):
        o1 = torch.full_like(q, float("nan"))
        l1 = torch.full((B, H, N), float("nan"), device="cuda")
        gpu.fa_fwd(q, k, v, causal=causal, out=o1, lse=l1)
        o2, l2 = gpu.fa_fwd(q, k, v, causal=causal)
        o3, none = gpu.fa_fwd(q, k, v, causal=causal, return_lse=False)
        torch.cuda.synchronize()
        assert none is None
        assert not torch.isnan(o1).any() and not torch.isnan(l1).any()
        assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(o1, o3)


def test_runs_on_a_side_stream(gpu):
    B, H, N, D = 1, 2, 256, 64
    q, k, v = (x.cuda() for x in ai.qkv(B, H, N, D, seed=9))
    ref, _ = gpu.fa_fwd(q, k, v, causal=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o, _ = gpu.fa_fwd(q, k, v, causal=True)
    s.synchronize()
    assert torch.equal(o, ref)


def test_causal_workload_full_oracle(gpu):
    """B4 H32 N4096 D128 causal (the benchmark's launch): every element of O
    and every row of L against the oracle, one batch index at a time (so the
    fp64 copies stay near 2 GB)."""
    w = ai.CAUSAL
    say("case", w.name)
    q, k, v = ai.qkv(w.B, w.H, w.N, w.D, w.seed)
    o, lse = _run(gpu, q, k, v, w.scale, True)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    for b in range(w.B):
        sl = slice(b, b + 1)
        o_ref, l_ref = oracle.fwd(q[sl], k[sl], v[sl], w.scale, True)
        check_fwd(o[sl], lse[sl], o_ref, l_ref, "%s b%d (all %d heads)" % (w.name, b, w.H))


def test_long_context_sampled(gpu):
    """B1 H32 N65536 D128 causal: 256 seeded (head, row) pairs against full
    oracle rows (the oracle never sees more than one head at a time)."""
    w = ai.LONG
    say("case", w.name)
    q, k, v = ai.qkv(w.B, w.H, w.N, w.D, w.seed, chunk_rows=1 << 20)
    o, lse = _run(gpu, q, k, v, w.scale, True)
    heads, rows = ai.sample_rows(ai.LONG_SAMPLE_SEED, w.H, w.N, 256,
                                 extra=[(0, 0), (0, w.N - 1)])
    o_ref, l_ref = oracle_rows_dense(q, k, v, w.scale, True, heads, rows)
    check_fwd(o[0][heads, rows], lse[0][heads, rows], o_ref, l_ref, w.name)
