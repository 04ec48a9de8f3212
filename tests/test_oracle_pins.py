"""Pins for the fp64 oracle: checks against what the pages and mathematics fix.

Every check here is independent of the oracle's own code path: closed forms,
invariants the pages state, special cases that reduce to a library routine
(scipy's logsumexp, torch's CPU scaled_dot_product_attention and autograd),
central finite differences, and 50-digit mpmath on tiny inputs.
"""
import math
import os

import mpmath
import numpy as np
import pytest
import scipy.special
import torch

import attn_inputs
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split("=")
            out[key.strip()] = [float(x) for x in val.split()]
    return out


def _one_query(scores):
    """Inputs whose single query row has exactly the given scores (scale 1).

    D = len(scores); q = e0, k_j = scores[j] * e0, v_j = e_j, so O = P.
    """
    n = len(scores)
    q = np.zeros((1, 1, 1, n))
    q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, 1, n, n))
    k[0, 0, :, 0] = scores
    v = np.eye(n)[None, None]
    # the oracle's dense layout has equal Q and K lengths: pad Q with copies
    q = np.repeat(q, n, axis=2)
    return q, k, v


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# --------------------------------------------------------------------------
# P1: the split-tile example of tensortonic section 4.
# --------------------------------------------------------------------------
def test_split_tile_example_one_normalisation():
    g = _golden("split_tile_1234.txt")
    scores, t0, t1 = g["scores"], g["tile0"], g["tile1"]
    assert t0 + t1 == scores
    q, k, v = _one_query(scores)
    o, lse = oracle.fwd(q, k, v, scale=1.0, causal=False)
    p = o[0, 0, 0]
    mpmath.mp.dps = 40
    ex = [mpmath.e ** mpmath.mpf(s) for s in scores]
    tot = mpmath.fsum(ex)
    # closed form of softmax of [1, 2, 3, 4] and of its log-sum-exp
    for j in range(4):
        assert abs(p[j] - float(ex[j] / tot)) < 1e-15
    assert abs(lse[0, 0, 0] - float(mpmath.log(tot))) < 1e-14
    assert abs(p.sum() - 1.0) < 1e-15
    # the wrong per-tile softmax gives each tile a full unit of weight; the
    # correct weights give the tiles very different shares
    share0, share1 = p[:2].sum(), p[2:].sum()
    assert abs(share0 - float((ex[0] + ex[1]) / tot)) < 1e-15
    assert share0 < 0.2 and share1 > 0.8
    tile_local = np.concatenate([scipy.special.softmax(t0),
                                 scipy.special.softmax(t1)])
    assert abs(tile_local.sum() - 2.0) < 1e-15
    assert np.abs(tile_local - p).max() > 0.1
    assert np.abs(0.5 * tile_local - p).max() > 0.1  # averaging does not fix it


def test_split_tile_example_running_softmax_agrees():
    """The running-softmax rule (tensortonic section 5), applied tile by tile
    in 40-digit arithmetic, reaches the oracle's one-pass weights and L."""
    g = _golden("split_tile_1234.txt")
    q, k, v = _one_query(g["scores"])
    o, lse = oracle.fwd(q, k, v, scale=1.0, causal=False)
    mpmath.mp.dps = 40
    m, l, u = mpmath.mpf("-inf"), mpmath.mpf(0), [mpmath.mpf(0)] * 4
    for tile, cols in ((g["tile0"], (0, 1)), (g["tile1"], (2, 3))):
        m_new = max(m, max(mpmath.mpf(s) for s in tile))
        a = mpmath.e ** (m - m_new) if m != mpmath.mpf("-inf") else 0
        e = [mpmath.e ** (mpmath.mpf(s) - m_new) for s in tile]
        l = a * l + sum(e)
        u = [a * x for x in u]
        for c, w in zip(cols, e):
            u[c] += w  # value vectors are one-hot
        m = m_new
    for j in range(4):
        assert abs(o[0, 0, 0, j] - float(u[j] / l)) < 1e-15
    assert abs(lse[0, 0, 0] - float(m + mpmath.log(l))) < 1e-14
    # the per-tile log-sum-exps merge into the full one
    lse_t = [scipy.special.logsumexp(g["tile0"]),
             scipy.special.logsumexp(g["tile1"])]
    assert abs(np.logaddexp(*lse_t) - lse[0, 0, 0]) < 1e-14


# --------------------------------------------------------------------------
# P2/P3: weights sum to one; constant values come back unchanged.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_return_themselves(causal):
    B, H, N, D = 2, 3, 37, 8
    q, k = _rand((B, H, N, D), 1), _rand((B, H, N, D), 2)
    c = _rand((D,), 3)
    v = np.broadcast_to(c, (B, H, N, D)).copy()
    o, _ = oracle.fwd(q, k, v, 0.35, causal)
    assert np.abs(o - c).max() <= 1e-14 * np.abs(c).max() * 4
    ones = np.ones((B, H, N, D))
    o1, _ = oracle.fwd(q, k, ones, 0.35, causal)  # row sums of P
    assert np.abs(o1 - 1.0).max() < 1e-13


# --------------------------------------------------------------------------
# P4/P8: causal row 0 reads only key 0; N = 1; shift and permutation.
# --------------------------------------------------------------------------
def test_causal_row0_and_single_token():
    B, H, N, D = 1, 2, 9, 5
    q, k, v = (_rand((B, H, N, D), s) for s in (4, 5, 6))
    scale = 0.7
    o, lse = oracle.fwd(q, k, v, scale, True)
    for h in range(H):
        assert np.array_equal(o[0, h, 0], v[0, h, 0])
        s00 = scale * math.fsum(q[0, h, 0] * k[0, h, 0])
        assert abs(lse[0, h, 0] - s00) < 1e-15
    o1, l1 = oracle.fwd(q[:, :, :1], k[:, :, :1], v[:, :, :1], scale, False)
    assert np.array_equal(o1[0, :, 0], v[0, :, 0])


@pytest.mark.parametrize("causal", [False, True])
def test_score_shift_moves_lse_only(causal):
    """Adding c to every key adds scale*<q_i, c> to every score of row i:
    weights are unchanged (stable softmax, tensortonic section 4) and L moves
    by exactly that amount."""
    B, H, N, D = 1, 2, 23, 6
    q, k, v = (_rand((B, H, N, D), s) for s in (7, 8, 9))
    c = _rand((D,), 10)
    scale = 0.4
    o, lse = oracle.fwd(q, k, v, scale, causal)
    o2, lse2 = oracle.fwd(q, k + c, v, scale, causal)
    shift = scale * np.einsum("bhnd,d->bhn", q, c)
    assert np.abs(o2 - o).max() < 1e-12
    assert np.abs(lse2 - lse - shift).max() < 1e-12


def test_key_value_permutation_invariance_noncausal():
    B, H, N, D = 1, 1, 19, 7
    q, k, v = (_rand((B, H, N, D), s) for s in (11, 12, 13))
    perm = np.random.default_rng(14).permutation(N)
    o, lse = oracle.fwd(q, k, v, 0.3, False)
    o2, lse2 = oracle.fwd(q, k[:, :, perm], v[:, :, perm], 0.3, False)
    assert np.abs(o2 - o).max() < 1e-13
    assert np.abs(lse2 - lse).max() < 1e-13


def test_outputs_are_convex_combinations():
    B, H, N, D = 2, 2, 31, 4
    q, k, v = (_rand((B, H, N, D), s) for s in (15, 16, 17))
    for causal in (False, True):
        o, _ = oracle.fwd(q, k, v, 1.3, causal)
        for i in range(N):
            kv = v[:, :, : (i + 1 if causal else N)]
            assert (o[:, :, i] <= kv.max(axis=2) + 1e-13).all()
            assert (o[:, :, i] >= kv.min(axis=2) - 1e-13).all()


# --------------------------------------------------------------------------
# P5/P10: L is the log-sum-exp of the row; exp(s - L) recovers the weights.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_lse_is_logsumexp_and_recomputes_weights(causal):
    B, H, N, D = 1, 2, 16, 16  # D >= N: one-hot values expose P itself
    q, k = _rand((B, H, N, D), 18), _rand((B, H, N, D), 19)
    v = np.broadcast_to(np.eye(N, D), (B, H, N, D)).copy()
    scale = 0.45
    o, lse = oracle.fwd(q, k, v, scale, causal)
    s = scale * np.matmul(q, np.swapaxes(k, -1, -2))
    for h in range(H):
        for i in range(N):
            n = i + 1 if causal else N
            ref = scipy.special.logsumexp(s[0, h, i, :n])
            assert abs(lse[0, h, i] - ref) < 1e-13
            p = o[0, h, i, :N]
            assert np.abs(p[:n] - np.exp(s[0, h, i, :n] - lse[0, h, i])).max() < 1e-14
            assert np.abs(p[n:]).max(initial=0.0) == 0.0


# --------------------------------------------------------------------------
# P6: 50-digit brute force on tiny inputs.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1), (1, 2, 5, 3), (2, 1, 8, 4)])
def test_mpmath_brute_force(shape, causal):
    q, k, v = (_rand(shape, s) for s in (20, 21, 22))
    scale = 0.6
    o, lse = oracle.fwd(q, k, v, scale, causal)
    mpmath.mp.dps = 50
    B, H, N, D = shape
    for b in range(B):
        for h in range(H):
            for i in range(N):
                n = i + 1 if causal else N
                s = [mpmath.mpf(scale) * mpmath.fsum(
                    mpmath.mpf(q[b, h, i, d]) * mpmath.mpf(k[b, h, j, d])
                    for d in range(D)) for j in range(n)]
                w = [mpmath.e ** x for x in s]
                tot = mpmath.fsum(w)
                for d in range(D):
                    ref = mpmath.fsum(w[j] * mpmath.mpf(v[b, h, j, d])
                                      for j in range(n)) / tot
                    assert abs(o[b, h, i, d] - float(ref)) <= 1e-13 * (1 + abs(float(ref)))
                assert abs(lse[b, h, i] - float(mpmath.log(tot))) < 1e-13


# --------------------------------------------------------------------------
# P7: a library routine in the special case it covers (equal lengths).
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,D", [(1, 64), (63, 64), (129, 128), (300, 64)])
def test_matches_torch_sdpa_fp64(N, D, causal):
    g = torch.Generator().manual_seed(N * 7 + D)
    q, k, v = (torch.randn(2, 2, N, D, generator=g, dtype=torch.float64)
               for _ in range(3))
    scale = 1.0 / math.sqrt(D)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, is_causal=causal, scale=scale).numpy()
    o, _ = oracle.fwd(q, k, v, scale, causal)
    assert np.abs(o - ref).max() < 1e-12


# --------------------------------------------------------------------------
# Selected-row and packed entry points agree with the dense forward.
# --------------------------------------------------------------------------
def test_rows_and_varlen_agree_with_dense():
    B, H, N, D = 2, 3, 41, 8
    q, k, v = (_rand((B, H, N, D), s) for s in (23, 24, 25))
    for causal in (False, True):
        o, lse = oracle.fwd(q, k, v, 0.5, causal)
        bh = np.array([0, 5, 3, 2, 4])
        rows = np.array([0, 40, 17, 1, 39])
        orows, lrows = oracle.fwd_rows(q, k, v, 0.5, causal, bh, rows)
        of, lf = o.reshape(B * H, N, D), lse.reshape(B * H, N)
        assert np.array_equal(orows, of[bh, rows])
        assert np.array_equal(lrows, lf[bh, rows])
    # packing: sequences of lengths 5, 0, 17, 1 behave as independent runs
    lengths = [5, 0, 17, 1]
    cu = attn_inputs.cu_seqlens(lengths).numpy()
    total = int(cu[-1])
    qp, kp, vp = (_rand((H, total, D), s) for s in (26, 27, 28))
    for causal in (False, True):
        o, lse = oracle.fwd_varlen(qp, kp, vp, cu, 0.5, causal)
        for b, n in enumerate(lengths):
            if n == 0:
                continue
            sl = slice(cu[b], cu[b + 1])
            od, ld = oracle.fwd(qp[None, :, sl], kp[None, :, sl],
                                vp[None, :, sl], 0.5, causal)
            assert np.array_equal(o[:, sl], od[0])
            assert np.array_equal(lse[:, sl], ld[0])
        heads = np.array([0, 2, 1, 2])
        toks = np.array([0, 4, 5, total - 1])
        orow, lrow = oracle.fwd_varlen_rows(qp, kp, vp, cu, 0.5, causal,
                                            heads, toks)
        assert np.array_equal(orow, o[heads, toks])
        assert np.array_equal(lrow, lse[heads, toks])


# --------------------------------------------------------------------------
# P11: the stability variant (Q * 8) of the tiny workload.
# --------------------------------------------------------------------------
def test_stability_variant_large_scores():
    q, k, v, q8 = attn_inputs.tiny_inputs()
    scale = attn_inputs.TINY.scale
    raw = torch.matmul(q8.double(), k.double().transpose(-1, -2))
    assert raw.abs().max() > 100  # raw scores exceed 100
    # exp of a raw score this large overflows fp32 (max ~ e^88.7): only the
    # max-subtraction of the stable softmax keeps the weights finite
    assert float(raw.max()) > 88.8
    o, lse = oracle.fwd(q8, k, v, scale, False)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    mpmath.mp.dps = 50
    q8d, kd, vd = (x.double().numpy()[0, 0] for x in (q8, k, v))
    for i in (0, 17, 64, 127):
        s = [mpmath.mpf(scale) * mpmath.fsum(
            mpmath.mpf(a) * mpmath.mpf(b) for a, b in zip(q8d[i], kd[j]))
            for j in range(128)]
        w = [mpmath.e ** x for x in s]
        tot = mpmath.fsum(w)
        assert abs(lse[0, 0, i] - float(mpmath.log(tot))) < 1e-12
        for d in (0, 31, 63):
            ref = float(mpmath.fsum(w[j] * mpmath.mpf(vd[j, d])
                                    for j in range(128)) / tot)
            assert abs(o[0, 0, i, d] - ref) < 1e-13


# --------------------------------------------------------------------------
# P9: backward.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences(causal):
    B, H, N, D = 1, 2, 6, 3
    q, k, v, do = (_rand((B, H, N, D), s) for s in (30, 31, 32, 33))
    scale = 0.8
    dq, dk, dv = oracle.bwd(q, k, v, do, scale, causal)

    def f(qq, kk, vv):
        o, _ = oracle.fwd(qq, kk, vv, scale, causal)
        return float(np.sum(o * do))

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = f(args["q"], args["k"], args["v"])
            args[name] = xm
            fm = f(args["q"], args["k"], args["v"])
            num[idx] = (fp - fm) / (2 * h)
        err = np.linalg.norm(num - g) / np.linalg.norm(g)
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_autograd_and_invariants(causal):
    B, H, N, D = 2, 2, 70, 16
    g = torch.Generator().manual_seed(34)
    q, k, v, do = (torch.randn(B, H, N, D, generator=g, dtype=torch.float64)
                   for _ in range(4))
    scale = 0.25
    qa, ka, va = (x.clone().requires_grad_(True) for x in (q, k, v))
    s = scale * torch.matmul(qa, ka.transpose(-1, -2))
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1),
                          float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), va)
    o.backward(do)
    dq, dk, dv = oracle.bwd(q, k, v, do, scale, causal)
    for ref, got in ((qa.grad, dq), (ka.grad, dk), (va.grad, dv)):
        ref = ref.numpy()
        assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 1e-12
    # softmax is shift-invariant in the keys: sum_j dK_j = 0
    assert np.abs(dk.sum(axis=2)).max() < 1e-11
    # rows of P sum to one: sum_j dV_j = sum_i dO_i
    assert np.abs(dv.sum(axis=2) - do.numpy().sum(axis=2)).max() < 1e-11


@pytest.mark.parametrize("causal", [False, True])
def test_packed_backward_matches_autograd_on_block_diagonal_mask(causal):
    """The packed backward against torch fp64 autograd through attention over
    the whole packed token axis with an explicit mask: key j is allowed for
    query i only inside i's sequence (and j <= i there if causal), the
    packed forward's definition.  Empty sequences included."""
    lengths = [0, 37, 1, 0, 60, 23]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    H, total, D = 2, int(cu[-1]), 8
    g = torch.Generator().manual_seed(35)
    q, k, v, do = (torch.randn(H, total, D, generator=g, dtype=torch.float64)
                   for _ in range(4))
    scale = 0.3
    seq = torch.empty(total, dtype=torch.long)
    pos = torch.empty(total, dtype=torch.long)
    for b in range(len(lengths)):
        seq[cu[b]:cu[b + 1]] = b
        pos[cu[b]:cu[b + 1]] = torch.arange(lengths[b])
    allowed = seq[:, None] == seq[None, :]
    if causal:
        allowed &= pos[None, :] <= pos[:, None]
    qa, ka, va = (x.clone().requires_grad_(True) for x in (q, k, v))
    sc = (scale * torch.matmul(qa, ka.transpose(-1, -2))).masked_fill(~allowed, float("-inf"))
    o = torch.matmul(torch.softmax(sc, dim=-1), va)
    o.backward(do)
    dq, dk, dv = oracle.bwd_varlen(q, k, v, do, cu, scale, causal)
    for ref, got in ((qa.grad, dq), (ka.grad, dk), (va.grad, dv)):
        ref = ref.numpy()
        assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 1e-12


def test_packed_backward_has_no_cross_sequence_gradient():
    """Changing one sequence's inputs leaves every other sequence's
    gradients bitwise unchanged (no attention across sequence bounds)."""
    cu = np.array([0, 20, 45, 70], dtype=np.int32)
    g = torch.Generator().manual_seed(36)
    q, k, v, do = (torch.randn(2, 70, 8, generator=g, dtype=torch.float64)
                   for _ in range(4))
    base = oracle.bwd_varlen(q, k, v, do, cu, 0.4, True)
    q2, v2 = q.clone(), v.clone()
    q2[:, 20:45] += 1.0
    v2[:, 20:45] *= -2.0
    moved = oracle.bwd_varlen(q2, k, v2, do, cu, 0.4, True)
    for a, b in zip(base, moved):
        assert np.array_equal(a[:, :20], b[:, :20])
        assert np.array_equal(a[:, 45:], b[:, 45:])
        assert not np.array_equal(a[:, 20:45], b[:, 20:45])


def test_input_generators_are_seeded_bf16():
    a = attn_inputs.randn_bf16((2, 3, 5, 8), 7)
    b = attn_inputs.randn_bf16((2, 3, 5, 8), 7)
    assert a.dtype == torch.bfloat16 and torch.equal(a, b)
    c = attn_inputs.randn_bf16((2, 3, 5, 8), 7, chunk_rows=4)
    assert c.shape == a.shape and torch.isfinite(c.float()).all()
    lengths = attn_inputs.varlen_lengths(2)
    assert len(lengths) == 16 and all(128 <= n <= 8192 for n in lengths)
    cu = attn_inputs.cu_seqlens(lengths)
    assert cu.dtype == torch.int32 and int(cu[-1]) == sum(lengths)


# --------------------------------------------------------------------------
# Unequal query and key lengths.  The square causal mask is not right for
# every unequal-length layout (tensortonic section 9); the queries are the
# last Nq positions of the key sequence, so the mask is aligned bottom-right.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk", [(1, 37), (5, 64), (64, 17), (33, 33), (100, 260)])
def test_unequal_lengths_match_torch_sdpa_with_explicit_mask(Nq, Nk, causal):
    g = torch.Generator().manual_seed(Nq * 1000 + Nk)
    D = 16
    q = torch.randn(2, 3, Nq, D, generator=g, dtype=torch.float64)
    k, v = (torch.randn(2, 3, Nk, D, generator=g, dtype=torch.float64) for _ in range(2))
    scale = 0.3
    o, lse = oracle.fwd_qk(q, k, v, scale, causal)
    mask = torch.ones(Nq, Nk, dtype=torch.bool)
    if causal:
        mask = mask.tril(diagonal=Nk - Nq)  # query i reads keys j <= i + Nk - Nq
    live = mask.any(dim=1).numpy()
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=mask, scale=scale).numpy()
    assert np.abs(o[:, :, live] - ref[:, :, live]).max() < 1e-12
    s = scale * (q @ k.transpose(-1, -2))
    ref_l = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1).numpy()
    assert np.abs(lse[:, :, live] - ref_l[:, :, live]).max() < 1e-12
    # rows with no readable key (more queries than keys under the causal mask)
    assert (o[:, :, ~live] == 0).all() and np.isneginf(lse[:, :, ~live]).all()
    assert live.all() == (not causal or Nq <= Nk)


def test_unequal_lengths_special_cases():
    q, k, v = (_rand(s, seed) for s, seed in (((2, 2, 9, 8), 30), ((2, 2, 9, 8), 31),
                                               ((2, 2, 9, 8), 32)))
    for causal in (False, True):  # equal lengths: the square definition
        a = oracle.fwd_qk(q, k, v, 0.4, causal)
        b = oracle.fwd(q, k, v, 0.4, causal)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    kl, vl = _rand((2, 2, 40, 8), 33), _rand((2, 2, 40, 8), 34)
    oc, lc = oracle.fwd_qk(q, kl, vl, 0.4, True)
    on, ln = oracle.fwd_qk(q, kl, vl, 0.4, False)
    # the last query reads every key; one query alone (decoding) reads them all
    assert np.abs(oc[:, :, -1] - on[:, :, -1]).max() < 1e-15
    o1, l1 = oracle.fwd_qk(q[:, :, -1:], kl, vl, 0.4, True)
    assert np.abs(o1[:, :, 0] - on[:, :, -1]).max() < 1e-15
    # query i reads exactly keys 0 .. i + Nk - Nq: the same row of a square
    # problem over the last Nq + shift positions
    shift = 40 - 9
    for i in (0, 4, 8):
        oi, li = oracle.fwd(np.concatenate([np.zeros((2, 2, shift, 8)), q], axis=2),
                            kl, vl, 0.4, True)
        assert np.abs(oi[:, :, shift + i] - oc[:, :, i]).max() < 1e-14
    rows = np.array([0, 5, 8, 3]); bh = np.array([0, 3, 1, 2])
    orow, lrow = oracle.fwd_qk_rows(q, kl, vl, 0.4, True, bh, rows)
    for t in range(4):
        b, h = divmod(int(bh[t]), 2)
        assert np.array_equal(orow[t], oc[b, h, rows[t]]) and lrow[t] == lc[b, h, rows[t]]


@pytest.mark.parametrize("causal", [False, True])
def test_unequal_lengths_mpmath(causal):
    Nq, Nk, D = 3, 6, 3
    q, k, v = _rand((1, 1, Nq, D), 35), _rand((1, 1, Nk, D), 36), _rand((1, 1, Nk, D), 37)
    scale = 0.7
    o, lse = oracle.fwd_qk(q, k, v, scale, causal)
    mpmath.mp.dps = 50
    for i in range(Nq):
        n = i + Nk - Nq + 1 if causal else Nk
        s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[0, 0, i, d]) * mpmath.mpf(k[0, 0, j, d])
                                             for d in range(D)) for j in range(n)]
        w = [mpmath.e ** x for x in s]
        tot = mpmath.fsum(w)
        for d in range(D):
            ref = mpmath.fsum(w[j] * mpmath.mpf(v[0, 0, j, d]) for j in range(n)) / tot
            assert abs(o[0, 0, i, d] - float(ref)) <= 1e-13 * (1 + abs(float(ref)))
        assert abs(lse[0, 0, i] - float(mpmath.log(tot))) < 1e-13


def test_key_split_partials_merge_by_lse():
    """Attention over disjoint key ranges combines exactly: L = logsumexp of
    the partial L's and O = sum_s exp(L_s - L) O_s (the running-softmax rule of
    tensortonic section 5 applied to whole ranges; the decode path splits the
    keys this way)."""
    q, k, v = _rand((2, 3, 4, 16), 38), _rand((2, 3, 300, 16), 39), _rand((2, 3, 300, 16), 40)
    o, lse = oracle.fwd_qk(q, k, v, 0.25, False)
    cuts = [0, 7, 130, 131, 300]
    parts = [oracle.fwd_qk(q, k[:, :, a:b], v[:, :, a:b], 0.25, False)
             for a, b in zip(cuts[:-1], cuts[1:])]
    L = scipy.special.logsumexp(np.stack([p[1] for p in parts]), axis=0)
    O = sum(np.exp(p[1] - L)[..., None] * p[0] for p in parts)
    assert np.abs(L - lse).max() < 1e-13 and np.abs(O - o).max() < 1e-13


# --------------------------------------------------------------------------
# Attention dropout (tensortonic section 7: the backward replays the forward's
# drop decisions).  The generator is Philox4x32-10 as published by Salmon et
# al.; its stream is pinned by the published known-answer vectors, its
# statistics are checked besides, and every use of it is pinned by closed
# forms and library routines on the same mask.
# --------------------------------------------------------------------------
def test_philox_known_answer_vectors():
    """The oracle's generator reproduces the known-answer vectors published
    with Philox4x32-10 (tests/golden/philox4x32_10_kat.txt): a wrong round
    multiplier, key increment, round count or output word order fails them."""
    n = 0
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split("->")
            words = [int(x, 16) for x in lhs.split()]
            want = [int(x, 16) for x in rhs.split()]
            got = [int(x) for x in oracle.philox4x32_10(words[:4], words[4:])]
            assert got == want, (line, ["%08x" % x for x in got])
            n += 1
    assert n == 3


def test_philox_statistics_and_injectivity():
    outs = np.array([oracle.philox4x32_10([c, 7, 3, 0], [11, 22]) for c in range(4096)],
                    dtype=np.uint64)
    bits = np.array([(outs >> b) & 1 for b in range(32)], dtype=float)  # [32, 4096, 4]
    frac = bits.mean(axis=(1, 2))
    n = outs.size
    assert np.abs(frac - 0.5).max() < 5 * 0.5 / math.sqrt(n)        # every bit balanced
    by = np.concatenate([(outs >> (8 * t)) & 0xFF for t in range(4)]).ravel()
    hist = np.bincount(by.astype(np.int64), minlength=256)
    chi2 = ((hist - by.size / 256) ** 2 / (by.size / 256)).sum()
    assert chi2 < 255 + 6 * math.sqrt(2 * 255)                       # bytes uniform
    u = outs.astype(float) / 2.0 ** 32
    assert abs(np.corrcoef(u[:-1, 0], u[1:, 0])[0, 1]) < 5 / math.sqrt(4096)
    assert abs(np.corrcoef(u[:, 0], u[:, 1])[0, 1]) < 5 / math.sqrt(4096)
    words = {tuple(o) for o in outs.tolist()}
    assert len(words) == 4096                                         # no collisions
    assert not np.array_equal(oracle.philox4x32_10([5, 7, 3, 0], [11, 22]),
                              oracle.philox4x32_10([5, 7, 3, 0], [12, 22]))


def test_dropout_threshold_and_mask_structure():
    assert [oracle.dropout_threshold(p) for p in (0.0, 1 / 512, 0.1, 0.25, 0.999)] == \
        [0, 1, 26, 64, 255]
    big = oracle.dropout_mask(3, 100, 100, 0.3, 77, 5)
    assert np.array_equal(oracle.dropout_mask(3, 64, 64, 0.3, 77, 5), big[:64, :64])
    assert not np.array_equal(oracle.dropout_mask(4, 64, 64, 0.3, 77, 5), big[:64, :64])
    assert not np.array_equal(oracle.dropout_mask(3, 64, 64, 0.3, 78, 5), big[:64, :64])
    assert not np.array_equal(oracle.dropout_mask(3, 64, 64, 0.3, 77, 6), big[:64, :64])
    assert oracle.dropout_mask(3, 64, 64, 0.0, 77, 5).all()
    m = oracle.dropout_mask(0, 256, 2048, 0.3, 9, 0)
    keep = 1 - oracle.dropout_threshold(0.3) / 256
    assert abs(m.mean() - keep) < 5 * math.sqrt(keep * (1 - keep) / m.size)


def _masked_reference(q, k, v, scale, causal, p, seed, offset):
    """torch fp64: O = (softmax(S) * keep / (1 - p')) V, per head, with the
    oracle's mask, plus autograd gradients of <dO, O>."""
    B, H, N, D = q.shape
    keep = np.stack([oracle.dropout_mask(bh, N, N, p, seed, offset) for bh in range(B * H)])
    z = torch.tensor(keep.reshape(B, H, N, N), dtype=torch.float64) * \
        (256 / (256 - oracle.dropout_threshold(p)))
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = scale * qt @ kt.transpose(-1, -2)
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), -math.inf)
    o = (torch.softmax(s, dim=-1) * z) @ vt
    return o, torch.logsumexp(s, dim=-1), (qt, kt, vt)


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_forward_backward_match_torch_on_the_same_mask(causal):
    B, H, N, D = 2, 2, 37, 8
    q, k, v, do = (_rand((B, H, N, D), s) for s in (50, 51, 52, 53))
    scale, p, seed, offset = 0.4, 0.3, 1234, 99
    o, lse = oracle.fwd_dropout(q, k, v, scale, causal, p, seed, offset)
    o_ref, l_ref, leaves = _masked_reference(q, k, v, scale, causal, p, seed, offset)
    assert np.abs(o - o_ref.detach().numpy()).max() < 1e-12
    assert np.abs(lse - l_ref.detach().numpy()).max() < 1e-12
    (o_ref * torch.tensor(do)).sum().backward()
    grads = oracle.bwd_dropout(q, k, v, do, scale, causal, p, seed, offset)
    for g, leaf in zip(grads, leaves):
        assert np.abs(g - leaf.grad.numpy()).max() < 1e-12
    # p = 0 is attention without dropout, bit for bit
    o0, l0 = oracle.fwd_dropout(q, k, v, scale, causal, 0.0, seed, offset)
    a, b = oracle.fwd(q, k, v, scale, causal)
    assert np.array_equal(o0, a) and np.array_equal(l0, b)
    g0 = oracle.bwd_dropout(q, k, v, do, scale, causal, 0.0, seed, offset)
    for x, y in zip(g0, oracle.bwd(q, k, v, do, scale, causal)):
        assert np.array_equal(x, y)


def test_dropout_is_unbiased():
    """Kept weights are scaled by 1 / (1 - p'): averaged over seeds the output
    approaches the output without dropout."""
    q, k, v = (_rand((1, 1, 8, 4), s) for s in (60, 61, 62))
    ref, _ = oracle.fwd(q, k, v, 0.5, False)
    runs = np.stack([oracle.fwd_dropout(q, k, v, 0.5, False, 0.4, seed, 0)[0]
                     for seed in range(3000)])
    mean, se = runs.mean(axis=0), runs.std(axis=0) / math.sqrt(len(runs))
    assert (np.abs(mean - ref) < 5 * se + 1e-12).all()


@pytest.mark.parametrize("causal", [False, True])
def test_packed_dropout_matches_torch_on_assembled_masks(causal):
    """Packed dropout forward and backward against torch fp64 (forward and
    autograd) over the whole packed axis: the allowed set is block diagonal
    (causal inside each sequence) and sequence b of head h keeps the weights
    dropout_mask(b * H + h, ...) keeps, positions counted from its start."""
    lengths = [0, 29, 1, 40, 0, 17]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    H, total, D = 2, int(cu[-1]), 8
    p, seed, offset = 0.25, 1234, 7
    g = torch.Generator().manual_seed(37)
    q, k, v, do = (torch.randn(H, total, D, generator=g, dtype=torch.float64)
                   for _ in range(4))
    scale = 0.35
    allowed = torch.zeros(total, total, dtype=torch.bool)
    z = torch.zeros(H, total, total, dtype=torch.float64)
    inv_keep = 256.0 / (256.0 - oracle.dropout_threshold(p))
    for b, n in enumerate(lengths):
        s, e = int(cu[b]), int(cu[b + 1])
        if n == 0:
            continue
        blk = torch.ones(n, n, dtype=torch.bool)
        allowed[s:e, s:e] = blk.tril() if causal else blk
        for h in range(H):
            keep = oracle.dropout_mask(b * H + h, n, n, p, seed, offset)
            z[h, s:e, s:e] = torch.from_numpy(keep.astype(np.float64)) * inv_keep
    qa, ka, va = (x.clone().requires_grad_(True) for x in (q, k, v))
    sc = (scale * torch.matmul(qa, ka.transpose(-1, -2))).masked_fill(~allowed, float("-inf"))
    lse_ref = torch.logsumexp(sc, dim=-1)
    o_ref = torch.matmul(torch.softmax(sc, dim=-1) * z, va)
    o_ref.backward(do)
    o, lse = oracle.fwd_varlen_dropout(q, k, v, cu, scale, causal, p, seed, offset)
    assert np.abs(o - o_ref.detach().numpy()).max() < 1e-12
    assert np.abs(lse - lse_ref.detach().numpy()).max() < 1e-12
    grads = oracle.bwd_varlen_dropout(q, k, v, do, cu, scale, causal, p, seed, offset)
    for ref, got in ((qa.grad, grads[0]), (ka.grad, grads[1]), (va.grad, grads[2])):
        ref = ref.numpy()
        assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 1e-12


def test_packed_dropout_at_zero_is_the_packed_oracle():
    cu = np.array([0, 33, 33, 90], dtype=np.int32)
    g = torch.Generator().manual_seed(38)
    q, k, v, do = (torch.randn(2, 90, 8, generator=g, dtype=torch.float64) for _ in range(4))
    o0, l0 = oracle.fwd_varlen(q, k, v, cu, 0.3, True)
    o1, l1 = oracle.fwd_varlen_dropout(q, k, v, cu, 0.3, True, 0.0, 5, 0)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    g0 = oracle.bwd_varlen(q, k, v, do, cu, 0.3, True)
    g1 = oracle.bwd_varlen_dropout(q, k, v, do, cu, 0.3, True, 0.0, 5, 0)
    for a, b in zip(g0, g1):
        assert np.abs(a - b).max() < 1e-13
