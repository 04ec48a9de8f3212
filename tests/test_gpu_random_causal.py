"""GPU parity on seeded random causal shapes, aimed at the orders in which
the kernels visit tiles: a causal pair's light query tile walks its keys from
the top down (forward), and a dK/dV unit's first key tile walks its query
stages from the last one down, so the lengths drawn here put every count of
masked and unmasked steps, odd and even, in front of those walks.  Each case
is compared with the fp64 oracle over every element (forward O and L; the
gradients by relative L2 per tensor and per 64-row block)."""
import numpy as np
import pytest

import attn_inputs as ai
import oracle
from _parity import check_fwd, check_grad, say

pytestmark = pytest.mark.gpu

_RNG = np.random.default_rng(31337)


def _draw(lo, hi):
    return int(_RNG.integers(lo, hi + 1))


# (B, H, N, D) dense causal forward
FWD = [(_draw(1, 2), _draw(1, 3), _draw(129, 3000), int(_RNG.choice([64, 128])))
       for _ in range(8)]
# (Nq, Nk, D): bottom-right causal; half the key surpluses are 32m + 31, where
# the light tile's first row has all its keys in unmasked tiles
QK = []
for i in range(8):
    nq = _draw(129, 1200)
    surplus = _draw(0, 40) * 32 + (31 if i % 2 == 0 else _draw(0, 31))
    QK.append((nq, nq + surplus, int(_RNG.choice([64, 128]))))
# (B, H, N, D) dense causal backward
BWD = [(1, _draw(1, 2), _draw(257, 2600), int(_RNG.choice([64, 128]))) for _ in range(6)]
# (lengths, H, D) packed causal forward and backward, empty sequences allowed
VARLEN = [([_draw(0, 1500) for _ in range(_draw(1, 5))], _draw(1, 2), int(_RNG.choice([64, 128])))
          for _ in range(5)]


@pytest.mark.parametrize("case", FWD, ids=lambda c: "B%dH%dN%dD%d" % c)
def test_forward(gpu, case):
    B, H, N, D = case
    say("case random causal forward", case)
    q, k, v = ai.qkv(B, H, N, D, seed=9000 + N)
    o, lse = gpu.fa_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True)
    o_ref, l_ref = oracle.fwd(q, k, v, ai.default_scale(D), True)
    check_fwd(o, lse, o_ref, l_ref, "random causal forward")


@pytest.mark.parametrize("case", QK, ids=lambda c: "Nq%dNk%dD%d" % c)
def test_unequal_lengths(gpu, case):
    Nq, Nk, D = case
    say("case random bottom-right causal", case)
    g = ai.generator(9100 + Nk)
    q = ai.randn_bf16((1, 2, Nq, D), g)
    k, v = ai.randn_bf16((1, 2, Nk, D), g), ai.randn_bf16((1, 2, Nk, D), g)
    o, lse = gpu.fa_fwd_qk(q.cuda(), k.cuda(), v.cuda(), causal=True)
    o_ref, l_ref = oracle.fwd_qk(q, k, v, ai.default_scale(D), True)
    check_fwd(o, lse, o_ref, l_ref, "random bottom-right causal")


@pytest.mark.parametrize("case", BWD, ids=lambda c: "B%dH%dN%dD%d" % c)
def test_backward(gpu, case):
    B, H, N, D = case
    say("case random causal backward", case)
    q, k, v, do = ai.backward_inputs(B, H, N, D, seed=9200 + N)
    qc, kc, vc, doc = (x.cuda() for x in (q, k, v, do))
    o, lse = gpu.fa_fwd(qc, kc, vc, causal=True)
    grads = gpu.fa_bwd(qc, kc, vc, o, lse, doc, causal=True)
    refs = oracle.bwd(q, k, v, do, ai.default_scale(D), True)
    for name, g_, r in zip(("dq", "dk", "dv"), grads, refs):
        check_grad(g_, r, "random causal backward " + name)


@pytest.mark.parametrize("case", VARLEN, ids=lambda c: "n%dH%dD%d" % (len(c[0]), c[1], c[2]))
def test_packed(gpu, case):
    lengths, H, D = case
    cu = ai.cu_seqlens(lengths)
    total = int(cu[-1])
    if total == 0:
        pytest.skip("all sequences empty")
    say("case random packed causal", lengths, H, D)
    g = ai.generator(9300 + total)
    q, k, v, do = (ai.randn_bf16((H, total, D), g) for _ in range(4))
    qc, kc, vc, doc, cuc = (x.cuda() for x in (q, k, v, do, cu))
    o, lse = gpu.fa_fwd_varlen(qc, kc, vc, cuc, max(lengths), causal=True)
    o_ref, l_ref = oracle.fwd_varlen(q, k, v, cu, ai.default_scale(D), True)
    check_fwd(o, lse, o_ref, l_ref, "random packed causal forward")
    grads = gpu.fa_bwd_varlen(qc, kc, vc, o, lse, doc, cuc, max(lengths), causal=True)
    refs = oracle.bwd_varlen(q, k, v, do, cu, ai.default_scale(D), True)
    for name, g_, r in zip(("dq", "dk", "dv"), grads, refs):
        check_grad(g_, r, "random packed causal " + name, cu=cu)
