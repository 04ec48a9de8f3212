"""Guard bands around every output: each entry point writes exactly its
outputs and nothing beside them.

Every output (o, lse, dq, dk, dv) and every workspace is placed inside a
larger device buffer whose bytes before and after it hold a fixed pattern.
After the call the pattern must be intact, and the outputs themselves must
match the oracle at the usual tolerances.  The shapes are ragged (partial
query and key tiles, an empty packed sequence), so the tail handling of the
range-checked loads and stores is what these tests exercise.
"""
import pytest
import torch

import attn_inputs as ai
import oracle
from _parity import check_fwd, check_grad, say

pytestmark = pytest.mark.gpu

FRONT = 4096          # bytes of pattern before each output (keeps 16-byte alignment)
BACK = 65536          # bytes of pattern after it
PATTERN = 0xA5


class Guarded:
    """A tensor of the given shape and dtype inside a pattern-filled buffer."""

    def __init__(self, shape, dtype):
        n = 1
        for s in shape:
            n *= int(s)
        self.nbytes = n * torch.tensor([], dtype=dtype).element_size()
        self.buf = torch.full((FRONT + self.nbytes + BACK,), PATTERN, dtype=torch.uint8,
                              device="cuda")
        self.t = self.buf[FRONT:FRONT + self.nbytes].view(dtype).view(*shape)

    def intact(self):
        head = self.buf[:FRONT]
        tail = self.buf[FRONT + self.nbytes:]
        return bool((head == PATTERN).all()) and bool((tail == PATTERN).all())


def _check_guards(what, **named):
    torch.cuda.synchronize()
    for name, g in named.items():
        assert g.intact(), "%s: bytes beside %s were written" % (what, name)


def test_fa_fwd_guard_bands(gpu):
    B, H, N, D = 1, 3, 200, 128
    q, k, v = ai.qkv(B, H, N, D, seed=5100)
    for causal in (False, True):
        say("canary fa_fwd", (B, H, N, D), causal)
        o, lse = Guarded((B, H, N, D), torch.bfloat16), Guarded((B, H, N), torch.float32)
        gpu.fa_fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, out=o.t, lse=lse.t)
        _check_guards("fa_fwd", o=o, lse=lse)
        o_ref, l_ref = oracle.fwd(q, k, v, ai.default_scale(D), causal)
        check_fwd(o.t, lse.t, o_ref, l_ref, "canary fa_fwd causal %d" % causal)


def test_fa_fwd_qk_guard_bands(gpu):
    B, H, Nq, Nk, D = 1, 2, 100, 333, 64
    g = ai.generator(5200)
    q = ai.randn_bf16((B, H, Nq, D), g)
    k, v = ai.randn_bf16((B, H, Nk, D), g), ai.randn_bf16((B, H, Nk, D), g)
    say("canary fa_fwd_qk")
    o, lse = Guarded((B, H, Nq, D), torch.bfloat16), Guarded((B, H, Nq), torch.float32)
    gpu.fa_fwd_qk(q.cuda(), k.cuda(), v.cuda(), causal=True, out=o.t, lse=lse.t)
    _check_guards("fa_fwd_qk", o=o, lse=lse)
    o_ref, l_ref = oracle.fwd_qk(q, k, v, ai.default_scale(D), True)
    check_fwd(o.t, lse.t, o_ref, l_ref, "canary fa_fwd_qk")


@pytest.mark.parametrize("nq", [3, 40])
def test_fa_fwd_splitkv_guard_bands(gpu, nq):
    """Decoding kernel (3 queries) and split forward tiles (40 queries), both
    with keys split over three ranges, so the workspace is in use."""
    B, H, Nk, D, splits = 1, 2, 700, 128, 3
    g = ai.generator(5300 + nq)
    q = ai.randn_bf16((B, H, nq, D), g)
    k, v = ai.randn_bf16((B, H, Nk, D), g), ai.randn_bf16((B, H, Nk, D), g)
    need = gpu.fa_fwd_splitkv_workspace_size(B, H, nq, Nk, D, splits)
    assert need > 0
    say("canary fa_fwd_splitkv", nq, "workspace", need)
    o, lse = Guarded((B, H, nq, D), torch.bfloat16), Guarded((B, H, nq), torch.float32)
    ws = Guarded((need,), torch.uint8)
    gpu.fa_fwd_splitkv(q.cuda(), k.cuda(), v.cuda(), causal=True, num_splits=splits,
                       out=o.t, lse=lse.t, workspace=ws.t)
    _check_guards("fa_fwd_splitkv", o=o, lse=lse, workspace=ws)
    o_ref, l_ref = oracle.fwd_qk(q, k, v, ai.default_scale(D), True)
    check_fwd(o.t, lse.t, o_ref, l_ref, "canary fa_fwd_splitkv nq %d" % nq)


def test_fa_fwd_varlen_guard_bands(gpu):
    lengths = [70, 0, 131, 5]
    H, D = 2, 128
    cu = ai.cu_seqlens(lengths)
    total = int(cu[-1])
    g = ai.generator(5400)
    q, k, v = (ai.randn_bf16((H, total, D), g) for _ in range(3))
    say("canary fa_fwd_varlen", lengths)
    o, lse = Guarded((H, total, D), torch.bfloat16), Guarded((H, total), torch.float32)
    gpu.fa_fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cu.cuda(), max(lengths), causal=True,
                      out=o.t, lse=lse.t)
    _check_guards("fa_fwd_varlen", o=o, lse=lse)
    o_ref, l_ref = oracle.fwd_varlen(q, k, v, cu, ai.default_scale(D), True)
    check_fwd(o.t, lse.t, o_ref, l_ref, "canary fa_fwd_varlen")


@pytest.mark.parametrize("dropout_p", [0.0, 0.2])
def test_fa_bwd_guard_bands(gpu, dropout_p):
    B, H, N, D = 1, 2, 300, 128
    q, k, v, do = ai.backward_inputs(B, H, N, D, seed=5500)
    scale = ai.default_scale(D)
    seed, offset = 77, 3
    say("canary fa_bwd", (B, H, N, D), "dropout", dropout_p)
    qc, kc, vc, doc = (x.cuda() for x in (q, k, v, do))
    o, lse = gpu.fa_fwd(qc, kc, vc, causal=True, dropout_p=dropout_p, seed=seed,
                        offset=offset)
    grads = [Guarded((B, H, N, D), torch.bfloat16) for _ in range(3)]
    ws = Guarded((gpu.fa_bwd_workspace_size(B, H, N, D),), torch.uint8)
    gpu.fa_bwd(qc, kc, vc, o, lse, doc, causal=True, dq=grads[0].t, dk=grads[1].t,
               dv=grads[2].t, workspace=ws.t, dropout_p=dropout_p, seed=seed, offset=offset)
    _check_guards("fa_bwd", dq=grads[0], dk=grads[1], dv=grads[2], workspace=ws)
    if dropout_p:
        refs = oracle.bwd_dropout(q, k, v, do, scale, True, dropout_p, seed, offset)
    else:
        refs = oracle.bwd(q, k, v, do, scale, True)
    for name, g, r in zip(("dq", "dk", "dv"), grads, refs):
        check_grad(g.t, r, "canary fa_bwd %s p %.1f" % (name, dropout_p))


def test_fa_bwd_varlen_guard_bands(gpu):
    lengths = [70, 0, 131, 5]
    H, D = 2, 64
    cu = ai.cu_seqlens(lengths)
    total = int(cu[-1])
    g = ai.generator(5600)
    q, k, v, do = (ai.randn_bf16((H, total, D), g) for _ in range(4))
    say("canary fa_bwd_varlen", lengths)
    qc, kc, vc, doc, cuc = (x.cuda() for x in (q, k, v, do, cu))
    o, lse = gpu.fa_fwd_varlen(qc, kc, vc, cuc, max(lengths), causal=True)
    grads = [Guarded((H, total, D), torch.bfloat16) for _ in range(3)]
    ws = Guarded((gpu.fa_bwd_workspace_size(1, H, total, D),), torch.uint8)
    gpu.fa_bwd_varlen(qc, kc, vc, o, lse, doc, cuc, max(lengths), causal=True,
                      dq=grads[0].t, dk=grads[1].t, dv=grads[2].t, workspace=ws.t)
    _check_guards("fa_bwd_varlen", dq=grads[0], dk=grads[1], dv=grads[2], workspace=ws)
    refs = oracle.bwd_varlen(q, k, v, do, cu, ai.default_scale(D), True)
    for name, g_, r in zip(("dq", "dk", "dv"), grads, refs):
        check_grad(g_.t, r, "canary fa_bwd_varlen " + name, cu=cu)


def test_fp16_guard_bands(gpu):
    B, H, N, D = 1, 2, 150, 64
    g = ai.generator(5700)
    q, k, v, do = (ai.randn_f16((B, H, N, D), g) for _ in range(4))
    say("canary fp16 forward and backward")
    qc, kc, vc, doc = (x.cuda() for x in (q, k, v, do))
    o, lse = Guarded((B, H, N, D), torch.float16), Guarded((B, H, N), torch.float32)
    gpu.fa_fwd(qc, kc, vc, causal=True, out=o.t, lse=lse.t)
    _check_guards("fa_fwd_f16", o=o, lse=lse)
    o_ref, l_ref = oracle.fwd(q, k, v, ai.default_scale(D), True)
    check_fwd(o.t, lse.t, o_ref, l_ref, "canary fp16 forward")
    grads = [Guarded((B, H, N, D), torch.float16) for _ in range(3)]
    gpu.fa_bwd(qc, kc, vc, o.t, lse.t, doc, causal=True, dq=grads[0].t, dk=grads[1].t,
               dv=grads[2].t)
    _check_guards("fa_bwd_f16", dq=grads[0], dk=grads[1], dv=grads[2])
    refs = oracle.bwd(q, k, v, do, ai.default_scale(D), True)
    for name, g_, r in zip(("dq", "dk", "dv"), grads, refs):
        check_grad(g_.t, r, "canary fp16 " + name)
