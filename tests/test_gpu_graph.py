"""The entry points allocate nothing, synchronise nothing and record no
memset, so a caller can capture them in a HIP graph (torch.cuda.CUDAGraph is
hipGraph on ROCm) and replay it.  Every replay, with eager work and
synchronisations between replays, must reproduce the eager results bit for
bit."""
import pytest
import torch

import attn_inputs as ai
from _parity import say

pytestmark = pytest.mark.gpu


def test_forward_backward_graph_replays_match_eager(gpu):
    B, H, N, D = 1, 4, 1000, 128
    q, k, v, do = (x.cuda() for x in ai.backward_inputs(B, H, N, D, seed=90))
    scale = ai.default_scale(D)
    o, lse = torch.empty_like(q), torch.empty(B, H, N, device="cuda")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(gpu.fa_bwd_workspace_size(B, H, N, D), dtype=torch.uint8, device="cuda")

    def step():
        gpu.fa_fwd(q, k, v, softmax_scale=scale, causal=True, out=o, lse=lse)
        gpu.fa_bwd(q, k, v, o, lse, do, softmax_scale=scale, causal=True, dq=dq, dk=dk, dv=dv,
                   workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, dq, dk, dv)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(3):
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say("replay", r)
        for name, got, want in zip(("o", "lse", "dq", "dk", "dv"), (o, lse, dq, dk, dv), ref):
            assert torch.equal(got, want), (r, name)


def test_varlen_graph_replays_match_eager(gpu):
    lengths = [300, 0, 77, 513]
    cu = ai.cu_seqlens(lengths).cuda()
    H, D, total = 2, 64, sum(lengths)
    g = ai.generator(91)
    q, k, v, do = (ai.randn_bf16((H, total, D), g).cuda() for _ in range(4))
    o, lse = torch.empty_like(q), torch.empty(H, total, device="cuda")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(gpu.fa_bwd_workspace_size(1, H, total, D), dtype=torch.uint8,
                     device="cuda")

    def step():
        gpu.fa_fwd_varlen(q, k, v, cu, max(lengths), causal=True, out=o, lse=lse)
        gpu.fa_bwd_varlen(q, k, v, o, lse, do, cu, max(lengths), causal=True, dq=dq, dk=dk,
                          dv=dv, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, dq, dk, dv)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(3):
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("o", "lse", "dq", "dk", "dv"), (o, lse, dq, dk, dv), ref):
            assert torch.equal(got, want), (r, name)
