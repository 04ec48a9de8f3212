"""The library called from a plain C++ host program (tests/c_abi_driver.cpp):
device memory from hipMalloc, a stream from hipStreamCreate, fa_fwd then
fa_bwd through include/fa.h, no Python or torch in the calling process.  The
inputs come from the seeded generators and the outputs are checked against
the oracle here."""
import os
import subprocess

import numpy as np
import pytest
import torch

import attn_inputs as ai
import c_abi_build
import oracle
from _parity import check_fwd, check_grad, say

pytestmark = pytest.mark.gpu


def _bf16(path, shape):
    raw = np.fromfile(path, dtype=np.int16).reshape(shape)
    return torch.from_numpy(raw).view(torch.bfloat16)


@pytest.mark.parametrize("shape,causal", [((1, 2, 333, 128), True), ((2, 1, 130, 64), False)])
def test_host_program_calls_the_library(gpu, tmp_path, shape, causal):
    B, H, N, D = shape
    q, k, v, do = ai.backward_inputs(B, H, N, D, seed=7500 + N)
    for name, t in (("q", q), ("k", k), ("v", v), ("do", do)):
        t.contiguous().view(torch.int16).numpy().tofile(str(tmp_path / (name + ".bin")))
    scale = ai.default_scale(D)
    exe = c_abi_build.build()
    cmd = [exe, str(tmp_path), str(B), str(H), str(N), str(D), str(int(causal)), "%.9g" % scale]
    say("case C host program", shape, causal)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    say(r.stdout.strip())
    assert r.returncode == 0, r.stderr
    o = _bf16(str(tmp_path / "o.bin"), shape)
    lse = torch.from_numpy(np.fromfile(str(tmp_path / "lse.bin"), dtype=np.float32).reshape(shape[:3]))
    o_ref, l_ref = oracle.fwd(q, k, v, scale, causal)
    check_fwd(o, lse, o_ref, l_ref, "C host program forward")
    refs = oracle.bwd(q, k, v, do, scale, causal)
    for name, r_ in zip(("dq", "dk", "dv"), refs):
        g = _bf16(str(tmp_path / (name + ".bin")), shape)
        check_grad(g, r_, "C host program " + name)
