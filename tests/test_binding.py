"""The Python binding rejects buffers the kernels cannot address: an L buffer
or workspace in host memory (or on another device) would hand a host address
to a GPU kernel.  The helper checks run on the CPU; the end-to-end checks need
a GPU tensor for q and are marked gpu (they launch nothing)."""
import pytest
import torch

import exact_io_aware_44_amd as fa

DEV = torch.device("cuda:0")


def test_lse_checks_on_host():
    ok = torch.empty(2, 3, 4)
    with pytest.raises(ValueError, match="lse must be on"):
        fa._check_lse(ok, (2, 3, 4), DEV)  # host tensor
    with pytest.raises(ValueError, match="float32"):
        fa._check_lse(torch.empty(2, 3, 4, dtype=torch.float64), (2, 3, 4), DEV)
    with pytest.raises(ValueError, match="float32"):
        fa._check_lse(torch.empty(2, 3, 5), (2, 3, 4), DEV)
    with pytest.raises(ValueError, match="float32"):
        fa._check_lse(torch.empty(4, 3, 2).permute(2, 1, 0), (2, 3, 4), DEV)  # not contiguous
    fa._check_lse(None, (2, 3, 4), DEV)  # no buffer: nothing to check


def test_workspace_checks_on_host():
    with pytest.raises(ValueError, match="workspace must be a GPU tensor"):
        fa._check_workspace(torch.empty(64, dtype=torch.uint8), DEV)
    fa._check_workspace(None, DEV)


def test_inputs_must_be_gpu_tensors():
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.fa_fwd(q, q, q)
    with pytest.raises(TypeError):
        fa.fa_fwd(q.float(), q, q)


@pytest.mark.gpu
def test_host_lse_and_workspace_rejected(gpu):
    q = torch.zeros(1, 2, 40, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="lse must be on"):
        gpu.fa_fwd(q, q, q, lse=torch.empty(1, 2, 40))
    with pytest.raises(ValueError, match="lse must be on"):
        gpu.fa_fwd_qk(q, q, q, lse=torch.empty(1, 2, 40))
    with pytest.raises(ValueError, match="workspace must be a GPU tensor"):
        gpu.fa_fwd_splitkv(q[:, :, :3].contiguous(), q, q, num_splits=2,
                           workspace=torch.empty(1 << 16, dtype=torch.uint8))
    qp = torch.zeros(2, 40, 64, dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, 40], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="lse must be on"):
        gpu.fa_fwd_varlen(qp, qp, qp, cu, 40, lse=torch.empty(2, 40))
    o, lse = gpu.fa_fwd(q, q, q)
    with pytest.raises(ValueError, match="lse must be on"):
        gpu.fa_bwd(q, q, q, o, lse.cpu(), q)
    with pytest.raises(ValueError, match="workspace must be a GPU tensor"):
        gpu.fa_bwd(q, q, q, o, lse, q, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    torch.cuda.synchronize()
