"""The Python binding rejects tensors that the C ABI cannot check (it sees
plain pointers): wrong dtypes and tensors that are not on a GPU are refused
before any call into the library, so these run on the CPU."""
import pytest
import torch

import rmsnorm_fwd_amd as rn


def _cpu(T=4, H=64, dtype=torch.bfloat16):
    return torch.zeros(T, H, dtype=dtype)


def test_forward_needs_bfloat16_activations():
    for dt in (torch.float32, torch.float16):
        with pytest.raises(TypeError, match="x must be bfloat16"):
            rn.rmsnorm_fwd(_cpu(dtype=dt), torch.ones(64))


def test_forward_needs_gpu_tensors():
    with pytest.raises(ValueError, match="x must be a GPU tensor"):
        rn.rmsnorm_fwd(_cpu(), torch.ones(64))


def test_backward_needs_bfloat16_and_gpu():
    x = _cpu()
    with pytest.raises(TypeError, match="x must be bfloat16"):
        rn.rmsnorm_bwd(x, x.float(), torch.ones(4), torch.ones(64))
    with pytest.raises(ValueError, match="x must be a GPU tensor"):
        rn.rmsnorm_bwd(x, x, torch.ones(4), torch.ones(64))
    with pytest.raises(ValueError, match="x must be a GPU tensor"):
        rn.rmsnorm_bwd_routed(x, x, torch.ones(4), torch.ones(64), (rn.RMSN_FORM_PAIR, 1))


def test_gated_calls_check_too():
    x = _cpu()
    with pytest.raises(TypeError, match="x must be bfloat16"):
        rn.rmsnorm_gated_fwd(x.half(), x, torch.ones(64))
    with pytest.raises(ValueError, match="x must be a GPU tensor"):
        rn.rmsnorm_gated_bwd(x, x, x, torch.ones(4), torch.ones(64))


def test_workspace_init_needs_a_gpu_workspace():
    with pytest.raises(ValueError, match="workspace must be a GPU tensor"):
        rn.rmsnorm_bwd_workspace_init(torch.zeros(4096, dtype=torch.uint8), 64)
