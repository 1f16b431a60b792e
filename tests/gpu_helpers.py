"""Shared helpers of the GPU parity tests (host <-> device marshalling only)."""
import numpy as np
import pytest
import torch

needs_gpu = [pytest.mark.gpu,
             pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def bits(t):
    """uint16 bit patterns of a bf16 tensor, on the host."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f32(t):
    return t.detach().contiguous().cpu().numpy()


def release():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
