"""Copy synthetic host inputs into torch tensors (device memory plumbing only)."""
import numpy as np
import torch


def to_torch(arr, device="cuda"):
    """uint16 arrays are bf16 bit patterns -> torch.bfloat16; other arrays keep their dtype."""
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(arr)
    return t.to(device) if device is not None else t


def from_torch_bf16(t):
    """bf16 tensor -> uint16 bit patterns on the host."""
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
