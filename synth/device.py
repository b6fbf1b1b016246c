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


def device_layer_weights(spec, seed, layer=0, device="cuda"):
    """Weights of one layer generated on the device, for timing runs whose size
    makes the host generator too slow (58 GB for 48 Qwen3-shaped layers).  Same
    law as ``layers.layer_weights`` (sigma * N(0, 1), rounded to the layer dtype),
    drawn from torch's seeded device generator, one stream per (seed, layer,
    tensor), one draw per tensor; not the host generator's values, so parity
    tests do not use them."""
    from . import lib
    from .layers import TAG_DOWN, TAG_GATE, TAG_UP
    dt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    out = []
    for tag, shape in ((TAG_GATE, (spec.N, spec.d_ff, spec.d)), (TAG_UP, (spec.N, spec.d_ff, spec.d)),
                       (TAG_DOWN, (spec.N, spec.d, spec.d_ff))):
        g = torch.Generator(device=device)
        g.manual_seed(lib.key_of(seed, layer, tag, 0xD) & ((1 << 63) - 1))
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32).mul_(spec.sigma).to(dt)
        out.append(t)
    return tuple(out)
