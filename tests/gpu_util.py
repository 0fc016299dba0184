"""Host <-> device helpers for the GPU tests (numpy arrays in, torch out)."""

import numpy as np
import torch

DEV = "cuda"


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def dev_bf16(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(DEV)


def dev_of(a, dtype):
    return dev_bf16(a) if dtype == "bf16" else dev_f32(a)


def host_of(t):
    """float32 array, or uint16 bits for a bfloat16 tensor."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def empty(N, dtype):
    return torch.empty(N, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device=DEV)
