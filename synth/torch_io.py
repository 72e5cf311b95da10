"""Moves seeded storage arrays (bf16 bit patterns as uint16, or fp32) to and from torch tensors."""
import numpy as np


def to_dev(arr, dtype, device="cuda"):
    import torch
    a = np.ascontiguousarray(arr)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def to_host(t, dtype):
    import torch
    if dtype == "bf16":
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.float().cpu().numpy()
