"""Helpers shared by the GPU tests: bit-exact host<->device transfers."""
import sys

import numpy as np


def say(*a):
    """Name the case about to run on the GPU, flushed (a fault may end the process)."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def torch_dtype(dtype):
    import torch
    return torch.float16 if dtype == "f16" else torch.bfloat16


def to_dev(bits, dtype, device="cuda:0"):
    import torch
    if bits is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch_dtype(dtype)).to(device)


def to_bits(t):
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def empty(shape, dtype, device="cuda:0", fill_bits=None):
    import torch
    t = torch.empty(shape, dtype=torch_dtype(dtype), device=device)
    if fill_bits is not None:
        t.view(torch.int16).fill_(np.int16(np.uint16(fill_bits).view(np.int16)))
    return t
