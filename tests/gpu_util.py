"""Helpers shared by the GPU parity tests (no quantization arithmetic here)."""
import sys

import numpy as np
import torch


def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def u16(t):
    """torch fp16/int16 tensor -> numpy uint16 bit patterns (host)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_u16(a, device):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.float16)


def first_diff(a, b):
    a, b = np.asarray(a), np.asarray(b)
    idx = np.argwhere(a != b)
    if idx.size == 0:
        return None
    i = tuple(idx[0])
    return "first mismatch at %s: got %r expected %r (%d mismatches of %d)" % (
        i, a[i], b[i], len(idx), a.size)
