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


GUARD_BYTES = 4096
GUARD_BYTE = 0xA7


class Guarded:
    """Device buffers with sentinel bands (4 KiB of 0xA7 bytes) right before
    and after each: a kernel that writes past either end of an output changes
    a band, and check() fails. Buffers stay 16-byte aligned."""

    def __init__(self, device=None):
        self.d = device if device is not None else dev()
        self.items = []

    def empty(self, shape, dtype, fill=None):
        n = 1
        for s in shape:
            n *= int(s)
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        raw = torch.full((2 * GUARD_BYTES + (nbytes + 15) // 16 * 16,), GUARD_BYTE, dtype=torch.uint8,
                         device=self.d)
        t = raw[GUARD_BYTES:GUARD_BYTES + nbytes].view(dtype).view(tuple(int(s) for s in shape))
        if fill is not None:
            t.fill_(fill)
        self.items.append((raw, nbytes))
        return t

    def like(self, x, fill=None):
        t = self.empty(x.shape, x.dtype)
        if fill is None:
            t.copy_(x)
        else:
            t.fill_(fill)
        return t

    def check(self, what=""):
        torch.cuda.synchronize()
        for raw, nbytes in self.items:
            pre = raw[:GUARD_BYTES]
            post = raw[GUARD_BYTES + nbytes:]
            assert bool((pre == GUARD_BYTE).all()), (what, "band before a buffer was written")
            assert bool((post == GUARD_BYTE).all()), (what, "band after a buffer was written")
