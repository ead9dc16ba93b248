"""Canary-padded device buffers for write-outside-bounds checks.

A `Padded` buffer is one allocation holding a guard region, the tensor the kernel is given (a
contiguous view), and a second guard region.  Every byte starts as CANARY.  After the call the
guard regions must still hold it (no store before the first or past the last element of the
output), and no element of the view may still hold it (every element the call owns was written:
a store that went to the wrong place would otherwise leave a hole).
"""

import math

import torch

CANARY = 0xA5
GUARD_BYTES = 64 * 1024


class Padded:
    def __init__(self, shape, dtype, device="cuda", guard_bytes=GUARD_BYTES):
        esize = torch.empty((), dtype=dtype).element_size()
        assert guard_bytes % esize == 0
        self.pad = guard_bytes // esize
        self.numel = math.prod(shape)
        self.guard_bytes = guard_bytes
        self.buf = torch.empty(self.numel + 2 * self.pad, dtype=dtype, device=device)
        self.buf.view(torch.uint8).fill_(CANARY)
        self.t = self.buf[self.pad:self.pad + self.numel].view(shape)

    def guards_intact(self) -> bool:
        b = self.buf.view(torch.uint8)
        head = b[:self.guard_bytes]
        tail = b[self.guard_bytes + self.numel * self.buf.element_size():]
        return bool((head == CANARY).all().item()) and bool((tail == CANARY).all().item())

    def untouched(self):
        """Boolean mask (same shape as the view) of elements whose bytes all still hold the canary."""
        esize = self.buf.element_size()
        b = self.t.contiguous().view(torch.uint8).view(*self.t.shape, esize)
        return (b == CANARY).all(dim=-1)


def padded(shape, dtype, device="cuda"):
    return Padded(tuple(shape), dtype, device)


def padded_workspace(nbytes, dtype=torch.uint8, device="cuda"):
    """A workspace of at least `nbytes` bytes with guard regions around it."""
    esize = torch.empty((), dtype=dtype).element_size()
    return Padded((max(1, -(-nbytes // esize)),), dtype, device)
