"""Helpers for the GPU tests: host <-> device copies of bf16 bit patterns and
guarded allocations (a sentinel band around every buffer, checked after the
call, so a write outside a buffer fails the test instead of passing)."""
import numpy as np

GUARD = 256  # elements of sentinel on each side


def dev():
    import torch
    return torch.device("cuda:0")


def up16(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(
        torch.bfloat16).to(dev())


def down16(t) -> np.ndarray:
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def down32(t) -> np.ndarray:
    return t.contiguous().cpu().numpy()


class Guarded:
    """A device buffer of n elements at element offset `offset` inside a larger
    allocation whose other elements hold a sentinel (all bits set)."""

    def __init__(self, n, dtype, offset=0, init=None):
        import torch
        self.n, self.offset, self.dtype = n, offset, dtype
        total = GUARD + offset + n + GUARD
        self.base = torch.empty(total, dtype=dtype, device=dev())
        ib = torch.int16 if dtype == torch.bfloat16 else torch.int32
        self.base.view(ib).fill_(-1)
        self.lo = GUARD + offset
        self.t = self.base[self.lo:self.lo + n]
        if init is not None:
            self.set(init)

    def set(self, host: np.ndarray):
        import torch
        if self.dtype == torch.bfloat16:
            self.t.copy_(up16(host))
        else:
            self.t.copy_(torch.from_numpy(np.ascontiguousarray(host, dtype=np.float32)).to(dev()))

    def get(self) -> np.ndarray:
        import torch
        return down16(self.t) if self.dtype == torch.bfloat16 else down32(self.t)

    def guards_intact(self) -> bool:
        import torch
        ib = torch.int16 if self.dtype == torch.bfloat16 else torch.int32
        b = self.base.view(ib)
        return bool((b[:self.lo] == -1).all()) and bool((b[self.lo + self.n:] == -1).all())

    def ptr(self) -> int:
        return self.t.data_ptr()


def bits(a: np.ndarray) -> np.ndarray:
    """Raw bits for bit-exact comparison of float32 or bf16 (uint16) arrays."""
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |v| (8 significant bits)."""
    a = np.abs(v.astype(np.float64))
    a = np.where(a == 0, 2.0 ** -133, a)
    return np.exp2(np.floor(np.log2(a)) - 7)
