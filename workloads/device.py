"""Seeded workload inputs placed in device memory (torch is the memory plumbing).

The values come from this package's seeded generators only; a buffer is
filled by writing each tensor's bits at the start the plan gives it, with a
recognisable NaN pattern everywhere else, so a kernel that reads padding
shows it. Nothing here computes any step of the layout transform; the
oracle regenerates whatever it checks from the same seeds.
"""
from __future__ import annotations

from typing import List

import numpy as np
import torch

from . import gen as W

POISON_BF16 = 0x7FC1          # a NaN pattern for padding of bf16 buffers
POISON_F32 = 0x7FC00001       # a NaN pattern for padding of fp32 buffers


def to_device_bits(bits: np.ndarray, torch_dtype, device) -> torch.Tensor:
    """Raw bit patterns (uint16 / uint32) -> a device tensor of the given dtype."""
    if bits.dtype == np.uint16:
        t = torch.from_numpy(bits.view(np.int16))
    else:
        t = torch.from_numpy(bits.view(np.int32))
    return t.to(device).view(torch_dtype)


def tensor_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy bit patterns (uint8 / uint16 / uint32)."""
    size = t.element_size()
    view = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[size]
    a = t.detach().contiguous().view(view).cpu().numpy()
    return a.view({1: np.uint8, 2: np.uint16, 4: np.uint32}[size])


class Inputs:
    """Device inputs of a workload for a given plan (S, starts, R_mat)."""

    def __init__(self, w, S: int, starts, R_mat: int, device="cuda:0"):
        self.w, self.S, self.starts, self.R = w, int(S), [int(s) for s in starts], int(R_mat)
        self.device = torch.device(device)
        self.pdtype = torch.bfloat16 if w.param_dtype == "bf16" else torch.float32

    # parameters -------------------------------------------------------
    def weight_bits(self, i: int) -> np.ndarray:
        return W.weight_bits(self.w, i).ravel()

    def gathered(self, arrange=None) -> torch.Tensor:
        """The all-gathered flat parameter buffer; padding holds a NaN pattern.

        ``arrange(i, bits)`` returns tensor i's row-major bits in the order of its
        interval in the buffer (default: row-major, every kind but TILEMAJOR)."""
        total = self.R * self.S
        fill = POISON_BF16 if self.pdtype == torch.bfloat16 else POISON_F32
        if self.pdtype == torch.bfloat16:
            G = torch.full((total,), fill, dtype=torch.int16, device=self.device).view(torch.bfloat16)
        else:
            G = torch.full((total,), fill, dtype=torch.int32, device=self.device).view(torch.float32)
        n_specs = len(self.w.specs)
        for lo in range(0, n_specs, 16):
            idx = list(range(lo, min(lo + 16, n_specs)))
            bits = W.parallel_map(self.weight_bits, idx)
            for i, b in zip(idx, bits):
                if arrange is not None:
                    b = arrange(i, b)
                s = self.starts[i]
                G[s: s + b.size].copy_(to_device_bits(np.ascontiguousarray(b), self.pdtype, self.device))
        return G

    def empty_params(self) -> List[torch.Tensor]:
        return [torch.empty(sp.rows, sp.cols, dtype=self.pdtype, device=self.device) for sp in self.w.specs]

    # gradients ---------------------------------------------------------
    def grad(self, i: int) -> np.ndarray:
        return W.tensor_values(self.w, i, W.Role.GRAD)

    def grads(self) -> List[torch.Tensor]:
        out = []
        n_specs = len(self.w.specs)
        for lo in range(0, n_specs, 16):
            idx = list(range(lo, min(lo + 16, n_specs)))
            vals = W.parallel_map(self.grad, idx)
            out.extend(torch.from_numpy(v).to(self.device) for v in vals)
        return out

    def prev_rank(self, k: int) -> np.ndarray:
        return W.prev_slice(self.w, k, self.S)

    def prev(self) -> torch.Tensor:
        P = torch.empty(self.R * self.S, dtype=torch.float32, device=self.device)
        for lo in range(0, self.R, 16):
            ks = list(range(lo, min(lo + 16, self.R)))
            vals = W.parallel_map(self.prev_rank, ks)
            for k, v in zip(ks, vals):
                P[k * self.S: (k + 1) * self.S].copy_(torch.from_numpy(v))
        return P

    def prev_range(self, b: int, e: int) -> np.ndarray:
        """prev[b:e] regenerated on the host."""
        parts = []
        for k in range(b // self.S, (e - 1) // self.S + 1):
            v = self.prev_rank(k)
            lo, hi = max(b, k * self.S) - k * self.S, min(e, (k + 1) * self.S) - k * self.S
            parts.append(v[lo:hi])
        return np.concatenate(parts)

    # Adam states -------------------------------------------------------
    def adam(self, i: int, which: str) -> np.ndarray:
        return W.adam_state(self.w, i, which)

    def adam_states(self, which: str) -> List[torch.Tensor]:
        return [torch.from_numpy(self.adam(i, which)).to(self.device) for i in range(len(self.w.specs))]


def garbage(n: int, dtype, device, byte: int = 0xA5) -> torch.Tensor:
    """A buffer of n elements filled with a recognisable byte pattern."""
    esz = torch.empty((), dtype=dtype).element_size()
    t = torch.full((n * esz,), byte, dtype=torch.uint8, device=device)
    return t.view(dtype)
