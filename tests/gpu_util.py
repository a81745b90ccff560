"""Helpers for GPU tests: seeded workload inputs on the device (from
``workloads.device``) and canary-guarded output buffers."""
from __future__ import annotations

import torch

from workloads.device import (  # noqa: F401  (re-exported for the tests)
    POISON_BF16, POISON_F32, Inputs, garbage, tensor_bits, to_device_bits)


def guarded(n: int, dtype, device, guard_bytes: int = 4096, byte: int = 0xCD):
    """(whole, body): body is n elements with guard_bytes of canary after it."""
    esz = torch.empty((), dtype=dtype).element_size()
    g = (guard_bytes + esz - 1) // esz
    whole = torch.full(((n + g) * esz,), byte, dtype=torch.uint8, device=device).view(dtype)
    return whole, whole[:n]


def guard_intact(whole: torch.Tensor, n: int, byte: int = 0xCD) -> bool:
    tail = whole[n:].contiguous().view(torch.uint8)
    return bool((tail == byte).all().item())
