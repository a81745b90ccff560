"""Seeded synthetic values.

Every array is drawn from NumPy's PCG64 with a SeedSequence keyed by
(base seed, workload index, role, item index), so any single tensor or rank
slice can be regenerated on its own (the oracle checks large workloads tensor
by tensor). bf16 values are obtained from fp32 by round-to-nearest-even on
the bit pattern. Nothing here knows about plans, scales or codes.
"""
from __future__ import annotations

import enum
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Callable, Iterable, List, Sequence

import numpy as np

BASE_SEED = 20260225


class Role(enum.IntEnum):
    WEIGHT = 0
    GRAD = 1
    PREV = 2
    ADAM_M = 3
    ADAM_V = 4
    EXTRA = 5


def seed_key(workload_index: int, role: int, item: int, base: int = BASE_SEED) -> np.random.Generator:
    ss = np.random.SeedSequence([base, int(workload_index), int(role), int(item)])
    return np.random.Generator(np.random.PCG64(ss))


def normal_f32(rng: np.random.Generator, n: int, sigma: float) -> np.ndarray:
    x = rng.standard_normal(n, dtype=np.float32)
    x *= np.float32(sigma)
    return x


def uniform_f32(rng: np.random.Generator, n: int, lo: float, hi: float) -> np.ndarray:
    x = rng.random(n, dtype=np.float32)
    x *= np.float32(hi - lo)
    x += np.float32(lo)
    return x


def draw(rng: np.random.Generator, n: int, dist) -> np.ndarray:
    if dist[0] == "normal":
        return normal_f32(rng, n, dist[1])
    if dist[0] == "uniform":
        return uniform_f32(rng, n, dist[1], dist[2])
    raise ValueError(f"unknown distribution {dist!r}")


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def tensor_values(w, i: int, role: Role) -> np.ndarray:
    """Values of tensor ``i`` of workload ``w`` for a role (weights or grads).

    Returns float32 of shape (rows, cols). For a bf16 parameter buffer the
    caller rounds weights with ``bf16_bits_from_f32``.
    """
    spec = w.specs[i]
    dist = w.weight_dist if role == Role.WEIGHT else w.grad_dist
    x = draw(seed_key(w.index, role, i), spec.numel, dist)
    return x.reshape(spec.rows, spec.cols)


def weight_bits(w, i: int) -> np.ndarray:
    """Weights of tensor ``i`` in the parameter dtype, as raw bits (uint16 bf16 or uint32 fp32)."""
    x = tensor_values(w, i, Role.WEIGHT)
    if w.param_dtype == "bf16":
        return bf16_bits_from_f32(x).reshape(x.shape)
    return x.view(np.uint32)


def prev_slice(w, rank: int, S: int) -> np.ndarray:
    """Previous packed-gradient values for one rank slice (S fp32 values, padding included)."""
    return draw(seed_key(w.index, Role.PREV, rank), S, w.prev_dist)


def adam_state(w, i: int, which: str) -> np.ndarray:
    """fp32 Adam state of tensor ``i``: m ~ N(0, sigma), v = (N(0, sigma))^2."""
    spec = w.specs[i]
    if which == "m":
        return normal_f32(seed_key(w.index, Role.ADAM_M, i), spec.numel, w.grad_dist[1]).reshape(
            spec.rows, spec.cols)
    if which == "v":
        g = normal_f32(seed_key(w.index, Role.ADAM_V, i), spec.numel, w.grad_dist[1])
        return (g * g).reshape(spec.rows, spec.cols)
    raise ValueError(which)


def worker_count() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def parallel_map(fn: Callable, items: Iterable, workers: int = 0) -> List:
    items = list(items)
    workers = workers or worker_count()
    if workers <= 1 or len(items) <= 1:
        return [fn(x) for x in items]
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))
