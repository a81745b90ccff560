"""Grouped RaggedShard layout plan, from the definitions on the pages.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Notation ([walk], the paragraph that states the planner as packing): tensors
T_1..T_N with n_i elements share one buffer of V*S elements; rank k owns
[kS, (k+1)S). Tensor i occupies the contiguous interval [s_i, s_i + n_i);
intervals are disjoint and lie inside [0, V*S); padding lives only in the
gaps. Where a rank boundary kS falls strictly inside T_i, its offset kS - s_i
must be a multiple of the atomic block size g_i. The objective is the
smallest S.

Readings where the pages are silent or garbled (each is listed in the design
notes):
  * g_i per block kind: ELEM 1, ROWS(k) k*cols, TILE(br, bc) br*cols (a tile
    of a row-major tensor stays whole only when cuts fall on br-row bands),
    FLAT(b) b, WHOLE n_i, TILEMAJOR(br, bc) br*bc (the tensor is stored tile
    by tile, each tile contiguous, so a cut may fall between any two tiles;
    the tiles must cover the tensor exactly). The block count is
    ceil(n_i / g_i); the last block may be partial.
  * Alignment: S and every s_i are multiples of an alignment a that the
    pages leave to the collective (16 elements here, a parameter).
  * Orders ([walk], the planner's tensor-order paragraph; [summary],
    Method): caller order, block size descending, shape descending (element
    count, then rows), each stable.
  * Search over S: for each order, the smallest feasible multiple of a that
    is at least the lower bound LB. The pages binary-search over aligned
    candidates on the claim that feasibility is monotone there; that claim
    does not hold in general (a multiple of the alignment of one prefix can
    be infeasible between two feasible ones), so this oracle scans every
    aligned candidate in increasing order. The result is the exact minimum
    per order.
  * Choice among orders: smallest S, then the smallest end max(s_i + n_i),
    then the order listed first.
  * Feasibility for a fixed order and S ([walk], the candidate-size
    paragraph): the pages' DP f(i, j) counts the shards needed to place the
    tensors before T_i and the first j blocks of T_i. Because T_i is
    contiguous, its placement is decided by s_i alone, and the constraint on
    s_i does not depend on the other tensors; so placing each tensor at its
    earliest valid start after the previous end gives every f(i, j) its
    minimum at once. ``earliest_starts`` finds that start shard by shard.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Sequence

import numpy as np

ALIGN = 16


def numel(spec) -> int:
    return int(spec.rows) * int(spec.cols)


def granularity(spec) -> int:
    """Flat size g of one atomic block ([walk], RaggedShard paragraph on the forbidden cut)."""
    n = numel(spec)
    k = spec.kind
    if k == "ELEM":
        return 1
    if k == "ROWS":
        return int(spec.p0) * int(spec.cols)
    if k == "TILE":
        return int(spec.p0) * int(spec.cols)
    if k == "FLAT":
        return int(spec.p0)
    if k == "WHOLE":
        return n
    if k == "TILEMAJOR":
        return int(spec.p0) * int(spec.p1)
    raise ValueError(f"unknown block kind {k!r}")


def layout_offsets(spec) -> np.ndarray:
    """Offset inside the tensor's interval of each element, in row-major element order.

    Row-major for every kind but TILEMAJOR, whose element (r, c) lives in tile
    (r // br, c // bc), tiles in row-major order, each tile row-major inside."""
    r, c = int(spec.rows), int(spec.cols)
    if spec.kind != "TILEMAJOR":
        return np.arange(r * c, dtype=np.int64)
    br, bc = int(spec.p0), int(spec.p1)
    rr = np.arange(r, dtype=np.int64)[:, None]
    cc = np.arange(c, dtype=np.int64)[None, :]
    tile = (rr // br) * (c // bc) + cc // bc
    return (tile * (br * bc) + (rr % br) * bc + cc % bc).ravel()


def atomic_blocks(spec) -> List[tuple]:
    """Flat [begin, end) of every atomic block of a tensor; the last may be partial."""
    n, g = numel(spec), granularity(spec)
    return [(j * g, min((j + 1) * g, n)) for j in range(-(-n // g))]


def align_up(x, a):
    return -(-x // a) * a


def lower_bound(specs, V: int, a: int = ALIGN) -> int:
    """LB: no shard can be smaller than the average load or the largest atomic block."""
    total = sum(numel(s) for s in specs)
    biggest = max(min(granularity(s), numel(s)) for s in specs)
    return align_up(max(-(-total // V), biggest), a)


def start_is_valid(s: int, n: int, g: int, S: int, a: int) -> bool:
    """The boundary condition for one tensor, straight from its definition."""
    if s % a:
        return False
    k = s // S + 1
    while k * S < s + n:
        if (k * S - s) % g:
            return False
        k += 1
    return True


def check_plan(specs, V: int, S: int, starts: Sequence[int], a: int = ALIGN) -> List[str]:
    """Every violated constraint of a plan ([walk], packing-problem paragraph); empty if valid."""
    bad = []
    if S <= 0 or S % a:
        bad.append(f"S={S} not a positive multiple of {a}")
        return bad
    iv = []
    for i, (spec, s) in enumerate(zip(specs, starts)):
        n, g = numel(spec), granularity(spec)
        if s < 0 or s + n > V * S:
            bad.append(f"tensor {i}: [{s},{s + n}) outside [0,{V * S})")
        if s % a:
            bad.append(f"tensor {i}: start {s} not a multiple of {a}")
        elif not start_is_valid(s, n, g, S, a):
            bad.append(f"tensor {i}: a rank boundary cuts an atomic block")
        iv.append((s, s + n, i))
    iv.sort()
    for (b0, e0, i0), (b1, e1, i1) in zip(iv, iv[1:]):
        if b1 < e0:
            bad.append(f"tensors {i0} and {i1} overlap")
    return bad


def earliest_starts(e, n: int, g: int, S, a: int, V: int) -> np.ndarray:
    """Smallest valid start s >= e of a tensor (n elements, block size g) for each
    (e, S) pair; -1 where none fits inside [0, V*S).

    Shard by shard from the one holding e: inside shard k the candidates are the
    aligned s in [max(e, kS), (k+1)S). Either the tensor ends by the boundary
    b = (k+1)S (then the first aligned candidate is the answer), or b falls
    inside it; then b - s must be a multiple of g and, since s and b are
    multiples of a, s = b (mod lcm(a, g)); the smallest such s is taken. Any
    further boundary b + S, b + 2S, ... inside the tensor lies S further on, so
    it is legal only when S is a multiple of g; otherwise no start in this
    shard works and the search moves to shard k + 1.
    """
    e = np.atleast_1d(np.asarray(e, dtype=np.int64)).copy()
    S = np.broadcast_to(np.asarray(S, dtype=np.int64), e.shape).copy()
    L = a * g // math.gcd(a, g)
    out = np.full(e.shape, -1, dtype=np.int64)
    k = e // S
    active = k < V
    while active.any():
        idx = np.nonzero(active)[0]
        kk, ee, SS = k[idx], e[idx], S[idx]
        lo = np.maximum(ee, kk * SS)
        b = (kk + 1) * SS
        s_a = align_up(lo, a)
        ok_a = s_a + n <= b
        s_b = b - L * ((b - lo) // L)
        ok_b = (~ok_a) & (s_b < b) & ((s_b + n <= b + SS) | (SS % g == 0))
        s = np.where(ok_a, s_a, s_b)
        done = ok_a | ok_b
        fits = done & (s + n <= V * SS)
        out[idx[fits]] = s[fits]
        k[idx[~done]] += 1
        active[idx[done]] = False
        active[idx[~done]] = k[idx[~done]] < V
    return out


def place(specs, order: Sequence[int], S, a: int, V: int) -> np.ndarray:
    """Greedy placement in the given order for each candidate S.

    Returns starts[len(S), N] in spec order, with -1 rows where S is infeasible.
    """
    S = np.atleast_1d(np.asarray(S, dtype=np.int64))
    starts = np.full((S.size, len(specs)), -1, dtype=np.int64)
    e = np.zeros(S.size, dtype=np.int64)
    ok = np.ones(S.size, dtype=bool)
    for i in order:
        n, g = numel(specs[i]), granularity(specs[i])
        s = np.full(S.size, -1, dtype=np.int64)
        if ok.any():
            s[ok] = earliest_starts(e[ok], n, g, S[ok], a, V)
        ok &= s >= 0
        starts[:, i] = np.where(ok, s, -1)
        e = np.where(ok, s + n, e)
    starts[~ok] = -1
    return starts


ORDER_NAMES = ("default", "by_block_size", "by_shape")


def orders(specs) -> List[List[int]]:
    """The three tensor orders the pages test, each a stable sort."""
    idx = list(range(len(specs)))
    by_block = sorted(idx, key=lambda i: -granularity(specs[i]))
    by_shape = sorted(idx, key=lambda i: (-numel(specs[i]), -int(specs[i].rows)))
    return [idx, by_block, by_shape]


def min_feasible_S(specs, order, V: int, a: int, lb: int):
    """Smallest feasible multiple of a that is >= lb, scanning every candidate."""
    S_max = align_up(sum(align_up(numel(s), a) for s in specs), a)  # one shard holds all
    S_max = max(S_max, lb)
    lo = lb
    batch = 4096
    while lo <= S_max:
        cand = lo + a * np.arange(batch, dtype=np.int64)
        cand = cand[cand <= S_max]
        st = place(specs, order, cand, a, V)
        feas = np.nonzero(st[:, 0] >= 0)[0] if len(specs) else np.array([0])
        if feas.size:
            j = feas[0]
            return int(cand[j]), st[j].copy()
        lo = int(cand[-1]) + a
        batch = min(batch * 2, 1 << 16)
    raise AssertionError("a single shard holding every tensor is always feasible")


@dataclass
class Plan:
    S: int
    starts: np.ndarray        # per tensor, in spec order
    order: List[int]          # placement order
    order_name: str
    V: int
    align: int
    LB: int
    numels: List[int]

    @property
    def end(self) -> int:
        return max(int(s) + n for s, n in zip(self.starts, self.numels))

    @property
    def R_used(self) -> int:
        return -(-self.end // self.S)


POLICIES = ("best",) + ORDER_NAMES


def plan(specs, V: int, a: int = ALIGN, policy: str = "best") -> Plan:
    """Plan S and the starts ([walk], planner paragraphs; [summary], Method (2)).

    policy "best" tries the three orders and keeps the best plan; "default",
    "by_block_size" or "by_shape" plans with that one order (the planner
    padding study compares them)."""
    if V < 1 or not specs:
        raise ValueError("need V >= 1 and at least one tensor")
    if policy not in POLICIES:
        raise ValueError(f"unknown order policy {policy!r}")
    lb = lower_bound(specs, V, a)
    ns = [numel(s) for s in specs]
    best = None
    cand_orders = list(enumerate(orders(specs)))
    if policy != "best":
        cand_orders = [cand_orders[ORDER_NAMES.index(policy)]]
    for oi, order in cand_orders:
        S, starts = min_feasible_S(specs, order, V, a, lb)
        end = max(int(s) + n for s, n in zip(starts, ns))
        key = (S, end, oi)
        if best is None or key < best[0]:
            best = (key, S, starts, order, oi)
    _, S, starts, order, oi = best
    return Plan(S, starts, list(order), ORDER_NAMES[oi], V, a, lb, ns)


def padding_ranges(specs, starts, S: int, R_mat: int) -> List[tuple]:
    """[begin, end) ranges of the materialised buffer [0, R_mat*S) not covered by a tensor."""
    iv = sorted((int(s), int(s) + numel(sp)) for sp, s in zip(specs, starts))
    out, pos, top = [], 0, R_mat * S
    for b, e in iv:
        b, e = min(b, top), min(e, top)
        if b > pos:
            out.append((pos, b))
        pos = max(pos, e)
    if pos < top:
        out.append((pos, top))
    return out
