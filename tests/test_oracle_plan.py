"""Pins of the oracle planner against brute force and closed forms.

The brute force here never uses the oracle's block size g: a start is valid
when every atomic block, enumerated from its meaning (k whole rows, the
br-row band that holds a row of br x bc tiles, b flat elements, the whole
tensor), maps to a single rank. That every br x bc tile then stays whole is
checked separately, as a consequence.
"""
import itertools
import math
import random

import numpy as np
import pytest

from oracle import plan as P
from workloads import TensorSpec, workload


# ---------------------------------------------------------------- brute force

def semantic_blocks(spec):
    """Lists of flat offsets (first, last) of every atomic block, from the block's meaning."""
    r, c, k = spec.rows, spec.cols, spec.kind
    if k == "ELEM":
        return [(e, e) for e in range(r * c)]
    if k == "ROWS":
        return [(r0 * c, min(r0 + spec.p0, r) * c - 1) for r0 in range(0, r, spec.p0)]
    if k == "TILE":   # the atomic RaggedShard block is the br-row band
        return [(r0 * c, min(r0 + spec.p0, r) * c - 1) for r0 in range(0, r, spec.p0)]
    if k == "FLAT":
        n = r * c
        return [(e, min(e + spec.p0, n) - 1) for e in range(0, n, spec.p0)]
    if k == "WHOLE":
        return [(0, r * c - 1)]
    raise ValueError(k)


def tiles(spec):
    """(top-left, bottom-right) flat offsets of every br x bc tile of a TILE tensor."""
    r, c = spec.rows, spec.cols
    out = []
    for r0 in range(0, r, spec.p0):
        for c0 in range(0, c, spec.p1):
            r1, c1 = min(r0 + spec.p0, r) - 1, min(c0 + spec.p1, c) - 1
            out.append((r0 * c + c0, r1 * c + c1))
    return out


def semantic_valid(s, spec, S):
    """Every block lies in one rank: rank of its first and last position agree."""
    return all((s + f) // S == (s + l) // S for f, l in semantic_blocks(spec))


def brute_earliest(e, spec, S, a, V):
    n = spec.rows * spec.cols
    s = -(-e // a) * a
    while s + n <= V * S:
        if semantic_valid(s, spec, S):
            return s
        s += a
    return -1


def brute_place(specs, order, S, a, V):
    e, starts = 0, [None] * len(specs)
    for i in order:
        s = brute_earliest(e, specs[i], S, a, V)
        if s < 0:
            return None
        starts[i] = s
        e = s + specs[i].rows * specs[i].cols
    return starts


def brute_min_S(specs, order, V, a):
    S = a
    while True:
        if brute_place(specs, order, S, a, V) is not None:
            return S
        S += a


def random_spec(rng: random.Random, name="t"):
    r, c = rng.randint(1, 7), rng.randint(1, 7)
    kind = rng.choice(["ELEM", "ROWS", "TILE", "FLAT", "WHOLE"])
    if kind == "ROWS":
        return TensorSpec(name, r, c, kind, rng.randint(1, 3))
    if kind == "TILE":
        return TensorSpec(name, r, c, kind, rng.randint(1, 4), rng.randint(1, 4))
    if kind == "FLAT":
        return TensorSpec(name, r, c, kind, rng.randint(1, 9))
    return TensorSpec(name, r, c, kind)


def random_instance(seed):
    rng = random.Random(seed)
    specs = [random_spec(rng, f"t{i}") for i in range(rng.randint(1, 4))]
    return specs, rng.randint(1, 5), rng.choice([1, 2, 4])


# ---------------------------------------------------------------- tests

def test_granularity_closed_forms():
    assert P.granularity(TensorSpec("a", 64, 48, "ROWS", 1)) == 48
    assert P.granularity(TensorSpec("a", 64, 48, "ROWS", 3)) == 144
    assert P.granularity(TensorSpec("a", 100, 32, "TILE", 16, 16)) == 512
    assert P.granularity(TensorSpec("a", 7, 130, "ELEM")) == 1
    assert P.granularity(TensorSpec("a", 9, 9, "FLAT", 2048)) == 2048
    assert P.granularity(TensorSpec("a", 9, 9, "WHOLE")) == 81
    assert P.atomic_blocks(TensorSpec("a", 5, 2, "ROWS", 2)) == [(0, 4), (4, 8), (8, 10)]


@pytest.mark.parametrize("seed", range(60))
def test_start_validity_matches_semantic_definition(seed):
    rng = random.Random(1000 + seed)
    spec = random_spec(rng)
    a = rng.choice([1, 2, 4])
    S = a * rng.randint(1, 12)
    for s in range(0, 6 * S, a):
        assert P.start_is_valid(s, spec.rows * spec.cols, P.granularity(spec), S, a) == \
            semantic_valid(s, spec, S), (spec, S, s, a)


@pytest.mark.parametrize("seed", range(60))
def test_earliest_start_matches_scan(seed):
    rng = random.Random(2000 + seed)
    spec = random_spec(rng)
    a = rng.choice([1, 2, 4, 8])
    V = rng.randint(1, 6)
    n, g = spec.rows * spec.cols, P.granularity(spec)
    Ss = np.array([a * rng.randint(1, 14) for _ in range(40)], dtype=np.int64)
    es = np.array([rng.randint(0, int(S) * V) for S in Ss], dtype=np.int64)
    got = P.earliest_starts(es, n, g, Ss, a, V)
    want = [brute_earliest(int(e), spec, int(S), a, V) for e, S in zip(es, Ss)]
    assert list(got) == want


@pytest.mark.parametrize("seed", range(50))
def test_min_S_per_order_matches_scan_from_the_alignment(seed):
    specs, V, a = random_instance(seed)
    lb = P.lower_bound(specs, V, a)
    for order in P.orders(specs):
        S, starts = P.min_feasible_S(specs, order, V, a, lb)
        assert S == brute_min_S(specs, order, V, a)
        assert list(starts) == brute_place(specs, order, S, a, V)
        assert P.check_plan(specs, V, S, starts, a) == []


@pytest.mark.parametrize("seed", range(40))
def test_valid_plans_never_cut_a_tile(seed):
    specs, V, a = random_instance(800 + seed)
    p = P.plan(specs, V, a)
    for spec, s in zip(specs, p.starts):
        if spec.kind == "TILE":
            assert all((int(s) + f) // p.S == (int(s) + l) // p.S for f, l in tiles(spec))


@pytest.mark.parametrize("seed", range(40))
def test_plan_within_twice_the_optimum_over_all_orders(seed):
    """The pages call the planner a 2-approximation; check against every permutation."""
    specs, V, a = random_instance(500 + seed)
    p = P.plan(specs, V, a)
    opt = min(brute_min_S(specs, list(perm), V, a) for perm in itertools.permutations(range(len(specs))))
    assert opt <= p.S <= 2 * opt
    assert p.S >= P.lower_bound(specs, V, a) >= 1


def test_the_three_orders_by_hand():
    """Default: the caller's order. By block size: g descending, ties in caller order. By shape:
    element count descending, then rows descending, ties in caller order."""
    specs = [TensorSpec("a", 8, 4, "ROWS", 1),      # g 4,  n 32, rows 8
             TensorSpec("b", 4, 8, "ROWS", 2),      # g 16, n 32, rows 4
             TensorSpec("c", 2, 2, "WHOLE"),        # g 4,  n 4
             TensorSpec("d", 1, 64, "FLAT", 16),    # g 16, n 64, rows 1
             TensorSpec("e", 32, 1, "ELEM")]        # g 1,  n 32, rows 32
    default, by_block, by_shape = P.orders(specs)
    assert default == [0, 1, 2, 3, 4]
    assert by_block == [1, 3, 0, 2, 4]
    assert by_shape == [3, 4, 0, 1, 2]


@pytest.mark.parametrize("seed", range(30))
def test_single_order_policies_against_brute_force(seed):
    """Each single-order policy gives the smallest S its order admits (brute force over S and
    starts), and "best" is the least of the three (ties: the smaller end, then the order
    listed first)."""
    specs, V, a = random_instance(3000 + seed)
    per = {}
    for k, name in enumerate(P.ORDER_NAMES):
        p = P.plan(specs, V, a, name)
        order = P.orders(specs)[k]
        assert p.order_name == name and p.order == order
        assert p.S == brute_min_S(specs, order, V, a)
        assert list(p.starts) == brute_place(specs, order, p.S, a, V)
        per[name] = p
    best = P.plan(specs, V, a, "best")
    want = min(P.ORDER_NAMES, key=lambda nm: (per[nm].S, per[nm].end, P.ORDER_NAMES.index(nm)))
    assert (best.S, best.order_name, list(best.starts)) == (per[want].S, want, list(per[want].starts))
    with pytest.raises(ValueError):
        P.plan(specs, V, a, "by_name")


def test_check_plan_catches_planted_errors():
    specs = [TensorSpec("a", 4, 4, "ROWS", 1), TensorSpec("b", 2, 8, "TILE", 2, 4)]
    V, S, a = 4, 16, 4
    good = [0, 16]
    assert P.check_plan(specs, V, S, good, a) == []
    assert P.check_plan(specs, V, S, [0, 8], a)          # overlap
    assert P.check_plan(specs, V, S, [0, 20], a)         # cuts the 2x4 tile band
    assert P.check_plan(specs, V, S, [2, 16], a)         # misaligned
    assert P.check_plan(specs, V, S, [0, 56], a)         # outside V*S
    assert P.check_plan(specs, V, 10, good, a)           # S not aligned


def _cfg_specs(i):
    return workload(i).specs


@pytest.mark.parametrize("idx", range(5))
def test_workload_plans_valid_and_balanced(idx):
    w = workload(idx)
    p = P.plan(w.specs, w.V)
    assert P.check_plan(w.specs, w.V, p.S, p.starts) == []
    # per-rank load is within 2x of the ideal balanced load
    assert p.S <= 2 * p.LB
    # every atomic block owned by exactly one rank (first and last element agree)
    for spec, s in zip(w.specs, p.starts):
        n, g = spec.rows * spec.cols, P.granularity(spec)
        first = int(s) + np.arange(0, n, g, dtype=np.int64)
        last = np.minimum(first + g, int(s) + n) - 1
        assert np.all(first // p.S == last // p.S)
        if spec.kind == "TILE":   # tile corners: top-left and bottom-right share a rank
            t = tiles(spec)
            for f, l in t[:: max(1, len(t) // 300)]:
                assert (int(s) + f) // p.S == (int(s) + l) // p.S


def test_tiny_workload_hand_derivation():
    """Worked by hand: the block-size order puts the 100x32 tensor (16-row bands, g=512) first.

    S=1920: starting it at 0 puts boundary 1920 at offset 1920 = 3*512+384, a cut; the
    largest start below 1920 congruent to 1920 mod 512 is 384, and its end 3584 is before
    the next boundary 3840. The 64x48 tensor (g=48) from 3584: boundary 3840 at offset 256
    is a cut; 3840 - 48*5 = 3600 works and 1920 % 48 == 0 keeps boundary 5760 legal too;
    it ends at 6672, where the 7x130 tensor (g=1) goes and ends at 7582 <= 4*1920.
    """
    w = workload(0)
    p = P.plan(w.specs, w.V)
    assert p.S == 1920 and p.order_name == "by_block_size"
    assert list(p.starts) == [3600, 384, 6672]
    assert p.R_used == 4
    specs = w.specs
    opt = min(brute_min_S(specs, list(perm), w.V, 16) for perm in itertools.permutations(range(3)))
    assert p.S <= 2 * opt


def test_llama8b_plan_closed_form():
    """gate/up/down exceed 2S, so S must be a multiple of their 128-row bands
    (128*4096 and 128*14336); the smallest common multiple is above the average load."""
    w = workload(1)
    p = P.plan(w.specs, w.V)
    band_a, band_b = 128 * 4096, 128 * 14336
    lcm = band_a * band_b // math.gcd(band_a, band_b)
    avg = -(-sum(s.rows * s.cols for s in w.specs) // w.V)
    assert lcm >= avg and lcm < 2 * avg
    assert p.S == lcm == 3670016
    assert p.LB == 3408000


def test_llama70b_whole_matrix_plan_closed_form():
    """With whole-matrix blocks S >= the largest matrix (28672*8192), which is already above
    the average load, and S = that size is feasible: four ranks hold the matrices."""
    w = workload(2)
    p = P.plan(w.specs, w.V)
    assert p.S == 28672 * 8192
    assert p.R_used == 4


def test_planted_tile_granularity_mistake_is_caught(monkeypatch):
    """Using the tile area instead of the row band as g would let ranks cut tiles."""
    orig = P.granularity

    def area(spec):
        if spec.kind == "TILE":
            return spec.p0 * spec.p1
        return orig(spec)

    monkeypatch.setattr(P, "granularity", area)
    specs = [TensorSpec("a", 6, 6, "TILE", 2, 2), TensorSpec("b", 5, 3, "ELEM")]
    p = P.plan(specs, 3, 1)
    assert any((int(s) + f) // p.S != (int(s) + l) // p.S
               for f, l in tiles(specs[0]) for s in [p.starts[0]])


def test_padding_ranges():
    specs = [TensorSpec("a", 2, 3, "ELEM"), TensorSpec("b", 1, 4, "ELEM")]
    assert P.padding_ranges(specs, [4, 16], 8, 3) == [(0, 4), (10, 16), (20, 24)]
    assert P.padding_ranges(specs, [0, 6], 5, 2) == []
