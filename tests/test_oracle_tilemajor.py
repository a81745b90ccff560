"""Pins of the tile-major layout in the oracle.

  * the layout is a permutation of the tensor's interval and every tile is a
    contiguous run of br*bc elements (brute force over tiles);
  * unpack(pack(x, 1, no accumulate)) == x through tile-major tensors;
  * the codes and scales of a tile-major tensor are those of the same tensor
    in the row-major tile layout, moved to the tile-major positions (the same
    values form each block, in another order);
  * brute-force planning with tile-sized blocks (every tile on one rank).
"""
import itertools
import random

import numpy as np
import pytest

from oracle import plan as P, transform as T
from workloads import TensorSpec


@pytest.mark.parametrize("r,c,br,bc", [(4, 6, 2, 3), (64, 96, 32, 32), (32, 12, 16, 3), (8, 8, 8, 8)])
def test_layout_is_a_permutation_with_contiguous_tiles(r, c, br, bc):
    spec = TensorSpec("t", r, c, "TILEMAJOR", br, bc)
    off = P.layout_offsets(spec)
    assert np.array_equal(np.sort(off), np.arange(r * c))
    grid = off.reshape(r, c)
    for tr in range(r // br):
        for tc in range(c // bc):
            tile = grid[tr * br:(tr + 1) * br, tc * bc:(tc + 1) * bc]
            first = (tr * (c // bc) + tc) * br * bc
            assert np.array_equal(tile.ravel(), np.arange(first, first + br * bc))


def test_pack_unpack_round_trip_through_tile_major():
    specs = [TensorSpec("a", 64, 96, "TILEMAJOR", 32, 32), TensorSpec("b", 10, 10, "ROWS", 1),
             TensorSpec("c", 32, 12, "TILEMAJOR", 16, 3)]
    p = P.plan(specs, 5)
    rng = np.random.default_rng(0)
    x = [rng.standard_normal((s.rows, s.cols)).astype(np.float32) for s in specs]
    flat = T.pack(x, None, specs, p.starts, p.S, 5, np.float32(1.0), False)
    for a, b in zip(x, T.unpack(flat, specs, p.starts)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    # and the flat buffer really is tile-major: tile (1, 2) of "a" is one run
    s = int(p.starts[0])
    assert np.array_equal(flat[s + (1 * 3 + 2) * 1024: s + (1 * 3 + 3) * 1024], x[0][32:64, 64:96].ravel())


@pytest.mark.parametrize("fmt", ["e4m3", "i8", "u8"])
def test_tile_major_quant_equals_row_major_tiles(fmt):
    rng = np.random.default_rng(2)
    r, c, br, bc = 96, 64, 32, 16
    x = rng.standard_normal((r, c)).astype(np.float32)
    if fmt == "u8":
        x = np.abs(x)
    tm, rm = TensorSpec("t", r, c, "TILEMAJOR", br, bc), TensorSpec("t", r, c, "TILE", br, bc)
    n = r * c
    q_rm, s_rm = T.block_quant(x.ravel(), [rm], [0], n, 1, fmt)
    flat_tm = np.zeros(n, np.float32)
    flat_tm[P.layout_offsets(tm)] = x.ravel()
    q_tm, s_tm = T.block_quant(flat_tm, [tm], [0], n, 1, fmt)
    assert np.array_equal(s_tm, s_rm)
    assert np.array_equal(q_tm[P.layout_offsets(tm)], q_rm)
    for out in ("f32", "bf16"):
        a = T.unpack_dequant(q_tm, s_tm, [tm], [0], fmt, out)[0]
        b = T.unpack_dequant(q_rm, s_rm, [rm], [0], fmt, out)[0]
        assert np.array_equal(a, b)


def _tm_valid(s, spec, S):
    tsz = spec.p0 * spec.p1
    return all((s + t * tsz) // S == (s + (t + 1) * tsz - 1) // S for t in range(spec.rows * spec.cols // tsz))


@pytest.mark.parametrize("seed", range(30))
def test_tile_major_plans_against_brute_force(seed):
    rng = random.Random(seed)
    specs = []
    for i in range(rng.randint(1, 3)):
        br, bc = rng.randint(1, 3), rng.randint(1, 3)
        specs.append(TensorSpec(f"t{i}", br * rng.randint(1, 3), bc * rng.randint(1, 3), "TILEMAJOR", br, bc))
    V, a = rng.randint(1, 4), rng.choice([1, 2])
    p = P.plan(specs, V, a)
    assert P.check_plan(specs, V, p.S, p.starts, a) == []
    for spec, s in zip(specs, p.starts):
        assert _tm_valid(int(s), spec, p.S)
    # brute force: smallest S over all orders where every tile stays on one rank
    best = None
    for perm in itertools.permutations(range(len(specs))):
        S = a
        while True:
            e, ok = 0, True
            for i in perm:
                n = specs[i].rows * specs[i].cols
                s = -(-e // a) * a
                while s + n <= V * S and not _tm_valid(s, specs[i], S):
                    s += a
                if s + n > V * S:
                    ok = False
                    break
                e = s + n
            if ok:
                break
            S += a
        best = S if best is None else min(best, S)
    assert best <= p.S <= 2 * best
