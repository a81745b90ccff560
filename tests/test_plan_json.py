"""Plans as data: a plan written by plan_to_json and read back by
plan_from_json has the same tensors, V, S, starts and materialised ranks, and
the oracle's validator accepts it (the GPU side of the round trip is in
test_gpu_parity.py)."""
import json

import pytest

from oracle import plan as OP
from workloads import tile_major_variant, workload


@pytest.mark.parametrize("idx,tm", [(0, False), (1, False), (1, True), (2, False), (3, False), (4, False)])
def test_round_trip(idx, tm):
    import structure_aware_grouped_amd as rs
    w = workload(idx)
    if tm:
        w = tile_major_variant(w)
    specs = list(w.specs)
    S, starts, _, _ = rs.rs_plan_build(specs, w.V)
    R = -(-max(s + sp.numel for s, sp in zip(starts, specs)) // S)
    text = rs.plan_to_json(specs, w.V, S, starts, R)
    specs2, V2, S2, starts2, R2 = rs.plan_from_json(text)
    assert (V2, S2, starts2, R2) == (w.V, S, starts, R)
    assert [(s.name, s.rows, s.cols, s.kind, s.p0, s.p1) for s in specs2] == \
           [(s.name, s.rows, s.cols, s.kind, s.p0, s.p1) for s in specs]
    assert OP.check_plan(specs2, V2, S2, starts2) == []
    assert rs.plan_to_json(specs2, V2, S2, starts2, R2) == text


def test_integer_kinds_and_default_ranks():
    import structure_aware_grouped_amd as rs
    spec = rs.PlanSpec("a", 32, 32, "TILE", 16, 16)
    text = rs.plan_to_json([spec._replace(kind=2)], 4, 256, [0])
    specs, V, S, starts, R = rs.plan_from_json(text)
    assert specs[0].kind == "TILE" and R == 4 and specs[0].numel == 1024


def test_rejects_other_formats():
    import structure_aware_grouped_amd as rs
    good = json.loads(rs.plan_to_json([rs.PlanSpec("a", 4, 4, "ELEM")], 2, 16, [0]))
    for change in ({"format": "rs-plan/0"}, {"starts": [0, 16]}):
        with pytest.raises(ValueError):
            rs.plan_from_json(json.dumps(dict(good, **change)))
    bad = dict(good, tensors=[dict(good["tensors"][0], kind="DIAGONAL")])
    with pytest.raises(ValueError):
        rs.plan_from_json(json.dumps(bad))
