"""HIP path vs the CPU oracle on seeded random groups: every block kind mixed in
one group, shapes with ragged tiles, flat blocks and tails, rank counts 1-64,
both parameter dtypes, and sometimes only the ranks that hold data
materialised. Each group goes through the whole check of the parity suite
(unpack, pack with and without accumulation and in place, quant and dequant
in the three code formats, 1-byte unpack, the fused gather side, with 2
vectors per thread on odd seeds and the plan's own choice, 4 for groups this
small, on even ones), and two chained 8-bit Adam steps run on it."""
import random

import pytest
import torch

from tests.test_gpu_parity import _full_check
from workloads import TensorSpec

pytestmark = pytest.mark.gpu


def random_group(seed):
    rng = random.Random(9000 + seed)
    specs = []
    for i in range(rng.randint(1, 8)):
        kind = rng.choice(["ELEM", "ROWS", "TILE", "TILE", "FLAT", "FLAT", "WHOLE", "TILEMAJOR"])
        if kind == "TILEMAJOR":
            br, bc = rng.choice([(8, 8), (16, 16), (4, 64), (32, 32), (16, 3), (2, 128)])
            specs.append(TensorSpec(f"t{i}", br * rng.randint(1, 5), bc * rng.randint(1, 5), kind, br, bc))
            continue
        r = rng.choice([1, 2, 7, 31, 64, 100, 129, 257, 600])
        c = rng.choice([1, 3, 16, 20, 48, 130, 256, 1000])
        p0 = p1 = 0
        if kind == "ROWS":
            p0 = rng.choice([1, 2, 5, 16])
        elif kind == "TILE":
            p0, p1 = rng.choice([1, 4, 16, 32, 128]), rng.choice([1, 6, 16, 64, 128])
        elif kind == "FLAT":
            p0 = rng.choice([1, 100, 256, 2048, 5000])
        # at most 2000 quantisation blocks per tensor, so that the oracle's per-block
        # loops stay within seconds
        while kind == "TILE" and -(-r // p0) * -(-c // p1) > 2000:
            p0, p1 = 2 * p0, 2 * p1
        while kind == "FLAT" and -(-(r * c) // p0) > 2000:
            p0 *= 2
        specs.append(TensorSpec(f"t{i}", r, c, kind, p0, p1))
    V = rng.choice([1, 2, 3, 4, 7, 8, 16, 64])
    pdtype = rng.choice([torch.float32, torch.bfloat16])
    only_used = rng.random() < 0.3
    return specs, V, pdtype, only_used


@pytest.mark.parametrize("seed", range(48))
def test_random_group(gpu_lib, seed, monkeypatch):
    import structure_aware_grouped_amd as rs
    if seed % 2:
        monkeypatch.setenv("RS_GATHER_VEC", "2")
    specs, V, pdtype, only_used = random_group(seed)
    R_mat = None
    if only_used:
        S, starts, _, _ = rs.rs_plan_build(specs, V)
        R_mat = -(-max(s + sp.numel for s, sp in zip(starts, specs)) // S)
    print(f"seed {seed}: V={V} {pdtype} R_mat={R_mat} specs={specs}", flush=True)
    _full_check(rs, specs, V, pdtype, 300 + seed, R_mat=R_mat)


@pytest.mark.parametrize("seed", range(16))
def test_adam_steps_on_a_random_group(gpu_lib, seed):
    """Two chained rs_adam8_step calls; params, codes and scales bit for bit after each."""
    import numpy as np
    from oracle import adam as OA, transform as OT
    from tests.gpu_util import tensor_bits
    from tests.test_gpu_adam import HYPERS, _run
    import structure_aware_grouped_amd as rs
    specs, V, _, only_used = random_group(seed)
    S, starts, _, _ = rs.rs_plan_build(specs, V)
    R = -(-max(s + sp.numel for s, sp in zip(starts, specs)) // S) if only_used else V
    print(f"seed {seed}: V={V} R_mat={R} specs={specs}", flush=True)
    plan = rs.rs_plan_load(specs, V, S, starts, R, 0)
    rng = np.random.default_rng(600 + seed)
    total = R * S
    param = rng.standard_normal(total).astype(np.float32)
    m = (rng.standard_normal(total) * 1e-3).astype(np.float32)
    v = ((rng.standard_normal(total) * 1e-3) ** 2).astype(np.float32)
    qm, sm = OT.block_quant(m, specs, starts, S, R, "i8")
    qv, sv = OT.block_quant(v, specs, starts, S, R, "u8")
    for h in HYPERS[:2]:
        grad = (rng.standard_normal(total) * 1e-3).astype(np.float32)
        want = OA.adam8_step(param, grad, qm, sm, qv, sv, specs, starts, h)
        got = _run(rs, plan, (param, grad, qm, sm, qv.astype(np.uint8), sv), h)
        for g, wv, name in zip(got, want, ("param", "q_m", "s_m", "q_v", "s_v")):
            assert np.array_equal(tensor_bits(g), np.asarray(wv).view(tensor_bits(g).dtype)), (name, h.step)
        param, qm, sm, qv, sv = want
    plan.close()
