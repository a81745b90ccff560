"""rs_adam8_step against the oracle: chained steps on small groups (every
output bit for bit after every step) and sampled blocks of the Adam-state
workload at full size."""
import random

import numpy as np
import pytest
import torch

from oracle import adam as OA, plan as OP, transform as OT
from tests.gpu_util import tensor_bits
from tests.test_gpu_parity import BIG_BLOCKS, MID, RAGGED
from workloads import TensorSpec, workload
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
HYPERS = [OA.AdamHyper(1e-3, 0.9, 0.999, 1e-8, 0.01, 1), OA.AdamHyper(3e-4, 0.95, 0.98, 1e-6, 0.1, 17),
          OA.AdamHyper(1e-2, 0.8, 0.9999, 1e-8, 0.0, 1000)]


def _run(rs, plan, state, h):
    param, grad, qm, sm, qv, sv = (torch.from_numpy(x).to(DEV) for x in state)
    rs.rs_adam8_step(plan, param, grad, qm, sm, qv, sv, h.lr, h.beta1, h.beta2, h.eps, h.weight_decay, h.step)
    torch.cuda.synchronize()
    return param, qm, sm, qv, sv


@pytest.mark.parametrize("V", [1, 4])
def test_chained_steps_on_a_ragged_group(gpu_lib, V):
    import structure_aware_grouped_amd as rs
    specs = RAGGED + [TensorSpec("tile32", 64, 96, "TILE", 32, 32),
                      TensorSpec("tm32", 64, 96, "TILEMAJOR", 32, 32)]
    S, starts, _, _ = rs.rs_plan_build(specs, V)
    plan = rs.rs_plan_load(specs, V, S, starts, V, 0)
    rng = np.random.default_rng(V)
    total = V * S
    param = rng.standard_normal(total).astype(np.float32)
    m = (rng.standard_normal(total) * 1e-3).astype(np.float32)
    v = ((rng.standard_normal(total) * 1e-3) ** 2).astype(np.float32)
    qm, sm = OT.block_quant(m, specs, starts, S, V, "i8")
    qv, sv = OT.block_quant(v, specs, starts, S, V, "u8")
    for h in HYPERS:
        grad = (rng.standard_normal(total) * 1e-3).astype(np.float32)
        want = OA.adam8_step(param, grad, qm, sm, qv, sv, specs, starts, h)
        got = _run(rs, plan, (param, grad, qm, sm, qv.astype(np.uint8), sv), h)
        for g, wv, name in zip(got, want, ("param", "q_m", "s_m", "q_v", "s_v")):
            assert np.array_equal(tensor_bits(g), np.asarray(wv).view(tensor_bits(g).dtype)), (name, h.step)
        param, qm, sm, qv, sv = want
    plan.close()


@pytest.mark.parametrize("max_grid", [None, "16"])
def test_two_steps_on_the_mid_size_group(gpu_lib, max_grid, monkeypatch):
    """More than 32 tiles, so the XCD-grouped tile order runs whole rounds and a tail;
    with RS_MAX_GRID=16 every workgroup also loops over many blocks."""
    import structure_aware_grouped_amd as rs
    if max_grid:
        monkeypatch.setenv("RS_MAX_GRID", max_grid)
    specs, V = MID, 7
    S, starts, _, _ = rs.rs_plan_build(specs, V)
    plan = rs.rs_plan_load(specs, V, S, starts, V, 0)
    rng = np.random.default_rng(7)
    total = V * S
    param = rng.standard_normal(total).astype(np.float32)
    m = (rng.standard_normal(total) * 1e-3).astype(np.float32)
    v = ((rng.standard_normal(total) * 1e-3) ** 2).astype(np.float32)
    qm, sm = OT.block_quant(m, specs, starts, S, V, "i8")
    qv, sv = OT.block_quant(v, specs, starts, S, V, "u8")
    for h in HYPERS[:2]:
        grad = (rng.standard_normal(total) * 1e-3).astype(np.float32)
        want = OA.adam8_step(param, grad, qm, sm, qv, sv, specs, starts, h)
        got = _run(rs, plan, (param, grad, qm, sm, qv.astype(np.uint8), sv), h)
        for g, wv, name in zip(got, want, ("param", "q_m", "s_m", "q_v", "s_v")):
            assert np.array_equal(tensor_bits(g), np.asarray(wv).view(tensor_bits(g).dtype)), (name, h.step)
        param, qm, sm, qv, sv = want
    plan.close()


def test_steps_on_blocks_beyond_the_register_paths(gpu_lib):
    """Tiles of 32768 elements and 6000-element flat blocks take the two-pass path."""
    import structure_aware_grouped_amd as rs
    specs, V = BIG_BLOCKS, 3
    S, starts, _, _ = rs.rs_plan_build(specs, V)
    plan = rs.rs_plan_load(specs, V, S, starts, V, 0)
    rng = np.random.default_rng(11)
    total = V * S
    param = rng.standard_normal(total).astype(np.float32)
    m = (rng.standard_normal(total) * 1e-3).astype(np.float32)
    v = ((rng.standard_normal(total) * 1e-3) ** 2).astype(np.float32)
    qm, sm = OT.block_quant(m, specs, starts, S, V, "i8")
    qv, sv = OT.block_quant(v, specs, starts, S, V, "u8")
    for h in HYPERS:
        grad = (rng.standard_normal(total) * 1e-3).astype(np.float32)
        want = OA.adam8_step(param, grad, qm, sm, qv, sv, specs, starts, h)
        got = _run(rs, plan, (param, grad, qm, sm, qv.astype(np.uint8), sv), h)
        for g, wv, name in zip(got, want, ("param", "q_m", "s_m", "q_v", "s_v")):
            assert np.array_equal(tensor_bits(g), np.asarray(wv).view(tensor_bits(g).dtype)), (name, h.step)
        param, qm, sm, qv, sv = want
    plan.close()


# groups whose largest tile picks each register path of the tile step: 32x32 tiles (strips of four
# side by side through LDS, else one wave a tile; the pages' 8-bit Adam blocks), 64x64 (one 256-thread workgroup a tile), 128x128 (1024
# threads a tile); each with ragged edge tiles, tiles whose width is not a multiple of 4 (the
# two-pass path inside the same launch), a tile-major tensor, flat blocks and a row tensor
TILE_PATHS = {
    # every group of four 32x32 tiles a 32 x 128 strip: the strip-only launch
    "32x32 strips": [TensorSpec("s256", 64, 256, "TILE", 32, 32), TensorSpec("s128", 96, 128, "TILE", 32, 32),
                     TensorSpec("flat", 1, 5000, "FLAT", 2048), TensorSpec("norm", 300, 1, "ROWS", 1)],
    "32x32": [TensorSpec("t32", 256, 320, "TILE", 32, 32), TensorSpec("t32_ragged", 100, 70, "TILE", 32, 32),
              TensorSpec("t32_odd", 40, 45, "TILE", 32, 32), TensorSpec("tm16", 32, 64, "TILEMAJOR", 16, 16),
              TensorSpec("flat", 1, 5000, "FLAT", 2048), TensorSpec("norm", 300, 1, "ROWS", 1)],
    "64x64": [TensorSpec("t64", 256, 320, "TILE", 64, 64), TensorSpec("t32", 64, 96, "TILE", 32, 32),
              TensorSpec("t64_ragged", 130, 150, "TILE", 64, 64), TensorSpec("flat", 1, 5000, "FLAT", 2048)],
    "128x128": [TensorSpec("t128", 384, 512, "TILE", 128, 128), TensorSpec("t128_ragged", 300, 400, "TILE", 128, 128),
                TensorSpec("t128_odd", 130, 131, "TILE", 128, 128), TensorSpec("t32", 64, 96, "TILE", 32, 32),
                TensorSpec("tm64", 128, 128, "TILEMAJOR", 64, 64), TensorSpec("flat", 1, 3000, "FLAT", 1024)],
}


@pytest.mark.parametrize("max_grid", [None, "8"])
@pytest.mark.parametrize("paths", sorted(TILE_PATHS))
def test_chained_steps_on_each_tile_register_path(gpu_lib, paths, max_grid, monkeypatch):
    import structure_aware_grouped_amd as rs
    if max_grid:
        monkeypatch.setenv("RS_MAX_GRID", max_grid)
    specs, V = TILE_PATHS[paths], 3
    S, starts, _, _ = rs.rs_plan_build(specs, V)
    plan = rs.rs_plan_load(specs, V, S, starts, V, 0)
    rng = np.random.default_rng(len(paths))
    total = V * S
    param = rng.standard_normal(total).astype(np.float32)
    m = (rng.standard_normal(total) * 1e-3).astype(np.float32)
    v = ((rng.standard_normal(total) * 1e-3) ** 2).astype(np.float32)
    qm, sm = OT.block_quant(m, specs, starts, S, V, "i8")
    qv, sv = OT.block_quant(v, specs, starts, S, V, "u8")
    for h in HYPERS:
        grad = (rng.standard_normal(total) * 1e-3).astype(np.float32)
        want = OA.adam8_step(param, grad, qm, sm, qv, sv, specs, starts, h)
        got = _run(rs, plan, (param, grad, qm, sm, qv.astype(np.uint8), sv), h)
        for g, wv, name in zip(got, want, ("param", "q_m", "s_m", "q_v", "s_v")):
            assert np.array_equal(tensor_bits(g), np.asarray(wv).view(tensor_bits(g).dtype)), (paths, name, h.step)
        param, qm, sm, qv, sv = want
    plan.close()


def test_nan_gradients_blank_their_blocks(gpu_lib):
    """NaN gradients in flat blocks, 32x32 strips and a ragged 32x32 tensor: two chained steps
    against the oracle. Codes and scales bit for bit (a blanked block's scale is 0x7FC00000);
    parameters bit for bit where finite and NaN where the oracle's are NaN."""
    import structure_aware_grouped_amd as rs
    specs = [TensorSpec("s", 64, 256, "TILE", 32, 32), TensorSpec("r", 40, 45, "TILE", 32, 32),
             TensorSpec("f", 1, 5000, "FLAT", 2048)]
    V = 2
    S, starts, _, _ = rs.rs_plan_build(specs, V)
    plan = rs.rs_plan_load(specs, V, S, starts, V, 0)
    rng = np.random.default_rng(77)
    total = V * S
    param = rng.standard_normal(total).astype(np.float32)
    m = (rng.standard_normal(total) * 1e-3).astype(np.float32)
    v = ((rng.standard_normal(total) * 1e-3) ** 2).astype(np.float32)
    qm, sm = OT.block_quant(m, specs, starts, S, V, "i8")
    qv, sv = OT.block_quant(v, specs, starts, S, V, "u8")
    for step, h in enumerate(HYPERS[:2]):
        grad = (rng.standard_normal(total) * 1e-3).astype(np.float32)
        if step == 0:
            for i, e in ((0, 5), (0, 300 * 1 + 70), (1, 1000), (2, 4100)):
                grad[int(starts[i]) + e] = np.nan
        with np.errstate(invalid="ignore"):
            want = OA.adam8_step(param, grad, qm, sm, qv, sv, specs, starts, h)
        got = _run(rs, plan, (param, grad, qm, sm, qv.astype(np.uint8), sv), h)
        gp = got[0].cpu().numpy()
        nan = np.isnan(want[0])
        assert nan.any() and np.array_equal(np.isnan(gp), nan), step
        assert np.array_equal(gp[~nan].view(np.uint32), want[0][~nan].view(np.uint32)), step
        for g, wv, name in zip(got[1:], want[1:], ("q_m", "s_m", "q_v", "s_v")):
            assert np.array_equal(tensor_bits(g), np.asarray(wv).view(tensor_bits(g).dtype)), (name, step)
        param, qm, sm, qv, sv = want
    plan.close()


def test_zero_state_and_gradient_blocks(gpu_lib):
    import structure_aware_grouped_amd as rs
    specs = [TensorSpec("f", 1, 4096, "FLAT", 1024)]
    plan = rs.rs_plan_load(specs, 1, 4096, [0], 1, 0)
    param = np.random.default_rng(0).standard_normal(4096).astype(np.float32)
    grad = np.zeros(4096, np.float32)
    grad[2048:] = 1e-3
    qm = np.zeros(4096, np.uint8)
    qv = np.zeros(4096, np.uint8)
    sm = np.ones(4, np.float32)
    sv = np.ones(4, np.float32)
    h = HYPERS[0]
    want = OA.adam8_step(param, grad, qm, sm, qv, sv, specs, [0], h)
    got = _run(rs, plan, (param, grad, qm, sm, qv, sv), h)
    for g, wv in zip(got, want):
        assert np.array_equal(tensor_bits(g), np.asarray(wv).view(tensor_bits(g).dtype))
    plan.close()


@pytest.mark.parametrize("blocks", ["flat2048", "tile32"])
def test_adam_workload_sampled_blocks(gpu_lib, blocks):
    """One step on the full Adam-state workload (2048-element flat blocks, or the pages'
    32x32 tiles at 32-row granularity); every element of 2000 sampled blocks (and the first
    and last block of every tensor) against the oracle."""
    import structure_aware_grouped_amd as rs
    w = workload(4) if blocks == "flat2048" else W.adam_tile32_variant(workload(4))
    specs = list(w.specs)
    S, starts, _, _ = rs.rs_plan_build(specs, w.V)
    R = w.V
    plan = rs.rs_plan_load(specs, w.V, S, starts, R, 0)
    total = R * S
    gen = torch.Generator(device="cpu").manual_seed(5)
    # packed buffers built from the seeded per-tensor states (placement by the plan's starts)
    def flat_from(fn):
        out = np.zeros(total, np.float32)
        for i, sp in enumerate(specs):
            out[starts[i]: starts[i] + sp.numel] = fn(i).ravel()
        return out
    param = flat_from(lambda i: W.tensor_values(w, i, W.Role.WEIGHT))
    grad = flat_from(lambda i: W.tensor_values(w, i, W.Role.GRAD))
    m = flat_from(lambda i: W.adam_state(w, i, "m"))
    v = flat_from(lambda i: W.adam_state(w, i, "v"))
    dp, dg, dm, dv = (torch.from_numpy(x).to(DEV) for x in (param, grad, m, v))
    qm = torch.empty(total, dtype=torch.uint8, device=DEV)
    qv = torch.empty(total, dtype=torch.uint8, device=DEV)
    sm = torch.empty(plan.n_qblocks, dtype=torch.float32, device=DEV)
    sv = torch.empty(plan.n_qblocks, dtype=torch.float32, device=DEV)
    rs.rs_block_quant(plan, dm, qm, "i8", sm)
    rs.rs_block_quant(plan, dv, qv, "u8", sv)
    torch.cuda.synchronize()
    qm0, sm0, qv0, sv0 = tensor_bits(qm), tensor_bits(sm).view(np.float32), tensor_bits(qv), tensor_bits(sv).view(np.float32)
    h = HYPERS[1]
    rs.rs_adam8_step(plan, dp, dg, qm, sm, qv, sv, h.lr, h.beta1, h.beta2, h.eps, h.weight_decay, h.step)
    torch.cuda.synchronize()
    gp, gqm, gsm, gqv, gsv = tensor_bits(dp).view(np.float32), tensor_bits(qm), tensor_bits(sm).view(np.float32), \
        tensor_bits(qv), tensor_bits(sv).view(np.float32)
    blocks = list(OT.quant_blocks(specs, starts))
    rnd = random.Random(7)
    firsts = {}
    for idx, (i, b, pos) in enumerate(blocks):
        firsts.setdefault(i, []).append(idx)
    pick = set(rnd.sample(range(len(blocks)), 2000))
    for lst in firsts.values():
        pick.update([lst[0], lst[-1]])
    k = OA.host_scalars(h)
    for idx in sorted(pick):
        i, b, pos = blocks[idx]
        m0 = OT.dequant_values(qm0[pos], sm0[b], "i8")
        v0 = OT.dequant_values(qv0[pos], sv0[b], "u8")
        p1, m1, v1 = OA.update_values(param[pos], grad[pos], m0, v0, k)
        assert np.array_equal(gp[pos], p1), idx
        c, s = OT.quantize_block(m1, "i8")
        assert np.array_equal(gqm[pos], c) and gsm[b] == s, idx
        c, s = OT.quantize_block(v1, "u8")
        assert np.array_equal(gqv[pos], c) and gsv[b] == s, idx
    for bgn, end in OP.padding_ranges(specs, starts, S, R):
        assert np.array_equal(gp[bgn:end], param[bgn:end])
    plan.close()
