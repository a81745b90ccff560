"""A dequant tile whose store offsets from the block's start would reach 2 GiB takes
the global store instead of the buffer store: one 2-row band of a 2^29-column
tensor, whose second row starts 2 GiB after the first. Sampled tiles (the first,
the last and random ones) are compared bit for bit with the oracle's values of
the same codes and scales. About 5 GiB of device memory. (The gather side's run
guard cannot be reached this way: the planner takes flat blocks of at most 2^24
elements and row runs hold at most 131,072, far below 2 GiB of output.)"""
import numpy as np
import pytest
import torch

from oracle import transform as OT
from workloads import TensorSpec

pytestmark = pytest.mark.gpu


def test_dequant_tile_spanning_2_gib(gpu_lib):
    import structure_aware_grouped_amd as rs
    cols = 1 << 29
    specs = [TensorSpec("wide", 2, cols, "TILE", 2, 128)]
    S, starts, _, _ = rs.rs_plan_build(specs, 1)
    plan = rs.rs_plan_load(specs, 1, S, starts, 1, 0)
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(5)
    q = torch.randint(0, 256, (plan.R_mat * plan.S,), dtype=torch.uint8, device=dev, generator=g)
    scales = torch.rand(plan.n_qblocks, dtype=torch.float32, device=dev, generator=g) + 0.25
    out = torch.full((plan.R_mat * plan.S,), float("nan"), dtype=torch.float32, device=dev)
    rs.rs_block_dequant(plan, q, "i8", scales, out)
    torch.cuda.synchronize()
    ntc = cols // 128
    tiles = [0, 1, ntc - 1] + [int(t) for t in np.random.default_rng(5).integers(0, ntc, 61)]
    s0 = int(starts[0])
    for t in tiles:
        for r in range(2):
            pos = s0 + r * cols + t * 128
            codes = q[pos:pos + 128].cpu().numpy()
            want = OT.dequant_values(codes, np.float32(scales[t].item()), "i8").astype(np.float32)
            got = out[pos:pos + 128].cpu().numpy()
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"tile {t} row {r}"
    del q, out, scales
    plan.close()
    torch.cuda.empty_cache()

