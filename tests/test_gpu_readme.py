"""The usage example in README.md runs as written on the GPU, and its results
hold what the example's comments say."""
import os
import re

import pytest
import torch

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_example_runs(gpu_lib):
    text = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```python\n(.*?)```", text, re.S)
    assert len(blocks) == 1
    env = {}
    exec(compile(blocks[0].replace("plan.close()", ""), "README.md", "exec"), env)
    torch.cuda.synchronize()
    plan, specs, starts, V, S = env["plan"], env["specs"], env["starts"], env["V"], env["S"]
    gathered, params, packed, grads = env["gathered"], env["params"], env["packed"], env["grads"]
    # the norm was unpacked bit for bit (wq was overwritten by the gather side)
    s1 = starts[1]
    assert torch.equal(params[1].reshape(-1).view(torch.int16), gathered[s1:s1 + 4096].view(torch.int16))
    # pack: g * fl32(1/64) is exact for a power of two, and padding is +0.0
    for g, s in zip(grads, starts):
        assert torch.equal(packed[s:s + g.numel()], g.reshape(-1) / 64)
    covered = torch.zeros(V * S, dtype=torch.bool, device="cuda")
    for g, s in zip(grads, starts):
        covered[s:s + g.numel()] = True
    assert bool((packed[~covered].view(torch.int32) == 0).all())
    # the gather side rebuilt wq within E4M3 rounding of the gathered weights
    x = gathered[starts[0]:starts[0] + 4096 * 4096].float().reshape(4096, 4096)
    y = params[0].float()
    assert bool(((y - x).abs() <= x.abs() * 2.0 ** -4 * 1.01 + x.abs() * 2.0 ** -8 + 2.0 ** -9 * 1.01).all())
    plan.close()
