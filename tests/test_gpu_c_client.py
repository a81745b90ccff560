"""The GPU path driven from plain C: tests/c/transform_from_c.c, compiled by gcc
against include/rs.h and the HIP runtime (hipMalloc / hipMemcpy, no torch), runs
unpack, pack and E4M3 block quant of a group in a child process. Its outputs
match the oracle bit for bit."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import plan as OP, transform as OT
from workloads import TensorSpec, workload

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "structure_aware_grouped_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
KINDS = {"ELEM": 0, "ROWS": 1, "TILE": 2, "FLAT": 3, "WHOLE": 4, "TILEMAJOR": 5}

GROUP = [
    TensorSpec("tile_partial", 37, 20, "TILE", 8, 6),
    TensorSpec("tile_vec", 130, 64, "TILE", 16, 16),
    TensorSpec("flat_tail", 1, 4099, "FLAT", 256),
    TensorSpec("elem", 7, 130, "ELEM"),
    TensorSpec("rows3", 10, 10, "ROWS", 3),
    TensorSpec("whole", 5, 5, "WHOLE"),
    TensorSpec("tm", 32, 64, "TILEMAJOR", 16, 32),
    TensorSpec("norm", 4096, 1, "ROWS", 1),
]


@pytest.fixture(scope="module")
def exe(tmp_path_factory, gpu_lib):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    out = str(tmp_path_factory.mktemp("cgpu") / "transform_from_c")
    cmd = [gcc, "-std=gnu99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "transform_from_c.c"), "-L", LIBDIR, "-lrs_hip",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{LIBDIR}", "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


@pytest.mark.parametrize("case", ["tiny", "ragged"])
def test_c_client_matches_the_oracle(exe, tmp_path, case):
    if case == "tiny":
        specs, V = list(workload(0).specs), 4
    else:
        specs, V = GROUP, 5
    ref = OP.plan(specs, V)
    S, starts, R = ref.S, [int(s) for s in ref.starts], V
    rng = np.random.default_rng(31 if case == "tiny" else 32)
    xs = [rng.uniform(-1, 1, sp.rows * sp.cols).astype(np.float32) for sp in specs]
    G = np.full(R * S, np.nan, dtype=np.float32)
    for x, s in zip(xs, starts):
        G[s: s + x.size] = x
    grads = [(rng.standard_normal(sp.rows * sp.cols) * 1e-3).astype(np.float32) for sp in specs]
    prev = (rng.standard_normal(R * S) * 1e-3).astype(np.float32)
    lines = [f"{len(specs)} {V} {S} {R}"] + [f"{sp.rows} {sp.cols} {KINDS[sp.kind]} {sp.p0} {sp.p1} {s}"
                                             for sp, s in zip(specs, starts)]
    (tmp_path / "plan.txt").write_text("\n".join(lines) + "\n")
    G.tofile(tmp_path / "gathered.f32")
    np.concatenate(grads).tofile(tmp_path / "grads.f32")
    prev.tofile(tmp_path / "prev.f32")
    print(f"C client, {case} group: S={S} R={R} tensors={len(specs)}", flush=True)
    r = subprocess.run([exe, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr[-2000:])

    got = np.fromfile(tmp_path / "unpacked.f32", dtype=np.uint32)
    want = np.concatenate([u.ravel() for u in OT.unpack(G.view(np.uint32), specs, starts)])
    assert np.array_equal(got, want)
    got = np.fromfile(tmp_path / "packed.f32", dtype=np.uint32)
    want = OT.pack([g.reshape(sp.rows, sp.cols) for g, sp in zip(grads, specs)], prev, specs, starts, S, R,
                   OT.inv_v(V), True)
    assert np.array_equal(got, want.view(np.uint32))
    wq, ws = OT.block_quant(G, specs, starts, S, R, "e4m3")
    assert np.array_equal(np.fromfile(tmp_path / "codes.u8", dtype=np.uint8), wq)
    assert np.array_equal(np.fromfile(tmp_path / "scales.f32", dtype=np.uint32), ws.view(np.uint32))
