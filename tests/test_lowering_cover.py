"""The work lists rs_plan_load uploads, checked on the host element by element
(tests/cpp/lowering_cover.cpp, which includes plan.cpp): unpack writes every
tensor element once from its own flat position; pack writes every flat
position once, from its own tensor element or as padding; quant writes every
code once (blocks whole, zero ranges outside them) and every scale once; the
gather side writes every element of every quantised tensor once with its own
block's scale; tile-major strips map tile-by-tile positions to row-major
elements. Planted mistakes in the lists are reported."""
import os
import random
import shutil
import subprocess

import pytest

from oracle import plan as OP
from workloads import TensorSpec, adam_tile32_variant, tile_major_variant, workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "structure_aware_grouped_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
KINDS = {"ELEM": 0, "ROWS": 1, "TILE": 2, "FLAT": 3, "WHOLE": 4, "TILEMAJOR": 5}


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    gxx = shutil.which("g++")
    if not gxx or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("needs g++ and the HIP headers")
    out = str(tmp_path_factory.mktemp("cover") / "lowering_cover")
    cmd = [gxx, "-std=c++17", "-O2", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(ROOT, "tests", "cpp", "lowering_cover.cpp"),
           os.path.join(CSRC, "planner.cpp"), "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-pthread", "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def _run(exe, specs, V, R=None, plant=0):
    ref = OP.plan(specs, V)
    R = V if R is None else R
    lines = [f"{len(specs)} {V} {ref.S} {R}"] + [f"{s.rows} {s.cols} {KINDS[s.kind]} {s.p0} {s.p1} {int(st)}"
                                                 for s, st in zip(specs, ref.starts)]
    args = [exe] + ([str(plant)] if plant else [])
    r = subprocess.run(args, input="\n".join(lines) + "\n", capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr
    return r.stdout.strip().split("\n")[0]


def _gather_shape(exe, specs, V, vec=None, shape_only=False):
    """(runs, split8, split4, vectors per thread) of the gather side; vec forces the vector
    count through RS_GATHER_VEC; shape_only skips the element-by-element check."""
    ref = OP.plan(specs, V)
    lines = [f"{len(specs)} {V} {ref.S} {V}"] + [f"{s.rows} {s.cols} {KINDS[s.kind]} {s.p0} {s.p1} {int(st)}"
                                                 for s, st in zip(specs, ref.starts)]
    env = dict(os.environ)
    env.pop("RS_GATHER_VEC", None)
    if vec is not None:
        env["RS_GATHER_VEC"] = str(vec)
    r = subprocess.run([exe] + (["shape"] if shape_only else []), input="\n".join(lines) + "\n",
                       capture_output=True, text=True, timeout=600, env=env)
    out = r.stdout.split("\n")
    assert out[0] == "ok", r.stdout
    w = out[1].split()
    return int(w[2]), int(w[4]), int(w[6]), int(w[8])


def _adam_strips(exe, specs, V):
    ref = OP.plan(specs, V)
    lines = [f"{len(specs)} {V} {ref.S} {V}"] + [f"{s.rows} {s.cols} {KINDS[s.kind]} {s.p0} {s.p1} {int(st)}"
                                                 for s, st in zip(specs, ref.starts)]
    r = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, timeout=600)
    out = r.stdout.split("\n")
    assert out[0] == "ok", r.stdout
    return out[2] == "adam strips 1"


def test_adam_strip_launch_follows_the_tensors(exe):
    # the check inside compares the lowering's flag with the tensor shapes on every
    # plan this file runs; here both values it can take on
    assert _adam_strips(exe, list(adam_tile32_variant(workload(4)).specs), 64)
    assert not _adam_strips(exe, list(workload(4).specs), 64)          # flat blocks only
    assert not _adam_strips(exe, list(workload(1).specs), 64)          # 128x128 tiles
    assert not _adam_strips(exe, [TensorSpec("a", 64, 256, "TILE", 32, 32),
                                  TensorSpec("b", 64, 96, "TILE", 32, 32)], 2)   # 3 tiles per band
    assert not _adam_strips(exe, [TensorSpec("a", 64, 256, "TILE", 32, 32),
                                  TensorSpec("b", 40, 128, "TILE", 32, 32)], 2)  # a partial band
    assert _adam_strips(exe, [TensorSpec("a", 64, 256, "TILE", 32, 32), TensorSpec("b", 96, 128, "TILE", 32, 32),
                              TensorSpec("c", 5000, 1, "FLAT", 2048), TensorSpec("d", 300, 1, "ROWS", 1)], 3)


@pytest.mark.parametrize("idx,tm", [(0, False), (1, False), (1, True), (2, False), (4, False)])
def test_workload_lists(exe, idx, tm):
    w = workload(idx)
    if tm:
        w = tile_major_variant(w)
    R = None if w.materialize_all_ranks else OP.plan(w.specs, w.V).R_used
    assert _run(exe, list(w.specs), w.V, R) == "ok"


def _random_group(rng):
    specs = []
    for i in range(rng.randint(1, 7)):
        kind = rng.choice(["ROWS", "TILE", "TILE", "FLAT", "WHOLE", "ELEM", "TILEMAJOR"])
        if kind == "TILEMAJOR":
            br, bc = rng.choice([(16, 16), (2, 8192), (4, 64), (16, 3), (32, 32)])
            specs.append(TensorSpec(f"t{i}", br * rng.randint(1, 3), bc * rng.randint(1, 3), kind, br, bc))
            continue
        r, c = rng.randint(1, 600), rng.choice([1, 3, 16, 130, 256, 1000])
        p0 = rng.choice([1, 3, 16, 128]) if kind in ("ROWS", "TILE") else (rng.choice([1, 7, 64, 2048, 5000])
                                                                         if kind == "FLAT" else 0)
        p1 = rng.choice([1, 5, 16, 64, 128]) if kind == "TILE" else 0
        specs.append(TensorSpec(f"t{i}", r, c, kind, p0, p1))
    return specs


@pytest.mark.parametrize("seed", range(30))
def test_random_group_lists(exe, seed):
    rng = random.Random(9000 + seed)
    specs = _random_group(rng)
    V = rng.choice([1, 2, 3, 5, 8, 16, 64])
    R = OP.plan(specs, V).R_used if seed % 3 == 0 else None
    assert _run(exe, specs, V, R) == "ok"


@pytest.mark.parametrize("seed", range(12))
def test_groups_of_32x32_tiles(exe, seed):
    # the pages' 8-bit Adam blocks: whole strips or not, by width and band; the coverage check and
    # the strip-launch check (against the tensor shapes) run on every one
    rng = random.Random(7000 + seed)
    specs = []
    for i in range(rng.randint(1, 5)):
        rows = 32 * rng.randint(1, 6) - (rng.choice([0, 0, 0, 7]))
        cols = rng.choice([128, 256, 384, 96, 160, 32 * rng.randint(1, 12)])
        specs.append(TensorSpec(f"t{i}", rows, cols, "TILE", 32, 32))
    if rng.random() < 0.5:
        specs.append(TensorSpec("norm", 300, 1, rng.choice(["ROWS", "FLAT"]), rng.choice([1, 2048])))
    V = rng.choice([1, 2, 3, 8])
    assert _run(exe, specs, V) == "ok"


def test_gather_runs_and_strips_of_a_mid_size_group(exe):
    specs = [TensorSpec("a", 1024, 2048, "TILE", 128, 128), TensorSpec("b", 300, 1000, "TILE", 64, 64),
             TensorSpec("c", 300001, 1, "FLAT", 2048), TensorSpec("d", 256, 512, "TILEMAJOR", 32, 32),
             TensorSpec("e", 64, 4096, "ROWS", 1), TensorSpec("f", 5000, 1, "ELEM")]
    assert _run(exe, specs, 7) == "ok"


@pytest.mark.parametrize("plant", [1, 2, 3, 4])
def test_planted_mistakes_are_reported(exe, plant):
    specs = [TensorSpec("a", 256, 512, "TILE", 128, 128), TensorSpec("c", 5000, 1, "FLAT", 2048),
             TensorSpec("d", 64, 64, "TILEMAJOR", 32, 32), TensorSpec("e", 100, 30, "ELEM")]
    out = _run(exe, specs, 4, plant=plant)
    assert out.startswith("FAIL"), out


def test_gather_runs_fill_their_workgroups(exe):
    # MoE-shaped experts (2880-wide rows, 128-row bands) with 2 vectors per thread (the long-launch
    # choice, forced), runs of 48 to 64 pieces of 1024 codes: the fewest workgroups come from 22-row
    # runs (63,360 codes, 62 pieces), five per band and one of the band's last 18 rows (the last
    # 64-row band of `down`: 22 + 22 + 20)
    specs = []
    for e in range(4):
        specs += [TensorSpec(f"e{e}.gate_up", 5760, 2880, "TILE", 128, 128),
                  TensorSpec(f"e{e}.down", 2880, 2880, "TILE", 128, 128)]
    runs, split8, split4, vec = _gather_shape(exe, specs, 8, vec=2)
    assert (split8, split4, vec) == (62, 124, 2)
    assert runs == 4 * (5760 // 128 * 6 + (2880 // 128 * 6 + 3))
    # 4 vectors per thread (pieces of 2048 codes): 43-row runs (123,840 codes, 61 pieces), three per
    # band (43 + 43 + 42; the last 64-row band of `down`: 43 + 21)
    runs, split8, split4, vec = _gather_shape(exe, specs, 8, vec=4)
    assert (split8, split4, vec) == (61, 121, 4)
    assert runs == 4 * (5760 // 128 * 3 + (2880 // 128 * 3 + 2))


def test_gather_vectors_per_thread_follow_the_launch_length(exe):
    # fewer than 2^29 elements in row runs: 4 vectors per thread; from 2^29 on: 2
    small = [TensorSpec(f"t{i}", 14336, 1024, "TILE", 128, 128) for i in range(4)]
    large = [TensorSpec(f"t{i}", 14336, 1024, "TILE", 128, 128) for i in range(37)]   # 543M elements
    assert sum(s.rows * s.cols for s in large) >= 1 << 29 > sum(s.rows * s.cols for s in large[:36])
    assert _gather_shape(exe, small, 8)[3] == 4
    assert _gather_shape(exe, large, 64, shape_only=True)[3] == 2
    assert _gather_shape(exe, large[:36], 64, shape_only=True)[3] == 4
    assert _gather_shape(exe, small, 8, vec=2)[3] == 2
