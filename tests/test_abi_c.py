"""The C ABI from plain C: a C99 program (tests/c/plan_from_c.c) that includes
only include/rs.h is compiled with gcc, linked against the built library and
plans groups on the host. Its plans equal the oracle's, and its errors come
back as the documented status and message."""
import os
import random
import shutil
import subprocess

import pytest

from oracle import plan as OP
from workloads import TensorSpec, workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "structure_aware_grouped_amd")
KINDS = {"ELEM": 0, "ROWS": 1, "TILE": 2, "FLAT": 3, "WHOLE": 4, "TILEMAJOR": 5}
ORDER_KINDS = {"default": 0, "by_block_size": 1, "by_shape": 2}


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    if not os.path.exists(os.path.join(LIBDIR, "librs_hip.so")):
        pytest.fail("librs_hip.so is not built: run __graft_entry__.build()")
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    out = str(tmp_path_factory.mktemp("c") / "plan_from_c")
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "plan_from_c.c"), "-L", LIBDIR, "-lrs_hip",
           f"-Wl,-rpath,{LIBDIR}", "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return out


def _run(exe, specs, V):
    lines = [f"{len(specs)} {V}"] + [f"{s.rows} {s.cols} {KINDS[s.kind]} {s.p0} {s.p1}" for s in specs]
    res = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stderr
    return res.stdout.split("\n")


@pytest.mark.parametrize("idx", range(5))
def test_c_client_plans_the_workloads_like_the_oracle(exe, idx):
    w = workload(idx)
    out = _run(exe, list(w.specs), w.V)
    ref = OP.plan(w.specs, w.V)
    assert int(out[0]) == ref.S
    assert [int(x) for x in out[1].split()] == [int(s) for s in ref.starts]
    assert int(out[2]) == ORDER_KINDS[ref.order_name]


@pytest.mark.parametrize("seed", range(10))
def test_c_client_plans_random_groups_like_the_oracle(exe, seed):
    rng = random.Random(4242 + seed)
    specs = []
    for i in range(rng.randint(1, 9)):
        kind = rng.choice(["ROWS", "TILE", "FLAT", "WHOLE", "ELEM", "TILEMAJOR"])
        if kind == "TILEMAJOR":
            br, bc = rng.choice([(16, 16), (4, 64), (16, 3)])
            specs.append(TensorSpec(f"t{i}", br * rng.randint(1, 4), bc * rng.randint(1, 4), kind, br, bc))
            continue
        r, c = rng.choice([1, 7, 64, 300]), rng.choice([1, 16, 130, 256])
        p0 = rng.choice([1, 2, 16]) if kind in ("ROWS", "TILE") else (rng.choice([64, 100, 2048]) if kind == "FLAT" else 0)
        p1 = rng.choice([8, 16, 32]) if kind == "TILE" else 0
        specs.append(TensorSpec(f"t{i}", r, c, kind, p0, p1))
    V = rng.choice([1, 2, 3, 8, 64])
    out = _run(exe, specs, V)
    ref = OP.plan(specs, V)
    assert int(out[0]) == ref.S
    assert [int(x) for x in out[1].split()] == [int(s) for s in ref.starts]


def test_c_client_sees_status_and_message(exe):
    out = _run(exe, [TensorSpec("bad", 4, 4, "TILE", 0, 4)], 2)   # a TILE with br = 0
    word, status, message = out[0].split(" ", 2)
    assert word == "error" and int(status) == -1 and message.strip()
