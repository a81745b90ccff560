"""The host planner and plan validation under AddressSanitizer and
UndefinedBehaviorSanitizer. planner.cpp and plan.cpp are compiled for the host
with g++ (no device code), linked with the plain C client of tests/c and run on
the five workloads, random groups, huge shapes near the 2^39-element limit and
bad specs. Every run must end cleanly, print the oracle's plan (or the
documented error), and leave no sanitizer report."""
import os
import random
import shutil
import subprocess

import pytest

from oracle import plan as OP
from workloads import TensorSpec, workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "structure_aware_grouped_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
KINDS = {"ELEM": 0, "ROWS": 1, "TILE": 2, "FLAT": 3, "WHOLE": 4, "TILEMAJOR": 5}
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=86",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=87")


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    gxx, gcc = shutil.which("g++"), shutil.which("gcc")
    if not gxx or not gcc or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("needs g++, gcc and the HIP headers")
    d = tmp_path_factory.mktemp("san")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), "-D__HIP_PLATFORM_AMD__"]
    objs = []
    for src in ("planner.cpp", "plan.cpp"):
        o = str(d / (src + ".o"))
        r = subprocess.run([gxx, "-std=c++17", *SAN, *inc, "-c", os.path.join(CSRC, src), "-o", o],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        objs.append(o)
    o = str(d / "client.o")
    r = subprocess.run([gcc, "-std=c99", *SAN, "-I", os.path.join(ROOT, "include"), "-c",
                        os.path.join(ROOT, "tests", "c", "plan_from_c.c"), "-o", o], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = str(d / "plan_san")
    libdir = os.path.join(ROCM, "lib")
    r = subprocess.run([gxx, *SAN, *objs, o, "-L", libdir, "-lamdhip64", f"-Wl,-rpath,{libdir}", "-pthread",
                        "-o", out], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def test_binary_is_instrumented(exe):
    r = subprocess.run(["ldd", exe], capture_output=True, text=True)
    assert "libasan" in r.stdout and "libubsan" in r.stdout, r.stdout


def _run(exe, specs, V):
    lines = [f"{len(specs)} {V}"] + [f"{s.rows} {s.cols} {KINDS[s.kind]} {s.p0} {s.p1}" for s in specs]
    r = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, timeout=600, env=ENV)
    assert r.returncode == 0 and "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    return r.stdout.split("\n")


def _same_as_oracle(out, specs, V):
    ref = OP.plan(specs, V)
    assert int(out[0]) == ref.S
    assert [int(x) for x in out[1].split()] == [int(s) for s in ref.starts]


@pytest.mark.parametrize("idx", range(5))
def test_workloads_under_sanitizers(exe, idx):
    w = workload(idx)
    _same_as_oracle(_run(exe, list(w.specs), w.V), w.specs, w.V)


def test_random_groups_under_sanitizers(exe):
    rng = random.Random(777)
    for _ in range(12):
        specs = []
        for i in range(rng.randint(1, 8)):
            kind = rng.choice(["ROWS", "TILE", "FLAT", "WHOLE", "ELEM", "TILEMAJOR"])
            if kind == "TILEMAJOR":
                br, bc = rng.choice([(16, 16), (4, 64), (32, 8)])
                specs.append(TensorSpec(f"t{i}", br * rng.randint(1, 5), bc * rng.randint(1, 5), kind, br, bc))
                continue
            r, c = rng.choice([1, 5, 64, 333]), rng.choice([1, 16, 130, 257])
            p0 = rng.choice([1, 3, 16]) if kind in ("ROWS", "TILE") else (rng.choice([7, 64, 2048]) if kind == "FLAT" else 0)
            p1 = rng.choice([1, 16, 40]) if kind == "TILE" else 0
            specs.append(TensorSpec(f"t{i}", r, c, kind, p0, p1))
        V = rng.choice([1, 2, 3, 7, 16, 100])
        _same_as_oracle(_run(exe, specs, V), specs, V)


def test_huge_shapes_under_sanitizers(exe):
    # sizes near the int64 paths: a 2^40-element whole matrix, and row bands of a 2^20 x 2^16 matrix
    specs = [TensorSpec("big", 1 << 20, 1 << 20, "WHOLE"), TensorSpec("band", 1 << 20, 1 << 16, "ROWS", 128),
             TensorSpec("norm", 1 << 16, 1, "ROWS", 1)]
    out = _run(exe, specs, 1024)
    S = int(out[0])
    starts = [int(x) for x in out[1].split()]
    assert OP.check_plan(specs, 1024, S, starts, 16) == []


def test_bad_specs_under_sanitizers(exe):
    for specs, V in (([TensorSpec("bad", 4, 4, "TILE", 0, 4)], 2), ([TensorSpec("neg", -3, 4, "ELEM")], 4),
                     ([TensorSpec("flat0", 4, 4, "FLAT", 0)], 2), ([TensorSpec("ok", 4, 4, "ELEM")], 0)):
        out = _run(exe, specs, V)
        word, status, message = out[0].split(" ", 2)
        assert word == "error" and int(status) < 0 and message.strip()
