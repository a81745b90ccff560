"""The C-ABI library on the host: it loads, exports every declared call, its
planner reproduces the oracle's plan exactly, and invalid plans or arguments
are rejected with the documented status before anything touches a GPU."""
import os
import random
import re
import time

import pytest

from oracle import plan as OP
from tests.test_oracle_plan import random_instance
from workloads import TensorSpec, workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def rs():
    import structure_aware_grouped_amd as pkg
    from structure_aware_grouped_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("librs_hip.so is not built: run __graft_entry__.build()")
    binding.load()
    return pkg


def _declared():
    text = open(os.path.join(ROOT, "include", "rs.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|void|const char\*)\s+(rs_\w+)\s*\(", text, re.M)))


def test_bench_helper_library_exports_its_declared_calls(rs):
    """librs_bench.so (the benchmark's streaming-copy ceiling, the square-root and store
    self-checks) exports what rs_bench.h declares; bad arguments are refused before any launch."""
    import ctypes
    text = open(os.path.join(ROOT, "include", "rs_bench.h")).read()
    names = sorted(set(re.findall(r"^\s*int\s+(rs_\w+)\s*\(", text, re.M)))
    assert names == ["rs_bench_copy", "rs_bench_sqrt_check", "rs_bench_store_check"]
    path = os.path.join(ROOT, "structure_aware_grouped_amd", "librs_bench.so")
    assert os.path.exists(path), "librs_bench.so is not built: run __graft_entry__.build()"
    lib = ctypes.CDLL(path)
    lib.rs_bench_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    a, b = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 21)
    assert lib.rs_bench_copy(a, b, 15, None) == -1                      # not a multiple of 16
    assert lib.rs_bench_copy(a, ctypes.c_void_p((1 << 20) + 16), 64, None) == -1   # overlapping
    assert lib.rs_bench_copy(a, b, 0, None) == 0                        # nothing to do
    lib.rs_bench_sqrt_check.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    n, f = ctypes.c_uint64(7), ctypes.c_uint32(7)
    assert lib.rs_bench_sqrt_check(2, 1, ctypes.byref(n), ctypes.byref(f)) == -1   # empty range
    assert lib.rs_bench_sqrt_check(1, 2, None, ctypes.byref(f)) == -1             # null result
    assert (n.value, f.value) == (7, 7)                                           # untouched
    lib.rs_bench_store_check.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    assert lib.rs_bench_store_check(None, 128, 0, None) == -1                      # null
    assert lib.rs_bench_store_check(a, 100, 0, None) == -1                         # not a multiple of 128
    assert lib.rs_bench_store_check(a, 128, 4, None) == -1                         # no such mode
    assert lib.rs_bench_store_check(ctypes.c_void_p((1 << 20) + 8), 128, 0, None) == -1   # not 16-byte aligned
    assert lib.rs_bench_store_check(a, (1 << 30) + 128, 0, None) == -1             # too many vectors


def test_library_exports_every_declared_call(rs):
    from structure_aware_grouped_amd import binding
    names = _declared()
    assert set(names) == set(binding.EXPORTS)
    lib = binding.load()
    for n in names:
        assert hasattr(lib, n), n


@pytest.mark.parametrize("idx", range(5))
def test_host_planner_matches_oracle_on_workloads(rs, idx):
    w = workload(idx)
    t0 = time.perf_counter()
    S, starts, order, name = rs.rs_plan_build(list(w.specs), w.V)
    dt = time.perf_counter() - t0
    ref = OP.plan(w.specs, w.V)
    assert S == ref.S
    assert starts == [int(s) for s in ref.starts]
    assert order == ref.order and name == ref.order_name
    assert dt < 0.3   # the pages report planning under 0.3 s


@pytest.mark.parametrize("seed", range(150))
def test_host_planner_matches_oracle_on_random_instances(rs, seed):
    specs, V, a = random_instance(10_000 + seed)
    for policy in ("best", "default", "by_block_size", "by_shape"):
        S, starts, order, name = rs.rs_plan_build(specs, V, a, policy)
        ref = OP.plan(specs, V, a, policy)
        assert (S, starts, order, name) == (ref.S, [int(s) for s in ref.starts], ref.order,
                                             ref.order_name)


@pytest.mark.parametrize("seed", range(40))
def test_host_planner_matches_oracle_on_larger_random_groups(rs, seed):
    rng = random.Random(77 + seed)
    specs = []
    for i in range(rng.randint(2, 12)):
        kind = rng.choice(["ROWS", "TILE", "FLAT", "WHOLE", "ELEM"])
        r, c = rng.choice([1, 7, 64, 100, 128, 300]), rng.choice([1, 16, 48, 96, 130, 256])
        p0 = rng.choice([1, 2, 16, 32]) if kind in ("ROWS", "TILE") else (rng.choice([64, 100, 2048]) if kind == "FLAT" else 0)
        p1 = rng.choice([8, 16, 32]) if kind == "TILE" else 0
        specs.append(TensorSpec(f"t{i}", r, c, kind, p0, p1))
    V = rng.choice([2, 3, 8, 16, 64])
    S, starts, order, name = rs.rs_plan_build(specs, V, 16)
    ref = OP.plan(specs, V, 16)
    assert (S, starts, name) == (ref.S, [int(s) for s in ref.starts], ref.order_name)
    assert OP.check_plan(specs, V, S, starts, 16) == []


def _status(fn):
    from structure_aware_grouped_amd import binding
    with pytest.raises(binding.RsError) as ei:
        fn()
    assert binding.load().rs_last_error().decode()
    return ei.value.status


def test_plan_build_rejects_bad_arguments(rs):
    from structure_aware_grouped_amd import binding as b
    good = [TensorSpec("a", 4, 4, "ROWS", 1)]
    assert _status(lambda: rs.rs_plan_build(good, 0)) == b.RS_EINVAL
    assert _status(lambda: rs.rs_plan_build(good, 4, 0)) == b.RS_EINVAL
    assert _status(lambda: rs.rs_plan_build([TensorSpec("a", 0, 4, "ELEM")], 4)) == b.RS_EINVAL
    assert _status(lambda: rs.rs_plan_build([TensorSpec("a", 4, 4, "TILE", 2, 0)], 4)) == b.RS_EINVAL
    assert _status(lambda: rs.rs_plan_build([TensorSpec("a", 4, 4, "ROWS", 0)], 4)) == b.RS_EINVAL
    assert _status(lambda: rs.rs_plan_build([TensorSpec("a", 4, 4, "ELEM", 3)], 4)) == b.RS_EINVAL
    assert _status(lambda: rs.rs_plan_build([TensorSpec("a", 4, 4, 9)], 4)) == b.RS_EINVAL


def test_plan_load_rejects_invalid_plans_before_touching_a_gpu(rs):
    from structure_aware_grouped_amd import binding as b
    specs = [TensorSpec("a", 4, 16, "ROWS", 1), TensorSpec("b", 2, 32, "TILE", 2, 16)]
    V, S = 4, 64
    L = rs.rs_plan_load
    assert _status(lambda: L(specs, V, 40, [0, 64])) == b.RS_EALIGN          # S % 16
    assert _status(lambda: L(specs, V, S, [8, 64])) == b.RS_EALIGN           # start % 16
    assert _status(lambda: L(specs, V, S, [0, 32])) == b.RS_EPLAN            # overlap
    assert _status(lambda: L(specs, V, S, [0, 96])) == b.RS_EPLAN            # boundary 128 cuts the band
    assert _status(lambda: L(specs, V, S, [0, 224])) == b.RS_EPLAN           # past V*S
    assert _status(lambda: L(specs, V, S, [-16, 64])) == b.RS_EPLAN          # negative start
    assert _status(lambda: L(specs, V, S, [0, 128], R_mat=2)) == b.RS_ERANGE  # R_mat < R_used = 3
    assert _status(lambda: L(specs, V, S, [0, 128], R_mat=5)) == b.RS_ERANGE  # R_mat > V
    assert _status(lambda: L(specs, 1 << 40, 1 << 30, [0, 128])) == b.RS_ERANGE  # V*S overflows
    assert _status(lambda: L([TensorSpec("a", 4, 16, "FLAT", 0)], V, S, [0])) == b.RS_EINVAL
    assert _status(lambda: L(specs, 0, S, [0, 128])) == b.RS_EINVAL
    assert _status(lambda: L(specs, V, S, [0, 128], device=-1)) == b.RS_EINVAL


def test_valid_plan_without_gpu_reports_a_hip_error(rs):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    from structure_aware_grouped_amd import binding as b
    specs = [TensorSpec("a", 4, 16, "ROWS", 1), TensorSpec("b", 2, 32, "TILE", 2, 16)]
    assert _status(lambda: rs.rs_plan_load(specs, 4, 64, [0, 128])) == b.RS_EHIP


def test_tile_major_specs_are_checked(rs):
    from structure_aware_grouped_amd import binding as b
    assert _status(lambda: rs.rs_plan_build([TensorSpec("a", 30, 32, "TILEMAJOR", 16, 16)], 4)) == b.RS_EINVAL
    assert _status(lambda: rs.rs_plan_build([TensorSpec("a", 32, 30, "TILEMAJOR", 16, 16)], 4)) == b.RS_EINVAL
    assert _status(lambda: rs.rs_plan_build([TensorSpec("a", 9, 9, "TILEMAJOR", 3, 3)], 4)) == b.RS_EINVAL
    assert _status(lambda: rs.rs_plan_build([TensorSpec("a", 1, 16384, "TILEMAJOR", 1, 16384)], 4)) == b.RS_EINVAL


@pytest.mark.parametrize("seed", range(30))
def test_host_planner_matches_oracle_on_tile_major_groups(rs, seed):
    rng = random.Random(500 + seed)
    specs = []
    for i in range(rng.randint(1, 6)):
        kind = rng.choice(["TILEMAJOR", "TILEMAJOR", "TILE", "ROWS"])
        br, bc = rng.choice([(16, 16), (32, 32), (8, 64), (128, 128), (16, 3)])
        r, c = br * rng.randint(1, 6), bc * rng.randint(1, 6)
        specs.append(TensorSpec(f"t{i}", r, c, kind, br if kind != "ROWS" else 1, bc if kind != "ROWS" else 0))
    V = rng.choice([1, 2, 3, 8, 16])
    S, starts, order, name = rs.rs_plan_build(specs, V, 16)
    ref = OP.plan(specs, V, 16)
    assert (S, starts, name) == (ref.S, [int(s) for s in ref.starts], ref.order_name)


def test_plan_larger_than_any_device_is_rejected(rs):
    """R_mat * S above 2^39 elements is refused on the host before any lowering
    (launches loop over their work items, so only the 32-bit indices bound a plan)."""
    from structure_aware_grouped_amd import binding as b
    big = [TensorSpec("big", 1 << 20, 1 << 19, "ELEM")]      # 2^39 elements
    assert _status(lambda: rs.rs_plan_load(big, 2, 1 << 39, [0], R_mat=2)) == b.RS_ERANGE
    assert "2^39" in b.load().rs_last_error().decode()


def test_empty_group_and_null_outputs_are_rejected(rs):
    from structure_aware_grouped_amd import binding as b
    assert _status(lambda: rs.rs_plan_build([], 4)) == b.RS_EINVAL
    lib = b.load()
    spec = b.specs_array([TensorSpec("a", 4, 4, "ROWS", 1)])
    S = b.ctypes.c_int64()
    assert lib.rs_plan_build(spec, 1, 4, 16, 0, None, None, None, None) == b.RS_EINVAL
    assert lib.rs_plan_build(spec, 1, 4, 16, 0, b.ctypes.byref(S), None, None, None) == b.RS_EINVAL
    assert lib.rs_plan_build(spec, 1, 4, 16, 7, b.ctypes.byref(S), (b.ctypes.c_int64 * 1)(), None, None) \
        == b.RS_EINVAL                                            # unknown order policy


def test_largest_tensor_plans_on_the_host(rs):
    """A single tensor of 2^40 elements (the spec limit) plans without overflow; one
    more row is rejected."""
    from structure_aware_grouped_amd import binding as b
    big = TensorSpec("big", 1 << 20, 1 << 20, "ROWS", 1)
    S, starts, _, _ = rs.rs_plan_build([big], 64)
    assert starts == [0] and S == (1 << 40) // 64 and S % 16 == 0
    ref = OP.plan([big], 64)
    assert (S, starts) == (ref.S, [int(x) for x in ref.starts])
    assert _status(lambda: rs.rs_plan_build([TensorSpec("big", (1 << 20) + 1, 1 << 20, "ROWS", 1)], 64)) \
        == b.RS_EINVAL


def test_missing_library_fails_loudly(tmp_path):
    """No CPU fallback: opening a library that is not there raises, naming the build."""
    import subprocess
    import sys
    code = ("import structure_aware_grouped_amd.binding as b\n"
            f"try:\n    b.load({str(tmp_path / 'librs_hip.so')!r})\n"
            "except RuntimeError as e:\n    print('raised:', e)\nelse:\n    print('loaded')\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert "raised:" in out.stdout and "no CPU fallback" in out.stdout, out.stdout + out.stderr


def test_binding_rejects_a_pointer_list_of_the_wrong_length(rs):
    """The C calls read one pointer per tensor: a shorter or longer list never reaches them."""
    import torch
    from structure_aware_grouped_amd import binding
    plan = binding.Plan.__new__(binding.Plan)   # host-only stand-in: nothing is loaded on a device
    plan._h, plan.numels, plan.device, plan.R_mat, plan.S, plan.n_qblocks = None, [16, 32], 0, 1, 48, 0
    t = torch.zeros(16)
    for call in (lambda: binding.rs_unpack_gathered(plan, torch.zeros(48), [t]),
                 lambda: binding.rs_pack_scatter(plan, [t, t, t], torch.zeros(48)),
                 lambda: binding.rs_unpack_dequant(plan, torch.zeros(48, dtype=torch.uint8), "e4m3",
                                                   torch.zeros(1), [None])):
        with pytest.raises(ValueError, match="entries for a plan of 2 tensors"):
            call()


def test_binding_rejects_gradients_of_another_dtype(rs):
    import torch
    from structure_aware_grouped_amd import binding
    plan = binding.Plan.__new__(binding.Plan)
    plan._h, plan.numels, plan.device, plan.R_mat, plan.S, plan.n_qblocks = None, [16], 0, 1, 16, 0
    with pytest.raises(ValueError, match="fp32 or bf16"):
        binding.rs_pack_scatter(plan, [torch.zeros(16, dtype=torch.float16)], torch.zeros(16))


@pytest.mark.parametrize("dtype", ["bfloat16", "float16", "int32", "float64"])
def test_binding_rejects_scales_of_another_dtype(rs, dtype):
    """Every call that reads or writes scales takes n_qblocks fp32 values: a scales tensor of
    another dtype with n_qblocks entries would be read or written past its end."""
    import torch
    from structure_aware_grouped_amd import binding
    plan = binding.Plan.__new__(binding.Plan)
    plan._h, plan.numels, plan.device, plan.R_mat, plan.S, plan.n_qblocks = None, [64], 0, 1, 64, 4
    plan.specs = [TensorSpec("t", 8, 8, "TILE", 4, 4)]
    sc = torch.zeros(4, dtype=getattr(torch, dtype))
    q = torch.zeros(64, dtype=torch.uint8)
    for call in (lambda: binding.rs_block_quant(plan, torch.zeros(64), q, "e4m3", sc),
                 lambda: binding.rs_block_dequant(plan, q, "e4m3", sc, torch.zeros(64)),
                 lambda: binding.rs_unpack_dequant(plan, q, "e4m3", sc, [torch.zeros(8, 8)])):
        with pytest.raises(ValueError, match="scales: fp32"):
            call()


def _llama70b_model(layers):
    specs = []
    for l in range(layers):
        for name, r, c in (("wq", 8192, 8192), ("wk", 1024, 8192), ("wv", 1024, 8192), ("wo", 8192, 8192),
                           ("gate", 28672, 8192), ("up", 28672, 8192), ("down", 8192, 28672)):
            specs.append(TensorSpec(f"{l}.{name}", r, c, "TILE", 128, 128))
        specs += [TensorSpec(f"{l}.n1", 8192, 1, "ROWS", 1), TensorSpec(f"{l}.n2", 8192, 1, "ROWS", 1)]
    return specs


def _moe_experts(layers, experts):
    """Per-expert tensors of DeepSeek-V3-sized MoE layers (7168 hidden, 2048 expert width)."""
    specs = []
    for l in range(layers):
        for e in range(experts):
            specs += [TensorSpec(f"{l}.{e}.gate", 2048, 7168, "TILE", 128, 128),
                      TensorSpec(f"{l}.{e}.up", 2048, 7168, "TILE", 128, 128),
                      TensorSpec(f"{l}.{e}.down", 7168, 2048, "TILE", 128, 128)]
    return specs


@pytest.mark.slow
def test_host_planner_matches_oracle_on_a_thousand_expert_tensors(rs):
    specs, V = _moe_experts(4, 256), 1024          # 3072 tensors, 45B parameters
    S, starts, _, name = rs.rs_plan_build(specs, V)
    ref = OP.plan(specs, V)
    assert (S, starts, name) == (ref.S, [int(s) for s in ref.starts], ref.order_name)


@pytest.mark.parametrize("case", ["llama70b_80_layers", "moe_58_layers_256_experts"])
def test_host_planner_on_whole_models(rs, case):
    """Whole-model groups plan within the pages' 0.3 s, validly, within twice the lower bound."""
    specs, V = (_llama70b_model(80), 1024) if case.startswith("llama") else (_moe_experts(58, 256), 4096)
    t0 = time.perf_counter()
    S, starts, _, _ = rs.rs_plan_build(specs, V)
    dt = time.perf_counter() - t0
    assert dt < 0.3, dt
    assert OP.check_plan(specs, V, S, starts, 16) == []
    n = sum(sp.numel for sp in specs)
    lb = -(-max(-(-n // V), max(min(OP.granularity(sp), sp.numel) for sp in specs)) // 16) * 16
    assert lb <= S <= 2 * lb
