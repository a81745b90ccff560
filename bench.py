"""Throughput of the RaggedShard / DBuffer layout transform on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1]

One step is one pass of the whole path over one batch of synthetic input that
is already resident in HBM: for the Llama-3-8B layer at V=64 (the default),
unpack of the gathered bf16 parameter buffer into the 9 parameter tensors,
pack of the 9 fp32 gradients into the fp32 rank slices (scale by 1/V,
accumulate into the previous packed buffer, zero the padding), and E4M3
quantisation of every 128x128 tile of the bf16 parameter buffer. The Adam
workload (--workload 4) steps through pack, int8/uint8 quant and dequant of m
and v.

Throughput counts algorithmic bytes (each byte a kernel must read or write
once). In the timed region every kernel launch follows a 1 GiB write that
leaves none of its inputs in L2 or the 256 MB MALL, and HIP events on the
stream the kernels run on bracket each launch; the headline divides one
step's bytes by the sum of its kernels' median durations over the K steps.
A warm pass (K steps back to back, wall clock) is reported apart, as is a
16-byte streaming copy that moves as many bytes as the dominant kernel, the
practical ceiling. The CPU baseline
times the CPU oracle on a bounded sample of the same workload, on one core
and on all host cores. Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E peak
FLUSH_BYTES = 1 << 30   # written before every timed launch: 4x the 256 MB MALL
METRIC = "DBuffer pack/unpack+blockquant GB/s, % HBM peak (Llama-3-8B layer, V=64)"
# committed counter summaries: (workload, mode, tile-major, Adam blocks) -> profiles/traffic_<name>.md
PROFILE_TRAFFIC = {
    (1, "step", False, "flat2048"): "llama3_8b_v64",
    (1, "step", True, "flat2048"): "llama3_8b_v64_tile_major",
    (1, "fp8_gather", False, "flat2048"): "llama3_8b_v64_fp8_gather",
    (1, "fp8_gather", True, "flat2048"): "llama3_8b_v64_tile_major_fp8_gather",
    (2, "step", False, "flat2048"): "llama3_70b_v1024",
    (3, "step", False, "flat2048"): "moe128_v256",
    (3, "fp8_gather", False, "flat2048"): "moe128_v256_fp8_gather",
    (4, "step", False, "flat2048"): "adam_states_llama3_8b_v64",
    (4, "adam8", False, "flat2048"): "adam8_llama3_8b_v64",
    (4, "adam8", False, "tile32"): "adam8_tile32_llama3_8b_v64",
}
KERNEL_SOURCES = [os.path.join(ROOT, "structure_aware_grouped_amd", "csrc", f)
                  for f in ("device_common.h", "host_common.h", "transform.hip", "quant.hip", "gather.hip",
                            "adam.hip", "rs_internal.h", "plan.cpp")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20,
                    help="timed steps; each kernel's figure is the median over them")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=1, choices=[0, 1, 2, 3, 4],
                    help="0 is the tiny three-tensor group: launch-bound, a parity case more than a bandwidth one")
    ap.add_argument("--mode", default="step", choices=["step", "fp8_gather", "adam8"],
                    help="step: the workload's steps; fp8_gather: block quant of the rank slices, then "
                         "the fused unpack-dequant of the codes into the bf16 tensors; adam8 (workload 4): "
                         "one AdamW step on the int8/uint8 block-quantised m and v")
    ap.add_argument("--adam-blocks", default="flat2048", choices=["flat2048", "tile32"],
                    help="workload 4's quantisation blocks: 2048-element flat blocks, or the pages' own 8-bit "
                         "Adam layout, 32x32 tiles of every matrix at 32-row granularity")
    ap.add_argument("--tile-major", action="store_true",
                    help="store the TILE tensors tile by tile (TILEMAJOR): unpack and pack reorder through LDS")
    ap.add_argument("--packed-bf16", action="store_true",
                    help="pack into a bf16 buffer (a bf16 ReduceScatter): each fp32 result rounded once")
    ap.add_argument("--cpu-sample", type=int, default=1, help="0 disables the CPU-oracle baseline")
    ap.add_argument("--no-check", action="store_true", help="skip the sampled output checks")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph after the warm-up and replay it in the warm pass "
                         "(the flushed timed region stays eager)")
    ap.add_argument("--flush", default="write", choices=["write", "read"],
                    help="how the 1 GiB buffer before each timed launch empties L2 and the MALL: written "
                         "(fill) or read (a sum over it, which leaves no dirty lines behind)")
    ap.add_argument("--fenced-events", action="store_true",
                    help="time with default HIP events (system-scope fence at every record)")
    ap.add_argument("--copy-mib", type=int, default=-1,
                    help="size of the streaming copy (rs_bench_copy) timed as the practical ceiling "
                         "(and used to calibrate HBM byte counters); -1 (default): the copy moves as many "
                         "bytes as the dominant kernel (reads + writes), 0 disables it")
    return ap.parse_args()


def algorithmic_bytes(w, plan, packed_bytes: int = 4) -> dict:
    """Bytes each kernel must move once per call (read + write); packed_bytes is the
    element size of the packed buffer (4 for fp32, 2 for bf16)."""
    n_all = sum(plan.numels)
    R, S = plan.R_mat, plan.S
    pb = 2 if w.param_dtype == "bf16" else 4
    out = {}
    nq_all = sum(n for sp, n in zip(w.specs, plan.numels) if sp.kind in ("TILE", "TILEMAJOR", "FLAT"))
    out["unpack_dequant"] = nq_all * (1 + pb) + 4 * plan.n_qblocks
    # param read + write, grad read, m and v codes read + write (fp32 param/grad); 2 scales read + write
    out["adam8_step"] = nq_all * (4 + 4 + 4 + 2 + 2) + 16 * plan.n_qblocks
    if w.adam_states:
        nq = sum(n for sp, n in zip(w.specs, plan.numels) if sp.kind in ("TILE", "TILEMAJOR", "FLAT"))
        pack = n_all * (4 + 4) + 4 * plan.padding
        quant = nq * 4 + R * S + 4 * plan.n_qblocks
        dequant = nq * 1 + 4 * plan.n_qblocks + 4 * R * S
        for which in ("m", "v"):
            out[f"pack_{which}"] = pack
            out[f"quant_{which}"] = quant
            out[f"dequant_{which}"] = dequant
        return out
    out["unpack"] = 2 * n_all * pb
    out["pack"] = n_all * (4 + (4 if w.accumulate else 0) + packed_bytes) + packed_bytes * plan.padding
    if w.quant:
        nq = sum(n for sp, n in zip(w.specs, plan.numels) if sp.kind in ("TILE", "TILEMAJOR", "FLAT"))
        out["quant"] = nq * pb + R * S + 4 * plan.n_qblocks
    return out


def padding_ranges(specs, starts, S, R):
    """[begin, end) ranges of [0, R*S) that hold no tensor."""
    iv = sorted((int(s), int(s) + sp.numel) for sp, s in zip(specs, starts))
    out, pos = [], 0
    for b, e in iv:
        if b > pos:
            out.append((pos, b))
        pos = max(pos, e)
    if pos < R * S:
        out.append((pos, R * S))
    return out


def tile_major_arrangement(specs):
    """Input preparation: row-major bits -> the tile-by-tile order of TILEMAJOR tensors."""
    def arrange(i, bits):
        sp = specs[i]
        if sp.kind != "TILEMAJOR":
            return bits
        return bits.reshape(sp.rows // sp.p0, sp.p0, sp.cols // sp.p1, sp.p1).transpose(0, 2, 1, 3).ravel()
    return arrange


def kernel_hash() -> str:
    """Hash of the sources that decide what the kernels do and how work is split."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def read_traffic(key, kernel: str):
    """Measured HBM bytes per launch of bench step `kernel` from the committed counter
    summary of this configuration, if there is one and it was taken on the current
    kernel source; else None."""
    name = PROFILE_TRAFFIC.get(key)
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.md") if name else None
    if not path or not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel sources sha256\[:16\]:\s*`?([0-9a-f]{16})", text, re.I)
    if not m or m.group(1) != kernel_hash():
        return None
    m = re.search(rf"^\|\s*{kernel}\s*\|[^\n]*?\|\s*([0-9]+)\s*\|\s*$", text, re.M)
    return int(m.group(1)) if m else None


class HipTimer:
    """HIP timing events recorded on a given stream.

    By default the events are created with hipEventDisableSystemFence: recording
    one then costs no system-scope cache writeback and invalidation between the
    kernels it separates (a default event record adds about 10 us of idle GPU
    time at every boundary of this step). The events are only read after a
    device-wide synchronisation, which is what that flag requires. The HIP
    runtime is the one torch loaded."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, torch, fenced: bool = False):
        path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
        hip = ctypes.CDLL(path if os.path.exists(path) else "libamdhip64.so")
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip, self.flags, self.events = hip, 0 if fenced else self.DISABLE_SYSTEM_FENCE, []

    @staticmethod
    def _ok(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def event(self):
        e = ctypes.c_void_p()
        self._ok(self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.flags), "hipEventCreateWithFlags")
        self.events.append(e)
        return e

    def record(self, e, stream: int):
        self._ok(self.hip.hipEventRecord(e, ctypes.c_void_p(stream)), "hipEventRecord")

    def ms(self, a, b) -> float:
        t = ctypes.c_float()
        self._ok(self.hip.hipEventElapsedTime(ctypes.byref(t), a, b), "hipEventElapsedTime")
        return t.value

    def close(self):
        for e in self.events:
            self.hip.hipEventDestroy(e)
        self.events = []


def bench_lib():
    """librs_bench.so (the streaming-copy ceiling), opened after torch's HIP runtime."""
    path = os.path.join(ROOT, "structure_aware_grouped_amd", "librs_bench.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with structure_aware_grouped_amd.build")
    lib = ctypes.CDLL(path)
    lib.rs_bench_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.rs_bench_copy.restype = ctypes.c_int
    return lib


def log(msg: str):
    """A progress line on stderr (the JSON result line goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _oracle_step_on(w, spec, sigma, fmt, wb, g, p, pb):
    """The oracle's unpack, pack and (for tiled tensors) block quant of one tensor or
    tile band; returns the algorithmic bytes that work moves."""
    from oracle import transform as OT
    import workloads as W
    n = spec.numel
    OT.unpack(wb, [spec], [0])                       # the tensor is its slice of the buffer
    OT.pack_values(g.ravel(), p, sigma, True)        # scale, accumulate
    moved = 2 * n * pb + n * 12
    if spec.kind in ("TILE", "TILEMAJOR", "FLAT") and fmt:
        x = W.f32_from_bf16_bits(wb) if wb.dtype == np.uint16 else wb.view(np.float32)
        for _, b, pos in OT.quant_blocks([spec], [0]):
            OT.quantize_block(x[pos], fmt)
        moved += n * pb + n + 4 * OT.count_quant_blocks([spec])
    return moved


def _cpu_units(w, starts, S, idx, rows_per_unit: int = 1024):
    """(tensor, r0, r1) pieces of the sampled tensors for the all-core leg: tile bands of
    about rows_per_unit rows (whole bands), whole tensors otherwise."""
    units = []
    for i in idx:
        sp = w.specs[i]
        step = sp.rows
        if sp.kind in ("TILE", "TILEMAJOR") and sp.rows > rows_per_unit:
            step = max(sp.p0, rows_per_unit // sp.p0 * sp.p0)
        for r0 in range(0, sp.rows, step):
            units.append((i, r0, min(sp.rows, r0 + step)))
    return units


def _cpu_worker(widx, tile_major, S, starts, units, barrier, results):
    """One process of the all-core leg: regenerate its pieces' inputs, wait for the
    others, run the oracle on its pieces, report (bytes, start, end) on the monotonic
    clock that all processes share."""
    from oracle import transform as OT
    import workloads as W
    w = W.workload(widx)
    if tile_major:
        w = W.tile_major_variant(w)
    pb = 2 if w.param_dtype == "bf16" else 4
    sigma = OT.inv_v(w.V)
    prev_cache = {}

    def prev_range(b, e):
        parts = []
        for k in range(b // S, (e - 1) // S + 1):
            if k not in prev_cache:
                prev_cache[k] = W.prev_slice(w, k, S)
            lo, hi = max(b, k * S) - k * S, min(e, (k + 1) * S) - k * S
            parts.append(prev_cache[k][lo:hi])
        return np.concatenate(parts)

    work, cache = [], {}
    for i, r0, r1 in units:
        sp = w.specs[i]
        if i not in cache:
            cache = {i: (W.weight_bits(w, i).reshape(sp.rows, sp.cols),
                         W.tensor_values(w, i, W.Role.GRAD))}
        wb, g = cache[i]
        band = W.TensorSpec(sp.name, r1 - r0, sp.cols, sp.kind, sp.p0, sp.p1)
        s = starts[i] + r0 * sp.cols
        work.append((band, np.ascontiguousarray(wb[r0:r1]).ravel(), np.ascontiguousarray(g[r0:r1]),
                     prev_range(s, s + band.numel)))
    cache = prev_cache = None
    barrier.wait()
    t0 = time.perf_counter()
    moved = sum(_oracle_step_on(w, band, sigma, w.quant, wb, g, p, pb) for band, wb, g, p in work)
    results.put((moved, t0, time.perf_counter()))


def _secs(t: float) -> str:
    return f"{t:.2f} s" if t >= 1 else f"{t * 1e3:.2f} ms"


def cpu_baseline(w, plan, tile_major: bool = False, max_seconds: float = 15.0) -> dict:
    """The CPU oracle (NumPy) on a bounded sample of the workload, single-threaded and
    then on all host cores.

    Single core: the tensors one at a time and in order until `max_seconds` of oracle
    time have passed (the Llama-3-8B and Llama-3-70B layers finish whole; the MoE layer
    stops after its first experts). All cores: the same tensors cut into tile bands,
    spread over one process per core (at most 16), each regenerating its inputs before a
    common start. Both use the bench's byte accounting; inputs are generated before the
    clock starts."""
    import multiprocessing
    from oracle import transform as OT
    from workloads.device import Inputs

    inp = Inputs(w, plan.S, plan.starts, plan.R_mat, device="cpu")
    pb = 2 if w.param_dtype == "bf16" else 4
    sigma = OT.inv_v(w.V)
    moved, dt, done = 0, 0.0, []
    for i in range(len(w.specs)):
        if dt >= max_seconds:
            break
        done.append(i)
        spec, s = w.specs[i], plan.starts[i]
        wb, g, p = inp.weight_bits(i), inp.grad(i), inp.prev_range(s, s + spec.numel)
        t0 = time.perf_counter()
        moved += _oracle_step_on(w, spec, sigma, w.quant, wb, g, p, pb)
        dt += time.perf_counter() - t0
    if len(done) == len(w.specs):
        what = "every tensor of the layer (one whole step)"
    elif len(done) <= 4:
        what = ", ".join(w.specs[i].name for i in done)
    else:
        what = f"the first {len(done)} of the layer's {len(w.specs)} tensors"
    work = f"unpack + pack{' + ' + w.quant + ' tile quant' if w.quant else ''}"
    size = (f"{moved / 1e9:.3f} GB" if moved >= 1e8 else f"{moved / 1e6:.3f} MB")
    single = {"value": round(moved / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
              "seconds": round(dt, 3)}

    affinity = len(os.sched_getaffinity(0))
    procs = max(1, min(16, affinity))
    units = _cpu_units(w, plan.starts, plan.S, done)
    loads = [[] for _ in range(procs)]
    sizes = [0] * procs
    for u in sorted(units, key=lambda u: -(u[2] - u[1]) * w.specs[u[0]].cols):   # largest first
        k = sizes.index(min(sizes))
        loads[k].append(u)
        sizes[k] += (u[2] - u[1]) * w.specs[u[0]].cols
    loads = [sorted(l) for l in loads if l]
    ctx = multiprocessing.get_context("spawn")       # the workers never touch the GPU
    barrier, results = ctx.Barrier(len(loads)), ctx.Queue()
    ps = [ctx.Process(target=_cpu_worker, args=(w.index, tile_major, plan.S, list(plan.starts), l, barrier, results))
          for l in loads]
    for p in ps:
        p.start()
    got = [results.get(timeout=600) for _ in ps]
    for p in ps:
        p.join()
    par_moved = sum(r[0] for r in got)
    wall = max(r[2] for r in got) - min(r[1] for r in got)
    assert par_moved == moved, "the all-core leg covers the same work as the single-core leg"
    return {"value": round(par_moved / wall / 1e9, 4), "unit": "GB/s", "cores": len(loads), "kind": "oracle",
            "sample": f"{what}: {work}, {size}; {len(loads)} processes in {_secs(wall)}, 1 core in {_secs(dt)}",
            "single_core": single, "nproc": os.cpu_count(), "affinity": affinity}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the V logical ranks are slices of one device buffer "
              f"and no collective is run (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import structure_aware_grouped_amd as rs
    from workloads.device import Inputs, garbage, tensor_bits
    from workloads import Role, adam_tile32_variant, tensor_values, tile_major_variant, workload

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    w = workload(args.workload)
    if args.tile_major:
        w = tile_major_variant(w)
    if args.adam_blocks == "tile32":
        if args.workload != 4:
            print("--adam-blocks applies to the Adam-state workload (4)", file=sys.stderr)
            sys.exit(2)
        w = adam_tile32_variant(w)
    specs = list(w.specs)

    t0 = time.perf_counter()
    S, starts, order, order_name = rs.rs_plan_build(specs, w.V)
    plan_ms = (time.perf_counter() - t0) * 1e3
    R_used = -(-max(s + sp.numel for s, sp in zip(starts, specs)) // S)
    R = w.V if w.materialize_all_ranks else R_used
    # validate, lower and upload the work lists (once per plan). The first load of the
    # process also pays for one-time HIP runtime set-up, so it is reported apart and the
    # plan is loaded again for load_ms.
    t0 = time.perf_counter()
    rs.rs_plan_load(specs, w.V, S, starts, R, 0).close()
    torch.cuda.synchronize()
    first_load_ms = (time.perf_counter() - t0) * 1e3
    t0 = time.perf_counter()
    plan = rs.rs_plan_load(specs, w.V, S, starts, R, 0)
    torch.cuda.synchronize()
    load_ms = (time.perf_counter() - t0) * 1e3
    log(f"plan: S={S}, R_mat={R}, lowered in {load_ms:.0f} ms (first load of the process {first_load_ms:.0f} ms)")
    inp = Inputs(w, S, starts, R, device=dev)
    if args.packed_bf16 and (w.adam_states or args.mode != "step"):
        print("--packed-bf16 applies to the step of workloads 0-3", file=sys.stderr)
        sys.exit(2)
    nbytes = algorithmic_bytes(w, plan, 2 if args.packed_bf16 else 4)
    avg_load = -(-sum(plan.numels) // w.V)

    # ---- inputs resident in HBM
    if args.mode == "adam8":
        if not w.adam_states:
            print("adam8 needs the Adam-state workload (4)", file=sys.stderr)
            sys.exit(2)
        flat = lambda: garbage(R * S, torch.float32, dev)
        param, grad, mbuf, vbuf = flat(), flat(), flat(), flat()
        weights = [torch.from_numpy(tensor_values(w, i, Role.WEIGHT)).to(dev) for i in range(len(specs))]
        rs.rs_pack_scatter(plan, weights, param, scale=1.0)
        del weights
        rs.rs_pack_scatter(plan, inp.grads(), grad, scale=1.0)
        rs.rs_pack_scatter(plan, inp.adam_states("m"), mbuf, scale=1.0)
        rs.rs_pack_scatter(plan, inp.adam_states("v"), vbuf, scale=1.0)
        qm = garbage(R * S, torch.uint8, dev)
        qv = garbage(R * S, torch.uint8, dev)
        sm = garbage(plan.n_qblocks, torch.float32, dev)
        sv = garbage(plan.n_qblocks, torch.float32, dev)
        rs.rs_block_quant(plan, mbuf, qm, "i8", sm)
        rs.rs_block_quant(plan, vbuf, qv, "u8", sv)
        del mbuf, vbuf
        counter = {"t": 0}

        def adam_step():
            counter["t"] += 1
            rs.rs_adam8_step(plan, param, grad, qm, sm, qv, sv, 1e-4, 0.9, 0.999, 1e-8, 0.01, counter["t"])

        steps = [("adam8_step", adam_step)]
        dominant = "adam8_step"
    elif w.adam_states:
        m = inp.adam_states("m")
        v = inp.adam_states("v")
        pm = garbage(R * S, torch.float32, dev)
        pv = garbage(R * S, torch.float32, dev)
        qm = garbage(R * S, torch.uint8, dev)
        qv = garbage(R * S, torch.uint8, dev)
        sm = garbage(plan.n_qblocks, torch.float32, dev)
        sv = garbage(plan.n_qblocks, torch.float32, dev)
        dm = garbage(R * S, torch.float32, dev)
        dv = garbage(R * S, torch.float32, dev)
        steps = [
            ("pack_m", lambda: rs.rs_pack_scatter(plan, m, pm, scale=1.0)),
            ("pack_v", lambda: rs.rs_pack_scatter(plan, v, pv, scale=1.0)),
            ("quant_m", lambda: rs.rs_block_quant(plan, pm, qm, "i8", sm)),
            ("quant_v", lambda: rs.rs_block_quant(plan, pv, qv, "u8", sv)),
            ("dequant_m", lambda: rs.rs_block_dequant(plan, qm, "i8", sm, dm)),
            ("dequant_v", lambda: rs.rs_block_dequant(plan, qv, "u8", sv, dv)),
        ]
        dominant = "pack_m"
    elif args.mode == "fp8_gather":
        if not w.quant:
            print("fp8_gather needs a workload with block quantisation (1 or 3)", file=sys.stderr)
            sys.exit(2)
        G = inp.gathered(tile_major_arrangement(specs))
        q = garbage(R * S, torch.uint8, dev)
        scales = garbage(plan.n_qblocks, torch.float32, dev)
        full = [torch.empty(sp.rows, sp.cols, dtype=inp.pdtype, device=dev)
                if sp.kind in ("TILE", "TILEMAJOR", "FLAT") else None for sp in specs]
        steps = [
            ("quant", lambda: rs.rs_block_quant(plan, G, q, w.quant, scales)),
            ("unpack_dequant", lambda: rs.rs_unpack_dequant(plan, q, w.quant, scales, full)),
        ]
        dominant = "unpack_dequant"
    else:
        G = inp.gathered(tile_major_arrangement(specs))
        params = inp.empty_params()
        grads = inp.grads()
        prev = inp.prev()
        packed = garbage(R * S, torch.bfloat16 if args.packed_bf16 else torch.float32, dev)
        steps = [
            ("unpack", lambda: rs.rs_unpack_gathered(plan, G, params)),
            ("pack", lambda: rs.rs_pack_scatter(plan, grads, packed, prev=prev)),
        ]
        if w.quant:
            q = garbage(R * S, torch.uint8, dev)
            scales = garbage(plan.n_qblocks, torch.float32, dev)
            steps.append(("quant", lambda: rs.rs_block_quant(plan, G, q, w.quant, scales)))
        dominant = "pack"
    torch.cuda.synchronize()
    log("inputs resident in HBM")

    stream = torch.cuda.current_stream(dev).cuda_stream
    timer = HipTimer(torch, fenced=args.fenced_events)
    flush = torch.ones(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    flush64 = flush.view(torch.int64)

    def empty_caches(k):
        """Touch 1 GiB (4x the MALL): nothing a kernel reads is left in L2 or the MALL."""
        if args.flush == "write":
            flush.fill_(k & 0xFF)
        else:
            flush64.sum()

    def flushed_launches(fn, n):
        """n launches of fn, each after the 1 GiB flush; HIP events around the launch only.
        Durations in ms."""
        ev = [(timer.event(), timer.event()) for _ in range(n)]
        for k, (a, b) in enumerate(ev):
            empty_caches(k)
            timer.record(a, stream)
            fn()
            timer.record(b, stream)
        torch.cuda.synchronize()
        return [timer.ms(a, b) for a, b in ev]

    copy = None
    if args.copy_mib:
        # the practical HBM ceiling: a 16-byte streaming copy of known size (the library's
        # benchmark helper), timed like the kernels; its counter readings calibrate
        # FETCH_SIZE / WRITE_SIZE. torch's own device copy is timed beside it for context.
        blib = bench_lib()
        # same size as the dominant kernel: it reads and writes half its bytes each
        nb = args.copy_mib << 20 if args.copy_mib > 0 else max(1 << 20, int(nbytes[dominant]) // 2 // 1024 * 1024)
        src_c = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
        dst_c = torch.empty_like(src_c)

        def own_copy():
            rc = blib.rs_bench_copy(ctypes.c_void_p(dst_c.data_ptr()), ctypes.c_void_p(src_c.data_ptr()),
                                    ctypes.c_int64(nb), ctypes.c_void_p(stream))
            if rc != 0:
                raise RuntimeError(f"rs_bench_copy returned {rc}")
        own_copy()
        torch.cuda.synchronize()
        assert bool(torch.equal(dst_c[:: 1 << 16], src_c[:: 1 << 16])), "rs_bench_copy"
        ms = flushed_launches(own_copy, args.steps)
        med = float(np.median(ms))
        tms = flushed_launches(lambda: dst_c.copy_(src_c), 5)
        copy = {"kernel": "rs_bench_copy: 16-byte nontemporal loads, nt-sc1 buffer stores, 64-thread workgroups of 1 KiB",
                "size": (f"{nb / 2**20:.0f} MiB copied: the {dominant} kernel's bytes" if args.copy_mib < 0
                         else f"{nb / 2**20:.0f} MiB copied"),
                "bytes": 2 * nb, "median_ms": round(med, 5), "GBps": round(2 * nb / (med * 1e-3) / 1e9, 1),
                "torch_copy_GBps": round(2 * nb / (float(np.median(tms)) * 1e-3) / 1e9, 1),
                "timing": f"median of {args.steps} flushed launches"}
        del src_c, dst_c

    for _ in range(args.warmup):
        for _, fn in steps:
            fn()
    torch.cuda.synchronize()

    # ---- timed region: K steps, cold. Before every kernel launch a 1 GiB buffer is written
    # (outside the events), so no kernel finds its inputs in L2 or the MALL; HIP events
    # on the stream the library launches on (torch's current stream, which the binding
    # passes) bracket each launch. Per kernel: the median over the K steps.
    graph = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _, fn in steps:
                fn()
        graph.replay()
    kev = [[(timer.event(), timer.event()) for _ in steps] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        for (name, fn), (a, b) in zip(steps, kev[k]):
            empty_caches(k)
            timer.record(a, stream)
            fn()
            timer.record(b, stream)
    torch.cuda.synchronize()
    wall_cold = time.perf_counter() - t0
    log(f"timed region: {args.steps} flushed steps in {wall_cold * 1e3:.1f} ms (flushes included)")
    per_kernel = {}
    for j, (name, _) in enumerate(steps):
        ms = [timer.ms(kev[k][j][0], kev[k][j][1]) for k in range(args.steps)]
        med, avg = float(np.median(ms)), float(np.mean(ms))
        per_kernel[name] = {"median_ms": round(med, 5), "avg_ms": round(avg, 5), "min_ms": round(float(np.min(ms)), 5),
                            "GBps": round(nbytes[name] / (med * 1e-3) / 1e9, 1), "bytes": int(nbytes[name])}
    step_bytes = sum(nbytes[name] for name, _ in steps)
    ms_per_step = sum(per_kernel[name]["median_ms"] for name, _ in steps)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    dom_avg_s = per_kernel[dominant]["avg_ms"] * 1e-3

    # ---- warm pass, labelled apart: K steps back to back, as a training loop calls them
    # (a kernel may find part of its input in the MALL, left there by the kernel before
    # it). Events around the dominant kernel only, the wall clock around the K steps; then
    # K more steps with events around every launch. With --graph each step is one replay
    # of the captured step.
    dom_ev = [(timer.event(), timer.event()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        if graph is not None:
            timer.record(dom_ev[k][0], stream)
            graph.replay()
            timer.record(dom_ev[k][1], stream)
            continue
        for name, fn in steps:
            if name == dominant:
                timer.record(dom_ev[k][0], stream)
                fn()
                timer.record(dom_ev[k][1], stream)
            else:
                fn()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dom_ms = [timer.ms(a, b) for a, b in dom_ev]
    del graph
    wev = [[(timer.event(), timer.event()) for _ in steps] for _ in range(args.steps)]
    for k in range(args.steps):
        for (name, fn), (a, b) in zip(steps, wev[k]):
            timer.record(a, stream)
            fn()
            timer.record(b, stream)
    torch.cuda.synchronize()
    warm = {"label": f"warm caches: {args.steps} steps back to back" +
                     (" (one HIP graph replay each)" if args.graph else ""),
            "value": round(step_bytes / (wall / args.steps) / 1e9, 1), "ms_per_step": round(wall / args.steps * 1e3, 4),
            ("graph_replay_avg_ms" if args.graph else f"{dominant}_in_steps_avg_ms"): round(float(np.mean(dom_ms)), 5)}
    for j, (name, _) in enumerate(steps):
        ms = [timer.ms(wev[k][j][0], wev[k][j][1]) for k in range(args.steps)]
        warm[name] = {"median_ms": round(float(np.median(ms)), 5),
                      "GBps": round(nbytes[name] / (float(np.median(ms)) * 1e-3) / 1e9, 1)}
    del flush, flush64

    # ---- sampled checks of the outputs of the last step
    check = "skipped"
    if not args.no_check and args.mode == "fp8_gather":
        # rebuilt weights stay within E4M3's rounding of the originals (half a step of a
        # 3-bit mantissa, or of the subnormal step times the block scale); no oracle needed
        from workloads import f32_from_bf16_bits
        i = 1
        x = f32_from_bf16_bits(inp.weight_bits(i)).astype(np.float64)
        y = full[i].float().cpu().numpy().ravel().astype(np.float64)
        amax = float(np.abs(x).max())
        assert np.all(np.abs(y - x) <= np.abs(x) * 2.0 ** -4 * 1.01 + amax / 448 * 2.0 ** -10 + np.abs(x) * 2.0 ** -8), \
            "unpack_dequant"
        check = f"ok ({specs[i].name}: rebuilt weights within E4M3 rounding of the originals)"
    elif not args.no_check and not w.adam_states:
        # checks that need no oracle (the oracle parity tests live in tests/): the tensors
        # unpack to their generated weights (every tensor; on the MoE layer the first and
        # last expert and the router), padding is +0.0, codes outside blocks are 0, scales
        # are finite and positive
        which = range(len(specs)) if len(specs) < 64 else [0, 1, len(specs) - 3, len(specs) - 2, len(specs) - 1]
        for i in which:
            assert np.array_equal(tensor_bits(params[i]).ravel(), inp.weight_bits(i)), f"unpack {specs[i].name}"
        pads = padding_ranges(specs, starts, S, R)
        pk = packed.view(torch.int16 if args.packed_bf16 else torch.int32)
        assert all(bool((pk[b:e] == 0).all()) for b, e in pads), "pack padding"
        if w.quant:
            assert all(bool((q[b:e] == 0).all()) for b, e in pads), "codes outside blocks"
            sf = scales.float()
            assert bool(torch.isfinite(sf).all()) and bool((sf > 0).all()), "scales"
        check = (f"ok ({'every tensor unpacks' if len(specs) < 64 else f'{len(which)} tensors unpack'} to its "
                 f"weights; padding and codes outside blocks are zero)")
    elif not args.no_check and args.mode == "step":
        # Adam-state layer, again without the oracle: the second tensor's m and v pack bit
        # for bit (sigma = 1, no accumulate), their dequantised values lie within half a
        # code step of the packed ones (plus the rounding of the fp32 product), and every
        # position outside the tensors is 0 in the packed, code and dequantised buffers
        i = 1
        s0, n1, b = int(starts[i]), specs[i].numel, specs[i].p0
        first = sum(-(-sp.numel // sp.p0) for sp in specs[:i])
        nb = -(-n1 // b)
        for name, src, pk, sc, dq in (("m", m, pm, sm, dm), ("v", v, pv, sv, dv)):
            x = pk[s0:s0 + n1]
            assert torch.equal(x.view(torch.int32), src[i].reshape(-1).view(torch.int32)), f"pack_{name}"
            s = sc[first:first + nb].double().repeat_interleave(b)[:n1]
            err = (dq[s0:s0 + n1].double() - x.double()).abs()
            assert bool((err <= 0.5 * s + 2.0 ** -20 * x.double().abs()).all()), f"dequant_{name}"
        pads = padding_ranges(specs, starts, S, R)
        for buf in (pm.view(torch.int32), pv.view(torch.int32), dm.view(torch.int32), dv.view(torch.int32), qm, qv):
            assert all(bool((buf[b0:e0] == 0).all()) for b0, e0 in pads), "outside the tensors"
        check = (f"ok ({specs[i].name}: m and v pack bit for bit and dequantise within half a code step; "
                 f"padding, codes and values outside the tensors are zero)")
    if not args.no_check and args.mode == "adam8":
        check = "skipped (the Adam step is checked by tests/test_gpu_adam.py)"
    achieved = nbytes[dominant] / dom_avg_s / 1e9
    # counter summaries exist for the fp32 packed buffer only
    traffic = None if args.packed_bf16 else read_traffic((args.workload, args.mode, bool(args.tile_major),
                                                          args.adam_blocks), dominant)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": dominant, "algorithmic_bytes_per_launch": int(nbytes[dominant]),
                "timing": f"mean of {args.steps} flushed launches in the timed region",
                "copy_ceiling_GBps": copy["GBps"] if copy else None,
                "frac_of_copy_ceiling": round(achieved / copy["GBps"], 4) if copy else None}

    log(f"check: {check}")
    cpu = None
    if args.cpu_sample and not w.adam_states and args.mode == "step":
        cpu = cpu_baseline(w, plan, tile_major=bool(args.tile_major))
        cpu["gpu_over_cpu"] = round(value / cpu["value"], 1)
        cpu["gpu_over_single_core"] = round(value / cpu["single_core"]["value"], 1)
        log(f"CPU oracle: {cpu['sample']}")

    names = {0: "tiny group (64x48 1-row blocks, 100x32 16x16 tiles, 7x130 elements; fp32), V=4: unpack + "
                "pack(1/V, accumulate)",
             1: "Llama-3-8B layer (bf16, 128x128 tiles%s), V=64: unpack + pack(1/V, accumulate) + e4m3 tile quant"
                % (" stored tile-major" if args.tile_major else ""),
             2: "Llama-3-70B layer (bf16, whole-matrix blocks), V=1024, 4 ranks materialised: unpack + pack",
             3: "MoE layer (128 experts, bf16, 128x128 tiles), V=256: unpack + pack + e4m3 tile quant",
             4: "8-bit Adam states on the Llama-3-8B layer shapes, 2048-element blocks, V=64: "
                "pack m,v + int8/uint8 quant + dequant"}
    if args.mode == "fp8_gather":
        names = {k: v.split(":")[0] + ": e4m3 quant of the rank slices + fused unpack-dequant to bf16"
                 for k, v in names.items()}
    if args.mode == "adam8":
        names[4] = ("8-bit Adam states on the Llama-3-8B layer shapes, 2048-element blocks, V=64: one fused "
                    "AdamW step (dequant m, v; update fp32 params; requant m int8, v uint8)")
    if args.adam_blocks == "tile32":
        names[4] = names[4].replace("2048-element blocks", "32x32 tiles at 32-row granularity (norms: "
                                                           "2048-element blocks)")
    metric = METRIC if (args.workload == 1 and args.mode == "step" and not args.tile_major
                        and not args.packed_bf16) else \
        f"DBuffer layout transform GB/s (workload {args.workload}, {args.mode}" + \
        (", tile-major" if args.tile_major else "") + (", bf16 packed" if args.packed_bf16 else "") + \
        (", 32x32 Adam blocks" if args.adam_blocks == "tile32" else "") + ")"
    line = {
        "metric": metric,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": names[args.workload], "V": w.V, "S": S, "R_mat": R,
                   "order": order_name, "padding_frac": round(plan.padding / (R * S), 5),
                   "S_over_avg_load": round(S / max(avg_load, 1), 4), "plan_ms": round(plan_ms, 2),
                   "load_ms": round(load_ms, 1), "first_load_ms": round(first_load_ms, 1),
                   "bytes_per_step": int(step_bytes), "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
                   "storage": {0: "fp32 params, grads, prev and packed", 2: "bf16 params, fp32 grads/prev/packed",
                               4: "fp32 m/v, int8/uint8 codes + fp32 scales"}.get(
                       args.workload, "bf16 params, fp32 grads/prev/packed, e4m3 codes + fp32 scales")
                   + ("; the packed buffer is bf16" if args.packed_bf16 else ""),
                   "e4m3_encoder": "sw" if os.environ.get("RS_E4M3_ENCODER") == "sw" else "hw",
                   "launch": "eager" + ("; warm pass: one HIP graph replay per step" if args.graph else "")},
        "timing": f"value: algorithmic bytes of one step over the sum of its kernels' median durations, "
                  f"{args.steps} launches each, every launch after a 1 GiB {args.flush} that empties L2 and the "
                  f"MALL (HIP events on the launch stream; the flush is outside the events)",
        "kernels": per_kernel,
        "warm": warm,
        "copy_ceiling": copy,
        "check": check,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    timer.close()
    plan.close()


if __name__ == "__main__":
    main()
