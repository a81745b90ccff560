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
once) per second of wall time over the K timed steps. Per-kernel durations
come from HIP events recorded on the stream the kernels run on. The CPU
baseline times the CPU oracle on a bounded sample of the same workload.
Prints one JSON line.
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
METRIC = "DBuffer pack/unpack+blockquant GB/s, % HBM peak (Llama-3-8B layer, V=64)"
# committed counter summaries: (workload, mode, tile-major) -> profiles/traffic_<name>.md
PROFILE_TRAFFIC = {(1, "step", False): "llama3_8b_v64", (1, "step", True): "llama3_8b_v64_tile_major",
                   (1, "fp8_gather", False): "llama3_8b_v64_fp8_gather", (4, "adam8", False): "adam8_llama3_8b_v64",
                   (2, "step", False): "llama3_70b_v1024", (3, "step", False): "moe128_v256",
                   (4, "step", False): "adam_states_llama3_8b_v64",
                   (3, "fp8_gather", False): "moe128_v256_fp8_gather",
                   (1, "fp8_gather", True): "llama3_8b_v64_tile_major_fp8_gather"}
KERNEL_SOURCES = [os.path.join(ROOT, "structure_aware_grouped_amd", "csrc", f)
                  for f in ("device_common.h", "host_common.h", "transform.hip", "quant.hip", "gather.hip",
                            "adam.hip", "rs_internal.h", "plan.cpp")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=1, choices=[0, 1, 2, 3, 4],
                    help="0 is the tiny three-tensor group: launch-bound, a parity case more than a bandwidth one")
    ap.add_argument("--mode", default="step", choices=["step", "fp8_gather", "adam8"],
                    help="step: the workload's steps; fp8_gather: block quant of the rank slices, then "
                         "the fused unpack-dequant of the codes into the bf16 tensors; adam8 (workload 4): "
                         "one AdamW step on the int8/uint8 block-quantised m and v")
    ap.add_argument("--tile-major", action="store_true",
                    help="store the TILE tensors tile by tile (TILEMAJOR): unpack and pack reorder through LDS")
    ap.add_argument("--packed-bf16", action="store_true",
                    help="pack into a bf16 buffer (a bf16 ReduceScatter): each fp32 result rounded once")
    ap.add_argument("--cpu-sample", type=int, default=1, help="0 disables the CPU-oracle baseline")
    ap.add_argument("--no-check", action="store_true", help="skip the sampled output checks")
    ap.add_argument("--cold-steps", type=int, default=5,
                    help="launches per kernel of the cold-cache pass after the timed region (0: skip)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph after the warm-up and replay it in the timed region "
                         "(the per-kernel and cold passes stay eager)")
    ap.add_argument("--fenced-events", action="store_true",
                    help="time with default HIP events (system-scope fence at every record)")
    ap.add_argument("--copy-mib", type=int, default=1024,
                    help="size of the device-to-device copy timed as the practical ceiling "
                         "(and used to calibrate HBM byte counters); 0 disables it")
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


def log(msg: str):
    """A progress line on stderr (the JSON result line goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_baseline(w, plan, names=None, max_seconds: float = 15.0) -> dict:
    """The CPU oracle (single-threaded NumPy) on a bounded sample of the workload:
    the tensors named in `names` (default: every tensor, i.e. one whole step),
    one at a time and in order, until `max_seconds` of oracle time have passed
    (the Llama-3-8B and Llama-3-70B layers finish whole; the MoE layer stops
    after its first experts), with the bench's byte accounting. Inputs are
    generated before the clock starts."""
    from oracle import transform as OT
    from workloads.device import Inputs
    import workloads as W

    names = [sp.name for sp in w.specs] if names is None else list(names)
    idx = [i for i, sp in enumerate(w.specs) if sp.name in names]
    inp = Inputs(w, plan.S, plan.starts, plan.R_mat, device="cpu")
    pb = 2 if w.param_dtype == "bf16" else 4
    sigma = OT.inv_v(w.V)
    moved, dt, done = 0, 0.0, []
    for i in idx:
        if dt >= max_seconds:
            break
        done.append(i)
        spec, s = w.specs[i], plan.starts[i]
        wb, g, p = inp.weight_bits(i), inp.grad(i), inp.prev_range(s, s + spec.numel)
        t0 = time.perf_counter()
        n = spec.numel
        # unpack: the tensor is its slice of the gathered buffer
        OT.unpack(wb, [spec], [0])
        moved += 2 * n * pb
        # pack: scale, accumulate
        OT.pack_values(g.ravel(), p, sigma, True)
        moved += n * 12
        # quant: every tile of the tensor
        if spec.kind in ("TILE", "TILEMAJOR", "FLAT") and w.quant:
            x = W.f32_from_bf16_bits(wb) if wb.dtype == np.uint16 else wb.view(np.float32)
            for _, b, pos in OT.quant_blocks([spec], [0]):
                OT.quantize_block(x[pos], w.quant)
            moved += n * pb + n + 4 * OT.count_quant_blocks([spec])
        dt += time.perf_counter() - t0
    if len(done) == len(w.specs):
        what = "every tensor of the layer (one whole step)"
    elif len(done) <= 4:
        what = ", ".join(w.specs[i].name for i in done)
    else:
        what = f"the first {len(done)} of the layer's {len(w.specs)} tensors"
    return {"value": round(moved / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{what}: unpack + pack{' + e4m3 tile quant' if w.quant else ''}, "
                      + (f"{moved / 1e9:.3f} GB in {dt:.1f} s" if moved >= 1e8 else
                         f"{moved / 1e6:.3f} MB in {dt * 1e3:.2f} ms")}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the V logical ranks are slices of one device buffer "
              f"and no collective is run (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import structure_aware_grouped_amd as rs
    from workloads.device import Inputs, garbage, tensor_bits
    from workloads import Role, tensor_values, tile_major_variant, workload

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    w = workload(args.workload)
    if args.tile_major:
        w = tile_major_variant(w)
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

    copy = None
    if args.copy_mib:
        # a plain device-to-device copy of known size: the practical HBM ceiling, and the
        # reference whose counter readings calibrate FETCH_SIZE / WRITE_SIZE
        nb = args.copy_mib << 20
        src_c = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
        dst_c = torch.empty_like(src_c)
        ms = []
        for _ in range(6):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            dst_c.copy_(src_c)
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        best = float(np.median(ms[1:]))
        copy = {"bytes": 2 * nb, "median_ms": round(best, 4), "GBps": round(2 * nb / (best * 1e-3) / 1e9, 1)}
        del src_c, dst_c

    for _ in range(args.warmup):
        for _, fn in steps:
            fn()
    torch.cuda.synchronize()

    # ---- timed region: K steps. HIP events, on the stream the library launches on
    # (torch's current stream, which the binding passes), bracket the dominant kernel
    # only: every event record adds idle GPU time at a kernel boundary, so the other
    # kernels are timed in the pass that follows.
    # With --graph the whole step is one captured HIP graph (the warm-up has made the
    # calls with these pointers, so the capture holds kernel launches only) and the
    # events bracket each replay.
    stream = torch.cuda.current_stream(dev).cuda_stream
    timer = HipTimer(torch, fenced=args.fenced_events)
    graph = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _, fn in steps:
                fn()
        graph.replay()
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
    log(f"timed region: {args.steps} steps in {wall * 1e3:.1f} ms")
    dom_ms = [timer.ms(a, b) for a, b in dom_ev]
    del graph

    # ---- per-kernel pass, right after the timed region and under the same warm
    # conditions: HIP events around every launch
    kev = [[(timer.event(), timer.event()) for _ in steps] for _ in range(args.steps)]
    for k in range(args.steps):
        for (name, fn), (a, b) in zip(steps, kev[k]):
            timer.record(a, stream)
            fn()
            timer.record(b, stream)
    torch.cuda.synchronize()
    per_kernel = {}
    for j, (name, _) in enumerate(steps):
        ms = [timer.ms(kev[k][j][0], kev[k][j][1]) for k in range(args.steps)]
        avg = float(np.mean(ms))
        per_kernel[name] = {"avg_ms": round(avg, 5), "median_ms": round(float(np.median(ms)), 5),
                            "min_ms": round(float(np.min(ms)), 5),
                            "GBps": round(nbytes[name] / (avg * 1e-3) / 1e9, 1),
                            "bytes": int(nbytes[name])}
    graph_info = None
    if args.graph:   # events around each replay: the whole step
        graph_info = {"replay_avg_ms": round(float(np.mean(dom_ms)), 5),
                      "replay_min_ms": round(float(np.min(dom_ms)), 5)}
    else:
        per_kernel[dominant]["timed_region_avg_ms"] = round(float(np.mean(dom_ms)), 5)
    step_bytes = sum(nbytes[name] for name, _ in steps)
    ms_per_step = wall / args.steps * 1e3
    value = step_bytes / (wall / args.steps) / 1e9

    # ---- cold-cache pass, after and outside the timed region: before every launch a
    # 1 GiB scratch buffer is written (outside the events), so neither L2 nor the
    # 256 MB MALL holds anything the kernel reads
    cold = None
    if args.cold_steps:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cev = [[(timer.event(), timer.event()) for _ in steps] for _ in range(args.cold_steps)]
        for k in range(args.cold_steps):
            for (name, fn), (a, b) in zip(steps, cev[k]):
                flush.fill_(k & 0xFF)
                timer.record(a, stream)
                fn()
                timer.record(b, stream)
        torch.cuda.synchronize()
        cold = {"label": f"cold L2 and MALL: a 1 GiB buffer written before each launch, "
                         f"{args.cold_steps} launches per kernel, median"}
        for j, (name, _) in enumerate(steps):
            ms = [timer.ms(cev[k][j][0], cev[k][j][1]) for k in range(args.cold_steps)]
            med = float(np.median(ms))
            cold[name] = {"median_ms": round(med, 5), "min_ms": round(float(np.min(ms)), 5),
                          "GBps": round(nbytes[name] / (med * 1e-3) / 1e9, 1)}
        del flush

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
        # sampled checks that need no oracle (the oracle parity tests live in tests/): the
        # second tensor unpacks to its generated weights, padding is +0.0, codes outside
        # blocks are 0, scales are finite and positive
        i = 1
        assert np.array_equal(tensor_bits(params[i]).ravel(), inp.weight_bits(i)), "unpack"
        pads = padding_ranges(specs, starts, S, R)
        pk = packed.view(torch.int16 if args.packed_bf16 else torch.int32)
        assert all(bool((pk[b:e] == 0).all()) for b, e in pads), "pack padding"
        if w.quant:
            assert all(bool((q[b:e] == 0).all()) for b, e in pads), "codes outside blocks"
            sf = scales.float()
            assert bool(torch.isfinite(sf).all()) and bool((sf > 0).all()), "scales"
        check = f"ok ({specs[i].name} unpacks to its weights; padding and codes outside blocks are zero)"
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
    # the dominant kernel inside the timed region (inside a graph replay it has no events
    # of its own: then its eager per-kernel average)
    dom_avg_s = (per_kernel[dominant]["avg_ms"] if args.graph else float(np.mean(dom_ms))) * 1e-3
    achieved = nbytes[dominant] / dom_avg_s / 1e9
    # counter summaries exist for the fp32 packed buffer only
    traffic = None if args.packed_bf16 else read_traffic((args.workload, args.mode, bool(args.tile_major)), dominant)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": dominant, "algorithmic_bytes_per_launch": int(nbytes[dominant])}

    log(f"check: {check}")
    cpu = None
    if args.cpu_sample and not w.adam_states and args.mode == "step":
        cpu = cpu_baseline(w, plan)
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
    metric = METRIC if (args.workload == 1 and args.mode == "step" and not args.tile_major
                        and not args.packed_bf16) else \
        f"DBuffer layout transform GB/s (workload {args.workload}, {args.mode}" + \
        (", tile-major" if args.tile_major else "") + (", bf16 packed" if args.packed_bf16 else "") + ")"
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
                   "launch": "one HIP graph replay per step" if args.graph else "eager"},
        "kernels": per_kernel,
        "graph": graph_info,
        "cold_cache": cold,
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
