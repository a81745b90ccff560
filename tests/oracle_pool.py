"""The oracle's block quantisation of whole tensors at full size, spread over
worker processes (test infrastructure).

The oracle quantises one block per call, a few milliseconds per 128x128 tile,
so the 13,312 tiles of the Llama-3-8B layer take most of a minute on one core.
Here each worker process takes one tensor and a list of tile bands (row
ranges that start and end on band boundaries), regenerates the tensor from
its seed, and returns what the oracle computes for those bands:

  * the codes of the bands' interval of the flat buffer (row-major tensors:
    rows r0..r1 of the tensor; tile-major tensors: tile rows r0/br..r1/br,
    which are also one contiguous run),
  * the bands' scales, in scale order,
  * the gather side: the bands' rows rebuilt from those codes and scales and
    rounded to bf16 (row-major bits).

The workers are started with the "spawn" method, so they import only numpy,
the oracle and the input generators: nothing of the HIP runtime or torch
reaches them. Nothing here computes a result of its own; every value comes
from oracle.transform.
"""
from __future__ import annotations

import multiprocessing
from concurrent.futures import ProcessPoolExecutor
from typing import Dict, List, Sequence, Tuple

import numpy as np

from oracle import transform as OT
import workloads as W


def _band_spec(spec, r0: int, r1: int):
    return W.TensorSpec(spec.name, r1 - r0, spec.cols, spec.kind, spec.p0, spec.p1)


def expected_bands(job) -> List[Tuple[int, int, np.ndarray, np.ndarray, np.ndarray]]:
    """job = (workload index, tile-major?, tensor index, fmt, [(r0, r1), ...]).
    Returns [(r0, r1, codes uint8, scale bits uint32, gathered bf16 uint16 (rows, cols))]."""
    widx, tile_major, i, fmt, bands = job
    w = W.workload(widx)
    if tile_major:
        w = W.tile_major_variant(w)
    spec = w.specs[i]
    bits = W.weight_bits(w, i)
    x = W.f32_from_bf16_bits(bits) if bits.dtype == np.uint16 else bits.view(np.float32)
    x = x.reshape(spec.rows, spec.cols)
    from oracle.plan import layout_offsets
    out = []
    for r0, r1 in bands:
        bs = _band_spec(spec, r0, r1)
        flat = np.empty(bs.rows * bs.cols, np.float32)
        flat[layout_offsets(bs)] = x[r0:r1].ravel()          # interval order of the band
        n_blocks = OT.count_quant_blocks([bs])
        q = np.zeros(flat.size, np.uint8)
        sc = np.zeros(n_blocks, np.float32)
        for _, b, pos in OT.quant_blocks([bs], [0]):
            c, s = OT.quantize_block(flat[pos], fmt)
            q[pos] = c
            sc[b] = s
        g = OT.unpack_dequant(q, sc, [bs], [0], fmt, "bf16")[0]
        out.append((r0, r1, q, sc.view(np.uint32), g))
    return out


def band_jobs(widx: int, tile_major: bool, fmt: str, wanted: Dict[int, Sequence[Tuple[int, int]]],
              max_rows_per_job: int = 1024):
    """Split each tensor's band list into jobs of at most max_rows_per_job rows."""
    jobs = []
    for i, bands in wanted.items():
        cur, rows = [], 0
        for r0, r1 in bands:
            cur.append((r0, r1))
            rows += r1 - r0
            if rows >= max_rows_per_job:
                jobs.append((widx, tile_major, i, fmt, cur))
                cur, rows = [], 0
        if cur:
            jobs.append((widx, tile_major, i, fmt, cur))
    return jobs


def run(jobs, workers: int = 0):
    """Yields (tensor index, result list) per job as the workers finish them."""
    workers = workers or W.worker_count()
    ctx = multiprocessing.get_context("spawn")
    with ProcessPoolExecutor(max_workers=min(workers, max(1, len(jobs))), mp_context=ctx) as ex:
        futs = [(job[2], ex.submit(expected_bands, job)) for job in jobs]
        for i, f in futs:
            yield i, f.result()
