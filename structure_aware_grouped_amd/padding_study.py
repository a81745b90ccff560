"""Planner padding study: padding of the host planner's plans for each tensor
order, over row granularities and FSDP sizes ("veScale-FSDP: flexible,
structure-aware sharding at 10K-GPU scale", feynmanwiki walkthrough, the
tensor-order paragraph and the ablation paragraph on planner padding).

    python -m structure_aware_grouped_amd.padding_study [layer ...]

Prints one markdown table per layer: for every row granularity k and FSDP
size V, the padding in % of V*S of the best plan and of the plan of each of
the three orders alone, and the slowest plan time of the row.
"""
from __future__ import annotations

import sys
import time

from workloads.study import STUDY_FSDP_SIZES, STUDY_GRANULARITIES, STUDY_LAYERS

from .binding import rs_plan_build

POLICIES = ("best", "default", "by_block_size", "by_shape")


def padding_pct(specs, V: int, S: int) -> float:
    total = sum(int(s.rows) * int(s.cols) for s in specs)
    return 100.0 * (V * S - total) / (V * S)


def study_point(specs, V: int) -> dict:
    """{policy: (S, padding %, order chosen)} plus the slowest plan time (s)."""
    out, worst = {}, 0.0
    for pol in POLICIES:
        t0 = time.perf_counter()
        S, _, _, name = rs_plan_build(specs, V, policy=pol)
        worst = max(worst, time.perf_counter() - t0)
        out[pol] = (S, padding_pct(specs, V, S), name)
    out["seconds"] = worst
    return out


def table(layer: str) -> str:
    fn = STUDY_LAYERS[layer]
    lines = [f"### {layer}", "",
             "| k | V | best | default | by block size | by shape | best order | plan ms |",
             "|---|---|---|---|---|---|---|---|"]
    for k in STUDY_GRANULARITIES:
        specs = fn(k)
        for V in STUDY_FSDP_SIZES:
            p = study_point(specs, V)
            lines.append(f"| {k} | {V} | " + " | ".join(f"{p[pol][1]:.2f}" for pol in POLICIES) +
                         f" | {p['best'][2]} | {p['seconds'] * 1e3:.0f} |")
    return "\n".join(lines)


def main(argv):
    for layer in (argv or list(STUDY_LAYERS)):
        print(table(layer), flush=True)
        print()


if __name__ == "__main__":
    main(sys.argv[1:])
