"""The five workloads, as data.

Each workload is a group of tensors that share one flat buffer split into V
equal rank slices. A tensor is described by its 2-D shape and the kind of
atomic block that must never be cut by a rank boundary (one element, k rows,
a br x bc tile, a flat run of b elements, or the whole tensor). A 1-D tensor
of n elements is given as (n, 1): its dim-0 unit is one element.

Shapes follow the public architectures the pages train (Llama-3 8B/70B dense
layers and a GPT-OSS-120B-style MoE layer with 128 experts); values are
synthetic and seeded (see ``gen``).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class TensorSpec:
    name: str
    rows: int
    cols: int
    kind: str          # "ELEM" | "ROWS" | "TILE" | "FLAT" | "WHOLE" | "TILEMAJOR"
    p0: int = 0        # ROWS: rows per block; TILE / TILEMAJOR: block rows; FLAT: block elements
    p1: int = 0        # TILE / TILEMAJOR: block columns

    @property
    def numel(self) -> int:
        return self.rows * self.cols


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    specs: Tuple[TensorSpec, ...]
    V: int
    param_dtype: str                 # dtype of the gathered parameter buffer: "f32" | "bf16"
    weight_dist: Tuple               # ("uniform", lo, hi) | ("normal", sigma)
    grad_dist: Tuple
    prev_dist: Tuple
    accumulate: bool                 # pack adds into a previous packed buffer
    inv_v_scale: bool                # pack scales by 1/V (else by 1)
    quant: Optional[str] = None      # "e4m3" on the parameter buffer, or None
    adam_states: bool = False        # pack + 8-bit quant of fp32 Adam m and v
    materialize_all_ranks: bool = True   # False: trailing all-padding ranks stay implicit
    steps: Tuple[str, ...] = field(default_factory=tuple)


def _llama_layer(hidden: int, kv: int, ffn: int, kind: str, p0: int = 0, p1: int = 0,
                 norm_kind: str = "ROWS", norm_p0: int = 1):
    mats = (
        TensorSpec("wq", hidden, hidden, kind, p0, p1),
        TensorSpec("wk", kv, hidden, kind, p0, p1),
        TensorSpec("wv", kv, hidden, kind, p0, p1),
        TensorSpec("wo", hidden, hidden, kind, p0, p1),
        TensorSpec("gate", ffn, hidden, kind, p0, p1),
        TensorSpec("up", ffn, hidden, kind, p0, p1),
        TensorSpec("down", hidden, ffn, kind, p0, p1),
    )
    norms = (
        TensorSpec("attn_norm", hidden, 1, norm_kind, norm_p0 if norm_kind == "ROWS" else 0),
        TensorSpec("mlp_norm", hidden, 1, norm_kind, norm_p0 if norm_kind == "ROWS" else 0),
    )
    return mats + norms


def _moe_layer(experts: int = 128, hidden: int = 2880, inter: int = 2880):
    specs = []
    for e in range(experts):
        specs.append(TensorSpec(f"e{e}.gate_up", 2 * inter, hidden, "TILE", 128, 128))
        specs.append(TensorSpec(f"e{e}.down", hidden, inter, "TILE", 128, 128))
    specs.append(TensorSpec("router", experts, hidden, "TILE", 128, 128))
    return tuple(specs)


def _flat_states(specs, b: int = 2048):
    return tuple(TensorSpec(s.name, s.rows, s.cols, "FLAT", b) for s in specs)


_W = (
    Workload(
        index=0,
        name="tiny: 3 fp32 tensors (64x48 row blocks, 100x32 16x16 tiles, 7x130 elements), V=4",
        specs=(
            TensorSpec("t64x48", 64, 48, "ROWS", 1),
            TensorSpec("t100x32", 100, 32, "TILE", 16, 16),
            TensorSpec("t7x130", 7, 130, "ELEM"),
        ),
        V=4, param_dtype="f32",
        weight_dist=("uniform", -1.0, 1.0), grad_dist=("uniform", -1.0, 1.0),
        prev_dist=("uniform", -1.0, 1.0),
        accumulate=True, inv_v_scale=True, quant=None,
        steps=("unpack", "pack"),
    ),
    Workload(
        index=1,
        name="Llama-3-8B layer, bf16, 128x128 tiles, V=64",
        specs=_llama_layer(4096, 1024, 14336, "TILE", 128, 128),
        V=64, param_dtype="bf16",
        weight_dist=("normal", 0.02), grad_dist=("normal", 1e-3), prev_dist=("normal", 1e-3),
        accumulate=True, inv_v_scale=True, quant="e4m3",
        steps=("unpack", "pack", "quant"),
    ),
    Workload(
        index=2,
        name="Llama-3-70B layer, bf16, whole-matrix blocks, V=1024",
        specs=_llama_layer(8192, 1024, 28672, "WHOLE", norm_kind="WHOLE"),
        V=1024, param_dtype="bf16",
        weight_dist=("normal", 0.02), grad_dist=("normal", 1e-3), prev_dist=("normal", 1e-3),
        accumulate=True, inv_v_scale=True, quant=None, materialize_all_ranks=False,
        steps=("unpack", "pack"),
    ),
    Workload(
        index=3,
        name="MoE layer (128 experts, gate_up 5760x2880, down 2880x2880, router 128x2880), "
             "bf16, 128x128 tiles, V=256",
        specs=_moe_layer(),
        V=256, param_dtype="bf16",
        weight_dist=("normal", 0.02), grad_dist=("normal", 1e-3), prev_dist=("normal", 1e-3),
        accumulate=True, inv_v_scale=True, quant="e4m3",
        steps=("unpack", "pack", "quant"),
    ),
    Workload(
        index=4,
        name="8-bit Adam states (fp32 m, v) on the Llama-3-8B layer shapes, 2048-element "
             "flat blocks, V=64",
        specs=_flat_states(_llama_layer(4096, 1024, 14336, "TILE", 128, 128)),
        V=64, param_dtype="f32",
        weight_dist=("normal", 1e-3), grad_dist=("normal", 1e-3), prev_dist=("normal", 1e-3),
        accumulate=False, inv_v_scale=False, quant=None, adam_states=True,
        steps=("pack_m", "pack_v", "quant_m", "quant_v", "dequant_m", "dequant_v"),
    ),
)

WORKLOADS = {w.index: w for w in _W}


def workload(index: int) -> Workload:
    return WORKLOADS[index]


def tiny_variant(base: Workload, **changes) -> Workload:
    """A copy of a workload with some fields changed (for parity-only variants)."""
    return replace(base, **changes)


def adam_tile32_variant(w: Workload) -> Workload:
    """The Adam-state workload with the pages' own 8-bit Adam blocks: every matrix in
    32x32 tiles (so 32-row rank granularity), 1-D tensors in 2048-element flat blocks."""
    specs = tuple(TensorSpec(s.name, s.rows, s.cols, "TILE", 32, 32) if s.rows > 1 and s.cols > 1 else s
                  for s in w.specs)
    return replace(w, specs=specs, name=w.name.replace("2048-element flat blocks",
                                                       "32x32 tiles (1-D tensors: 2048-element flat blocks)"))


def tile_major_variant(w: Workload) -> Workload:
    """The same workload with every TILE tensor stored tile by tile (TILEMAJOR, same tiles)."""
    specs = tuple(TensorSpec(s.name, s.rows, s.cols, "TILEMAJOR", s.p0, s.p1) if s.kind == "TILE" else s
                  for s in w.specs)
    return replace(w, specs=specs, name=w.name.replace("128x128 tiles", "128x128 tiles stored tile-major"))
