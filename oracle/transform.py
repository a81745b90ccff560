"""Unpack, pack, block quantisation and dequantisation, by definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Inputs are the tensor specs, the plan (V, S, starts), the number R_mat of
rank slices actually held in memory (ranks at or past R_mat hold only
padding and are not materialised), and plain arrays. Each function recomputes
the tensor intervals, padding and blocks itself from those inputs.

Readings (listed in the design notes):
  * Unpack ([walk], DBuffer paragraphs: a tensor *is* its planned slice of the
    buffer): T_i[e] = G[s_i + e], bit for bit.
  * Pack ([walk], DBuffer paragraph on fused add / scale / zero / copy before
    a collective): with sigma = fl32(1/V) (or a caller's factor),
    y = fl32(g * sigma) and out = fl32(prev + y) when accumulating, else y:
    scale first, then add, two roundings, no fused multiply-add. Every
    padding position is written as +0.0; padding of prev is never read.
  * Quantisation blocks ([walk], the block-quantisation paragraph: a block
    should sit whole on one device; the 8-bit Adam paragraph's 32x32 blocks at
    32-row granularity): TILE tensors are cut into br x bc tiles of the
    row-major tensor (partial at the right and bottom edges); TILEMAJOR
    tensors into their tiles (contiguous in the buffer); FLAT tensors into
    their b-element blocks. Other kinds are not quantised.
  * Layouts: a tensor occupies [s_i, s_i + n_i); element (r, c) sits at
    s_i + r*cols + c, except for TILEMAJOR tensors, stored tile by tile
    (tile-row-major, each tile row-major inside). Unpack and pack apply that
    reordering ([walk], RaggedShard paragraphs: 2-D blocks may be spread
    unevenly over the devices).
  * Per block: amax = max |x| (exact). If amax > 0 the stored scale is
    fl32(amax / Q) and values are multiplied by r = min(fl32(Q / amax),
    FLT_MAX) before encoding (one correctly rounded division per block; the
    clamp keeps r finite when amax is tiny). If amax == 0 the scale is 1.0 and
    every code is 0. Q = 448 (E4M3), 127 (int8), 255 (uint8).
  * Code bytes outside every quantisation block (padding, unquantised
    tensors) are 0x00. Dequantised values there are +0.0.
  * Scales are ordered by tensor (spec order), then tile row-major / flat
    block index.
  * Fused gather side of FP8 training ([summary] TL;DR and Key claims on
    DeepSeek-V3-style block-wise FP8; [walk] block-quantisation paragraph):
    after the codes and scales are all-gathered, each quantised tensor is
    rebuilt as fl32(decode(code) * scale) at its own positions and, for a
    bf16 parameter, rounded once more to bf16 (nearest, ties to even).
    Tensors that are not quantised are not produced by this step.
"""
from __future__ import annotations

from typing import Iterator, List, Sequence, Tuple

import numpy as np

from . import codes
from .plan import layout_offsets, numel, padding_ranges

FLT_MAX = float(np.finfo(np.float32).max)


def f32(x) -> np.ndarray:
    """Round float64 values to float32 (nearest, ties to even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def inv_v(V: int) -> np.float32:
    """sigma = fl32(1/V), correctly rounded."""
    return np.float32(np.float64(1.0) / np.float64(V))


# ---------------------------------------------------------------- unpack

def unpack(G: np.ndarray, specs, starts) -> List[np.ndarray]:
    """Full tensors from the gathered flat buffer: T_i[e] = G[s_i + L_i(e)] (any dtype,
    bitwise), L_i the tensor's layout (identity, or tile-major for TILEMAJOR)."""
    out = []
    for spec, s in zip(specs, starts):
        out.append(np.array(G[int(s) + layout_offsets(spec)]).reshape(spec.rows, spec.cols))
    return out


# ---------------------------------------------------------------- pack

def pack_values(g: np.ndarray, prev, sigma, accumulate: bool) -> np.ndarray:
    """fl32(g * sigma), then fl32(prev + that) when accumulating."""
    y = f32(np.asarray(g, dtype=np.float32).astype(np.float64) * np.float64(np.float32(sigma)))
    if accumulate:
        y = f32(np.asarray(prev, dtype=np.float32).astype(np.float64) + y.astype(np.float64))
    return y


def pack(grads: Sequence[np.ndarray], prev, specs, starts, S: int, R_mat: int,
         sigma, accumulate: bool) -> np.ndarray:
    """Packed flat fp32 buffer of R_mat*S values; padding is +0.0."""
    out = np.zeros(R_mat * S, dtype=np.float32)
    for g, spec, s in zip(grads, specs, starts):
        pos = int(s) + layout_offsets(spec)
        p = prev[pos] if accumulate else None
        out[pos] = pack_values(np.ravel(g), p, sigma, accumulate)
    return out


def pack_to_bf16(grads: Sequence[np.ndarray], prev, specs, starts, S: int, R_mat: int,
                 sigma, accumulate: bool) -> np.ndarray:
    """The packed buffer for a bf16 ReduceScatter (mixed-precision training): every
    fp32 value of `pack` rounded once to the nearest bf16, ties to even; uint16 bits,
    padding +0.0. Reading: the pages fuse the copy with the pre-communication ops
    (walkthrough, DBuffer paragraphs) and train in mixed precision (end-to-end
    paragraphs) without naming the reduce dtype; a bf16 buffer takes the fp32
    result of the fused ops and rounds it once, so no intermediate is bf16."""
    return bf16_round(pack(grads, prev, specs, starts, S, R_mat, sigma, accumulate))


# ---------------------------------------------------------------- quant blocks

def quant_blocks(specs, starts) -> Iterator[Tuple[int, int, np.ndarray]]:
    """(tensor index, scale index, flat positions) of every quantisation block, in scale order."""
    q = 0
    for i, (spec, s) in enumerate(zip(specs, starts)):
        s = int(s)
        if spec.kind == "TILE":
            br, bc = int(spec.p0), int(spec.p1)
            r, c = int(spec.rows), int(spec.cols)
            for r0 in range(0, r, br):
                rows = np.arange(r0, min(r0 + br, r), dtype=np.int64)
                for c0 in range(0, c, bc):
                    cols = np.arange(c0, min(c0 + bc, c), dtype=np.int64)
                    yield i, q, s + (rows[:, None] * c + cols[None, :]).ravel()
                    q += 1
        elif spec.kind == "FLAT":
            b, n = int(spec.p0), numel(spec)
            for e0 in range(0, n, b):
                yield i, q, s + np.arange(e0, min(e0 + b, n), dtype=np.int64)
                q += 1
        elif spec.kind == "TILEMAJOR":   # whole tiles, each contiguous, tile-row-major
            tsz = int(spec.p0) * int(spec.p1)
            for t in range(numel(spec) // tsz):
                yield i, q, s + t * tsz + np.arange(tsz, dtype=np.int64)
                q += 1


def count_quant_blocks(specs) -> int:
    total = 0
    for spec in specs:
        if spec.kind in ("TILE", "TILEMAJOR"):
            total += (-(-int(spec.rows) // int(spec.p0))) * (-(-int(spec.cols) // int(spec.p1)))
        elif spec.kind == "FLAT":
            total += -(-numel(spec) // int(spec.p0))
    return total


# quiet NaN, sign clear, no payload: the scale of a block that holds a NaN
SCALE_NAN = np.uint32(0x7FC00000).view(np.float32)


def quantize_block(x, fmt: str) -> Tuple[np.ndarray, np.float32]:
    """Codes and scale of one block of fp32 values.

    A block whose values include a NaN or an infinity cannot be scaled (the pages
    assume finite values; reading): its amax, taken with NaN propagating, is NaN or
    +inf; its scale is a quiet NaN (0x7FC00000) or +inf; every code is 0x00, so its
    dequantised values are all NaN (0 x NaN, 0 x inf) and a divergence stays visible."""
    x = np.asarray(x, dtype=np.float32)
    Q = codes.FORMAT_QMAX[fmt]
    with np.errstate(invalid="ignore"):       # a signalling NaN widens quietly
        amax = float(np.max(np.abs(x.astype(np.float64)))) if x.size else 0.0
    if amax == 0.0:
        return np.zeros(x.shape, dtype=np.uint8), np.float32(1.0)
    if not np.isfinite(amax):
        return np.zeros(x.shape, dtype=np.uint8), (SCALE_NAN if np.isnan(amax) else np.float32(np.inf))
    scale = np.float32(amax / Q)
    with np.errstate(over="ignore"):          # Q / amax may overflow fp32: clamp below
        r = min(float(np.float32(Q / amax)), FLT_MAX)
    y = f32(x.astype(np.float64) * r)
    return codes.encode(y, fmt), scale


def block_quant(src: np.ndarray, specs, starts, S: int, R_mat: int, fmt: str):
    """Codes (R_mat*S bytes) and scales of every quantisation block of the flat buffer.

    ``src`` holds fp32 values of the flat buffer (bf16 inputs widened exactly).
    """
    q = np.zeros(R_mat * S, dtype=np.uint8)
    scales = np.zeros(count_quant_blocks(specs), dtype=np.float32)
    for _, b, pos in quant_blocks(specs, starts):
        c, sc = quantize_block(src[pos], fmt)
        q[pos] = c
        scales[b] = sc
    return q, scales


def dequant_values(c, scale, fmt: str) -> np.ndarray:
    """fl32(decode(code) * scale)."""
    with np.errstate(invalid="ignore"):       # 0 x inf of a non-finite block is NaN
        return f32(codes.decode(c, fmt) * np.float64(np.float32(scale)))


def block_dequant(q: np.ndarray, scales, specs, starts, S: int, R_mat: int, fmt: str) -> np.ndarray:
    out = np.zeros(R_mat * S, dtype=np.float32)
    for _, b, pos in quant_blocks(specs, starts):
        out[pos] = dequant_values(q[pos], scales[b], fmt)
    return out


# ---------------------------------------------------------------- gather side

def bf16_round(x) -> np.ndarray:
    """Nearest bf16 of each fp32, ties to the even bf16 mantissa; uint16 bits.

    Finite x: the two candidates are x's bits truncated to the top 16 and the
    next bf16 step up in magnitude; the nearer one wins, a tie goes to the one
    whose lowest kept bit is 0. A candidate past the largest finite bf16 is
    infinity and is weighed as 2^128, the value the next step would have
    (IEEE 754 overflow under round to nearest: from the midpoint between the
    largest finite bf16 and 2^128 on, the result is infinity). Infinities are
    kept. NaN stays NaN (reading, the pages name no NaN rule): its sign and
    top seven payload bits are kept and the quiet bit 0x0040 is set, so no
    NaN payload can carry into the exponent and turn into a number."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lo = u & np.uint32(0xFFFF0000)
    hi = lo + np.uint32(0x10000)
    hi_exp_all_ones = (hi & np.uint32(0x7F800000)) == np.uint32(0x7F800000)
    with np.errstate(invalid="ignore"):   # NaN inputs, and NaN bit patterns among the candidates
        a = np.abs(x.astype(np.float64))
        lo_mag = np.abs(lo.view(np.float32).astype(np.float64))
        hi_mag = np.where(hi_exp_all_ones, 2.0 ** 128, np.abs(hi.view(np.float32).astype(np.float64)))
    finite = np.isfinite(a)
    a_f = np.where(finite, a, 0.0)
    d_lo = np.where(finite, a_f - np.where(finite, lo_mag, 0.0), 0.0)
    d_hi = np.where(finite, hi_mag - a_f, 1.0)
    pick_hi = finite & ((d_hi < d_lo) | ((d_hi == d_lo) & ((lo >> np.uint32(16)) & np.uint32(1)).astype(bool)))
    out = (np.where(pick_hi, hi, lo) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    return np.where(nan, ((u >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16), out)


def unpack_dequant(q: np.ndarray, scales, specs, starts, fmt: str, out: str):
    """Full tensors rebuilt from gathered codes and scales; None for tensors that are not
    quantised. out: "f32" (fp32 values) or "bf16" (uint16 bit patterns)."""
    full = {}
    for i, b, pos in quant_blocks(specs, starts):
        v = dequant_values(q[pos], scales[b], fmt)
        full.setdefault(i, np.zeros(numel(specs[i]), dtype=np.float32))[pos - int(starts[i])] = v
    for i in full:   # interval order -> row-major order
        full[i] = full[i][layout_offsets(specs[i])]
    res = []
    for i, spec in enumerate(specs):
        if i not in full:
            res.append(None)
            continue
        v = full[i].reshape(spec.rows, spec.cols)
        res.append(bf16_round(v) if out == "bf16" else v)
    return res


__all__ = [
    "bf16_round", "unpack_dequant",
    "f32", "inv_v", "unpack", "pack_values", "pack", "quant_blocks", "count_quant_blocks",
    "quantize_block", "block_quant", "dequant_values", "block_dequant", "padding_ranges",
]
