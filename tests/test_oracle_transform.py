"""Pins of the oracle's unpack / pack / quant / dequant.

  * fp32 arithmetic against exact rationals rounded by IEEE's definition
    (tests/exact.py), for the 1/V factor, scale-then-add, the per-block scale
    and reciprocal, the scaled values and their codes.
  * closed forms: V a power of two makes g/V exact; the element attaining
    amax maps to +-Q; an all-zero block has scale 1 and zero codes.
  * invariants: padding comes out +0.0 without reading prev's padding;
    unpack(pack(x, 1, no accumulate)) == x bit for bit; every quantisation
    block position is covered exactly once and never crosses a rank; the
    dequantised values stay within the rounding bound of the code grid.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import codes, plan as P, transform as T
from tests import exact
from workloads import TensorSpec, workload
import workloads as W


def _bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


@pytest.mark.parametrize("V", [1, 2, 3, 5, 6, 7, 64, 100, 1024, 4097])
def test_inv_v_is_correctly_rounded(V):
    assert T.inv_v(V) == np.float32(exact.round_f32(Fraction(1, V)))


@pytest.mark.parametrize("V,acc", [(3, True), (7, False), (64, True), (5, True), (1024, True)])
def test_pack_values_exact(V, acc):
    rng = np.random.default_rng(V)
    g = (rng.standard_normal(400) * 10.0 ** rng.integers(-6, 3, 400)).astype(np.float32)
    prev = (rng.standard_normal(400) * 10.0 ** rng.integers(-6, 3, 400)).astype(np.float32)
    g[:4] = np.float32([0.0, -0.0, 1e-41, -3e-39])     # signed zero and subnormals
    sigma = T.inv_v(V)
    got = T.pack_values(g, prev, sigma, acc)
    for k in range(g.size):
        y = exact.round_f32(Fraction(float(g[k])) * Fraction(float(sigma)),
                            negative_zero=bool(np.signbit(g[k])))
        if acc:
            y = exact.round_f32(Fraction(float(prev[k])) + Fraction(y),
                                negative_zero=bool(np.signbit(prev[k]) and np.signbit(y)))
        assert _bits(got[k]) == exact.f32_bits(y), (k, g[k], prev[k])


def test_pack_power_of_two_V_is_exact_scaling():
    rng = np.random.default_rng(1)
    g = rng.standard_normal(1000).astype(np.float32)
    y = T.pack_values(g, None, T.inv_v(64), False)
    e_g = (_bits(g) >> 23) & 0xFF
    assert np.array_equal((_bits(y) >> 23) & 0xFF, e_g - 6)          # exponent drops by 6
    assert np.array_equal(_bits(y) & 0x807FFFFF, _bits(g) & 0x807FFFFF)  # sign, mantissa kept


def _tiny_plan():
    w = workload(0)
    p = P.plan(w.specs, w.V)
    return w, p


def test_pack_zeroes_padding_and_ignores_prev_padding():
    w, p = _tiny_plan()
    S, R = p.S, w.V
    grads = [W.tensor_values(w, i, W.Role.GRAD) for i in range(3)]
    prev = np.concatenate([W.prev_slice(w, k, S) for k in range(R)])
    pads = P.padding_ranges(w.specs, p.starts, S, R)
    assert pads
    poisoned = prev.copy()
    for b, e in pads:
        poisoned[b:e] = np.nan
    out = T.pack(grads, poisoned, w.specs, p.starts, S, R, T.inv_v(w.V), True)
    ref = T.pack(grads, prev, w.specs, p.starts, S, R, T.inv_v(w.V), True)
    assert np.array_equal(_bits(out), _bits(ref))
    for b, e in pads:
        assert np.all(_bits(out[b:e]) == 0)
    covered = sum(e - b for b, e in pads) + sum(s.numel for s in w.specs)
    assert covered == R * S


def test_unpack_of_pack_is_identity():
    w, p = _tiny_plan()
    x = [W.tensor_values(w, i, W.Role.WEIGHT) for i in range(3)]
    flat = T.pack(x, None, w.specs, p.starts, p.S, w.V, np.float32(1.0), False)
    back = T.unpack(flat, w.specs, p.starts)
    for a, b in zip(x, back):
        assert np.array_equal(_bits(a), _bits(b))
        assert b.shape == a.shape


def _exact_quant(x, fmt):
    """Codes and scale of one block by exact arithmetic and exhaustive nearest-code search."""
    Q = {"e4m3": 448, "i8": 127, "u8": 255}[fmt]
    amax = max(abs(Fraction(float(v))) for v in x)
    if amax == 0:
        return [0] * len(x), 1.0
    scale = exact.round_f32(amax / Q)
    r = exact.round_f32(Fraction(Q) / amax)
    r = min(r, float(np.finfo(np.float32).max))
    out = []
    for v in x:
        y = exact.round_f32(Fraction(float(v)) * Fraction(r), negative_zero=bool(np.signbit(v)))
        if fmt == "e4m3":
            out.append(exact.e4m3_nearest(y))
        elif fmt == "i8":
            out.append(exact.int_nearest(y, -127, 127) & 0xFF)
        else:
            out.append(exact.int_nearest(y, 0, 255))
    return out, scale


@pytest.mark.parametrize("fmt", ["e4m3", "i8", "u8"])
@pytest.mark.parametrize("seed", range(6))
def test_quantize_block_exact(fmt, seed):
    rng = np.random.default_rng(seed)
    mag = 10.0 ** rng.integers(-30, 4)
    x = (rng.standard_normal(96) * mag).astype(np.float32)
    if fmt == "u8":
        x = np.abs(x)
    if seed == 0:
        x[5] = -0.0
    c, sc = T.quantize_block(x, fmt)
    want_c, want_s = _exact_quant(x, fmt)
    assert list(c) == want_c
    assert _bits(sc) == exact.f32_bits(want_s)


@pytest.mark.parametrize("fmt,Q,code", [("e4m3", 448, 0x7E), ("i8", 127, 127), ("u8", 255, 255)])
def test_amax_element_maps_to_Q(fmt, Q, code):
    rng = np.random.default_rng(5)
    for _ in range(50):
        x = np.abs(rng.standard_normal(64).astype(np.float32)) * np.float32(10.0 ** rng.integers(-20, 20))
        k = int(np.argmax(x))
        c, _ = T.quantize_block(x, fmt)
        assert c[k] == code
        if fmt != "u8":
            c2, _ = T.quantize_block(-x, fmt)
            assert c2[k] == ((code | 0x80) if fmt == "e4m3" else (-Q) & 0xFF)


def test_zero_block_and_tiny_block():
    c, s = T.quantize_block(np.zeros(40, np.float32), "e4m3")
    assert s == np.float32(1.0) and not c.any()
    # amax so small that Q/amax overflows fp32: r is clamped to FLT_MAX, zeros stay zero
    x = np.float32([1e-41, 0.0, -5e-42, -0.0])
    c, s = T.quantize_block(x, "e4m3")
    want_c, want_s = _exact_quant(x, "e4m3")
    assert list(c) == want_c and _bits(s) == exact.f32_bits(want_s)
    assert c[1] == 0x00 and c[3] == 0x80


@pytest.mark.parametrize("fmt", ["e4m3", "i8", "u8"])
def test_blocks_with_nan_or_infinity(fmt):
    """Reading: a block holding a NaN or an infinity gets amax NaN (NaN propagates, as
    torch.amax does) or +inf, scale 0x7FC00000 or +inf, and all-zero codes; it dequantises
    to NaN everywhere. Finite blocks beside it are untouched."""
    import torch
    rng = np.random.default_rng(31)
    base = rng.standard_normal(64).astype(np.float32)
    nan_bits = np.uint32([0x7FC00000, 0xFFC00000, 0x7F800001, 0x7FFFFFFF]).view(np.float32)
    for bad, want_scale in [(nan_bits[0], 0x7FC00000), (nan_bits[1], 0x7FC00000), (nan_bits[2], 0x7FC00000),
                            (nan_bits[3], 0x7FC00000), (np.float32(np.inf), 0x7F800000),
                            (np.float32(-np.inf), 0x7F800000)]:
        for where in (0, 17, 63):
            x = base.copy()
            x[where] = bad
            amax = torch.amax(torch.abs(torch.from_numpy(x))).item()
            assert (np.isnan(amax) and want_scale == 0x7FC00000) or (amax == np.inf and want_scale == 0x7F800000)
            c, s = T.quantize_block(x, fmt)
            assert not c.any() and _bits(s) == want_scale
            d = T.dequant_values(c, s, fmt)
            assert np.isnan(d).all()
    x = base.copy()                      # a NaN wins over an infinity
    x[3], x[40] = np.inf, np.nan
    c, s = T.quantize_block(x, fmt)
    assert not c.any() and _bits(s) == 0x7FC00000
    # a group: only the block holding the NaN changes
    specs = [TensorSpec("f", 1, 300, "FLAT", 100)]
    src = rng.standard_normal(300).astype(np.float32)
    q0, s0 = T.block_quant(src, specs, [0], 300, 1, fmt)
    src[150] = np.nan
    q1, s1 = T.block_quant(src, specs, [0], 300, 1, fmt)
    assert np.array_equal(q0[:100], q1[:100]) and np.array_equal(q0[200:], q1[200:]) and not q1[100:200].any()
    assert _bits(s1[1]) == 0x7FC00000 and _bits(s1[0]) == _bits(s0[0]) and _bits(s1[2]) == _bits(s0[2])


def test_quant_blocks_cover_each_position_once_and_stay_on_one_rank():
    specs = [TensorSpec("a", 37, 20, "TILE", 8, 6), TensorSpec("b", 3, 5, "ELEM"),
             TensorSpec("c", 1, 4099, "FLAT", 256)]
    V = 6
    p = P.plan(specs, V)
    seen = np.zeros(V * p.S, dtype=np.int64)
    nblk = 0
    for i, b, pos in T.quant_blocks(specs, p.starts):
        assert b == nblk
        nblk += 1
        seen[pos] += 1
        assert np.unique(pos // p.S).size == 1
    assert nblk == T.count_quant_blocks(specs) == 5 * 4 + 17
    s_a, s_c = int(p.starts[0]), int(p.starts[2])
    assert np.all(seen[s_a: s_a + 740] == 1) and np.all(seen[s_c: s_c + 4099] == 1)
    assert seen.sum() == 740 + 4099


@pytest.mark.parametrize("fmt", ["e4m3", "i8", "u8"])
def test_dequant_roundtrip_bounds(fmt):
    rng = np.random.default_rng(9)
    specs = [TensorSpec("a", 64, 40, "TILE", 16, 8), TensorSpec("b", 1, 5000, "FLAT", 512)]
    V = 4
    p = P.plan(specs, V)
    src = rng.standard_normal(V * p.S).astype(np.float32)
    if fmt == "u8":
        src = np.abs(src)
    q, sc = T.block_quant(src, specs, p.starts, p.S, V, fmt)
    out = T.block_dequant(q, sc, specs, p.starts, p.S, V, fmt)
    Q = codes.FORMAT_QMAX[fmt]
    for _, b, pos in T.quant_blocks(specs, p.starts):
        x, xr, s = src[pos].astype(np.float64), out[pos].astype(np.float64), float(sc[b])
        amax = np.max(np.abs(x))
        if fmt == "e4m3":
            # relative half-ulp of a 3-bit mantissa, or half the subnormal step, times the scale
            bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s) * (1 + 1e-6)
        else:
            bound = 0.5 * s * (1 + 1e-5) + np.abs(x) * 2.0 ** -20
        assert np.all(np.abs(x - xr) <= bound)
        k = int(np.argmax(np.abs(x)))
        assert abs(abs(xr[k]) - amax) <= amax * 2.0 ** -20
    for b, e in P.padding_ranges(specs, p.starts, p.S, V):
        assert not q[b:e].any() and not out[b:e].any()


def test_pack_pin_catches_add_before_scale(monkeypatch):
    """Planted mistake: (prev + g) * sigma instead of prev + g * sigma fails the exact pin."""
    def wrong(g, prev, sigma, accumulate):
        s = np.asarray(g, np.float32).astype(np.float64)
        if accumulate:
            s = T.f32(s + np.asarray(prev, np.float32).astype(np.float64)).astype(np.float64)
        return T.f32(s * np.float64(sigma))

    monkeypatch.setattr(T, "pack_values", wrong)
    with pytest.raises(AssertionError):
        test_pack_values_exact(3, True)


def test_bf16_round_matches_torch_and_hand_cases():
    import torch
    rng = np.random.default_rng(31)
    x = np.concatenate([
        (rng.standard_normal(200_000) * 10.0 ** rng.integers(-30, 30, 200_000)).astype(np.float32),
        # exact ties: low 16 bits 0x8000, with even and odd kept lsb
        (np.arange(1000, dtype=np.uint32) * np.uint32(0x10000) + np.uint32(0x3F808000)).view(np.float32),
        np.float32([0.0, -0.0, 1e-40, -1e-40, 3.3895314e38]),
    ])
    got = T.bf16_round(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to the even mantissa (1.0)
    assert T.bf16_round(np.float32([1 + 2 ** -8]))[0] == 0x3F80
    assert T.bf16_round(np.float32([1 + 3 * 2 ** -8]))[0] == 0x3F82


def test_bf16_round_overflow_and_infinities_match_torch():
    """IEEE overflow: the largest finite bf16 is 0x7F7F = (2 - 2^-7) * 2^127; from the midpoint
    between it and 2^128, (2 - 2^-8) * 2^127 = fp32 bits 0x7F7F8000, the result is infinity.
    Below the midpoint it stays 0x7F7F. torch's cast and the closed form agree."""
    import torch
    bits = np.array([0x7F7F7FFF, 0x7F7F8000, 0x7F7F8001, 0x7F7FFFFF, 0x7F800000,
                     0xFF7F7FFF, 0xFF7F8000, 0xFF7FFFFF, 0xFF800000, 0x7F7E8000, 0x7F7F0000], dtype=np.uint32)
    x = bits.view(np.float32)
    got = T.bf16_round(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    assert list(got) == [0x7F7F, 0x7F80, 0x7F80, 0x7F80, 0x7F80, 0xFF7F, 0xFF80, 0xFF80, 0xFF80, 0x7F7E, 0x7F7F]


def test_bf16_round_keeps_nan():
    """A NaN stays NaN (torch's cast does too) with its sign and the top payload bits; the
    quiet bit is set. A payload that rounding would carry into the exponent (0x7FFFFFFF,
    0xFFFFFFFF) must not come out as a number."""
    import torch
    bits = np.array([0x7FFFFFFF, 0xFFFFFFFF, 0x7FC00000, 0xFFC00000, 0x7F800001, 0xFF800001,
                     0x7FBFFFFF, 0x7FC0FFFF, 0x7FFF8000], dtype=np.uint32)
    x = bits.view(np.float32)
    got = T.bf16_round(x)
    as_f32 = (got.astype(np.uint32) << np.uint32(16)).view(np.float32)
    assert np.all(np.isnan(as_f32))
    assert np.isnan(torch.from_numpy(x).to(torch.bfloat16).float().numpy()).all()
    assert np.array_equal(got >> np.uint16(15), (bits >> np.uint32(31)).astype(np.uint16))   # sign kept
    assert list(got) == [0x7FFF, 0xFFFF, 0x7FC0, 0xFFC0, 0x7FC0, 0xFFC0, 0x7FFF, 0x7FC0, 0x7FFF]


@pytest.mark.parametrize("fmt", ["e4m3", "i8", "u8"])
def test_unpack_dequant_round_trips_values_on_the_code_grid(fmt):
    """Blocks whose values are code values times a power-of-two scale with amax exactly Q*2^k
    come back exactly (in fp32 and, being short-mantissa values, in bf16)."""
    specs = [TensorSpec("a", 48, 40, "TILE", 16, 8), TensorSpec("n", 9, 1, "ROWS", 1),
             TensorSpec("f", 1, 700, "FLAT", 256)]
    V = 3
    p = P.plan(specs, V)
    rng = np.random.default_rng(4)
    Q = codes.FORMAT_QMAX[fmt]
    src = np.zeros(V * p.S, dtype=np.float32)
    if fmt == "e4m3":
        grid = codes.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    elif fmt == "i8":
        grid = np.arange(-127, 128, dtype=np.float64)
    else:
        grid = np.arange(0, 256, dtype=np.float64)
    for _, b, pos in T.quant_blocks(specs, p.starts):
        k = int(rng.integers(-8, 8))
        v = rng.choice(grid, pos.size) * 2.0 ** k
        if fmt == "e4m3":
            v *= rng.choice([-1.0, 1.0], pos.size)
        v[0] = Q * 2.0 ** k
        src[pos] = v
    q, sc = T.block_quant(src, specs, p.starts, p.S, V, fmt)
    for out in ("f32", "bf16"):
        full = T.unpack_dequant(q, sc, specs, p.starts, fmt, out)
        assert full[1] is None
        for i in (0, 2):
            s, n = int(p.starts[i]), specs[i].rows * specs[i].cols
            want = src[s: s + n].reshape(specs[i].rows, specs[i].cols)
            got = full[i] if out == "f32" else (full[i].astype(np.uint32) << 16).view(np.float32)
            assert np.array_equal(got, want)


def test_pack_to_bf16_rounds_each_fp32_result_once():
    """A bf16 packed buffer is the fp32 pack rounded to nearest even once: equal to torch's
    fp32 -> bf16 cast of the fp32 result, ties to the even mantissa, padding +0.0."""
    import torch
    w, p = _tiny_plan()
    S, R = p.S, w.V
    grads = [W.tensor_values(w, i, W.Role.GRAD) for i in range(3)]
    prev = np.concatenate([W.prev_slice(w, k, S) for k in range(R)])
    for acc in (True, False):
        f32 = T.pack(grads, prev if acc else None, w.specs, p.starts, S, R, T.inv_v(w.V), acc)
        got = T.pack_to_bf16(grads, prev if acc else None, w.specs, p.starts, S, R, T.inv_v(w.V), acc)
        want = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert got.dtype == np.uint16 and np.array_equal(got, want)
        for b, e in P.padding_ranges(w.specs, p.starts, S, R):
            assert np.all(got[b:e] == 0)
    # exact midpoints between neighbouring bf16 values go to the even one (sigma = 1, no accumulation)
    spec = [TensorSpec("t", 1, 16, "ELEM")]
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0xBF818000, 0x3F80C000, 0x3F804000] + [0] * 10,
                    dtype=np.uint32).view(np.float32)
    out = T.pack_to_bf16([ties], None, spec, [0], 16, 1, np.float32(1.0), False)
    assert list(out[:6]) == [0x3F80, 0x3F82, 0xBF80, 0xBF82, 0x3F81, 0x3F80]
