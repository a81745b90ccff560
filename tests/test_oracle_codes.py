"""Pins of the oracle's 8-bit codecs against things other than itself.

  * OCP E4M3 facts: named codes, the value set enumerated as exact rationals,
    nearest-even by exhaustive comparison.
  * torch.float8_e4m3fn (c10's independent converter) after an explicit clamp
    to +-448, on a structured sweep of every exponent, every kept mantissa
    and the rounding-critical low bits, plus random values.
  * int8 / uint8: hand-derived round-half-even and clamp cases.
"""
import numpy as np
import pytest
import torch

from oracle import codes
from tests import exact


def test_named_e4m3_codes():
    d = codes.e4m3_decode(np.array([0x00, 0x80, 0x01, 0x07, 0x08, 0x38, 0x7E, 0xFE, 0x7F, 0xFF],
                                   dtype=np.uint8))
    assert d[0] == 0 and not np.signbit(d[0])
    assert d[1] == 0 and np.signbit(d[1])
    assert d[2] == 2.0 ** -9                  # smallest subnormal
    assert d[3] == 7 * 2.0 ** -9              # largest subnormal
    assert d[4] == 2.0 ** -6                  # smallest normal
    assert d[5] == 1.0
    assert d[6] == 448.0 and d[7] == -448.0   # largest finite
    assert np.isnan(d[8]) and np.isnan(d[9])


def test_decode_matches_exact_table_and_torch():
    table = exact.e4m3_table()
    c = np.array([code for code, _ in table], dtype=np.uint8)
    assert np.array_equal(codes.e4m3_decode(c), np.array([float(v) for _, v in table]))
    allc = np.arange(256, dtype=np.uint8)
    t = torch.from_numpy(allc.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    d = codes.e4m3_decode(allc)
    assert np.all((d == t) | (np.isnan(d) & np.isnan(t)))


def _structured_sweep():
    vals = []
    lows = [0, 1, 2, (1 << 19) - 1, 1 << 19, (1 << 19) + 1, (1 << 20) - 1, 0x5A5A5]
    for e in range(-14, 9):           # 2^-14 .. 2^8 (covers subnormal and saturation ranges)
        for m3 in range(8):
            for lo in lows:
                bits = ((e + 127) << 23) | (m3 << 20) | lo
                vals.append(bits)
    u = np.array(vals, dtype=np.uint32)
    x = u.view(np.float32)
    rng = np.random.default_rng(7)
    rnd = (rng.random(200_000) * 2 - 1).astype(np.float32) * np.float32(500)
    tiny = (rng.random(50_000) * 2 - 1).astype(np.float32) * np.float32(2 ** -8)
    return np.concatenate([x, -x, rnd, tiny, np.float32([0.0, -0.0, 448.0, 447.9, 464.0, 500.0])])


def test_encode_matches_torch_after_clamp():
    x = _structured_sweep()
    mine = codes.e4m3_encode(x)
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)


def test_encode_matches_exhaustive_nearest_even():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        (rng.random(400) * 2 - 1).astype(np.float32) * np.float32(460),
        (rng.random(400) * 2 - 1).astype(np.float32) * np.float32(2 ** -6),
    ])
    # exact midpoints between neighbouring codes go to the even code
    table = exact.e4m3_table()
    mids = [float((table[k][1] + table[k + 1][1]) / 2) for k in range(len(table) - 1)]
    x = np.concatenate([x, np.float32(mids), -np.float32(mids)])
    got = codes.e4m3_encode(x)
    want = np.array([exact.e4m3_nearest(float(v)) for v in x], dtype=np.uint8)
    assert np.array_equal(got, want)
    # and the midpoint rule itself: code k or k+1, whichever is even
    for k, m in enumerate(mids):
        assert codes.e4m3_encode(np.float32([m]))[0] == (k if k % 2 == 0 else k + 1)


def test_saturation_sign_and_nan():
    x = np.float32([448.0, 449.0, 463.9, 464.0, 1e30, np.inf, -np.inf, -0.0, 0.0, np.nan])
    got = codes.e4m3_encode(x)
    assert list(got[:6]) == [0x7E] * 6
    assert got[6] == 0xFE
    assert got[7] == 0x80 and got[8] == 0x00
    assert got[9] == 0x7F


def test_roundtrip_on_every_finite_code():
    c = np.array([k for k in range(256) if (k & 0x7F) != 0x7F], dtype=np.uint8)
    v = codes.e4m3_decode(c).astype(np.float32)
    assert np.array_equal(codes.e4m3_encode(v), c)


@pytest.mark.parametrize("y,i8,u8", [
    (0.5, 0, 0), (1.5, 2, 2), (2.5, 2, 2), (-0.5, 0, 0), (-1.5, -2, 0), (-2.5, -2, 0),
    (126.5, 126, 126), (127.49, 127, 127), (127.5, 127, 128), (200.0, 127, 200),
    (254.5, 127, 254), (255.5, 127, 255), (300.0, 127, 255), (-300.0, -127, 0),
    (-0.0, 0, 0), (0.49999997, 0, 0),
])
def test_integer_codes(y, i8, u8):
    assert codes.int_encode(np.float32([y]), "i8").view(np.int8)[0] == i8
    assert codes.int_encode(np.float32([y]), "u8")[0] == u8
    assert exact.int_nearest(float(np.float32(y)), -127, 127) == i8
    assert exact.int_nearest(float(np.float32(y)), 0, 255) == u8


def test_integer_codes_random_vs_exact():
    rng = np.random.default_rng(3)
    y = np.concatenate([(rng.random(300) * 2 - 1) * 140, np.arange(-130, 131) + 0.5]).astype(np.float32)
    got8 = codes.int_encode(y, "i8").view(np.int8)
    gotu = codes.int_encode(y, "u8")
    for v, a, b in zip(y, got8, gotu):
        assert a == exact.int_nearest(float(v), -127, 127)
        assert b == exact.int_nearest(float(v), 0, 255)


def test_pin_catches_ties_away_from_zero(monkeypatch):
    """A plausible mistake planted in the oracle (ties away from zero) fails the torch pin."""
    orig = codes.e4m3_encode

    def ties_away(y):
        y32 = np.asarray(y, dtype=np.float32)
        c = orig(y32)
        mag = c & 0x7F
        a = np.abs(y32.astype(np.float64))
        here = codes.e4m3_decode(mag)
        up = codes.e4m3_decode(np.minimum(mag + 1, 0x7E).astype(np.uint8))
        tie_below = (up > here) & (a - here == up - a)   # a tie that went down to the even code
        return np.where(tie_below, (mag + 1) | (c & 0x80), c).astype(np.uint8)

    monkeypatch.setattr(codes, "e4m3_encode", ties_away)
    x = _structured_sweep()
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert not np.array_equal(codes.e4m3_encode(x), ref)
