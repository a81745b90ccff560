"""The short correctly rounded square root of the 8-bit Adam step (used where
v1 lies in [2^-96, FLT_MAX]) checked on every fp32 of that range against the
general correctly rounded sequence, through librs_bench.so's self-check. The
Adam parity tests compare the whole step with the oracle (NumPy's fp32 square
root, correctly rounded) on top of this."""
import ctypes
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu


def _check(lo: int, hi: int):
    lib = ctypes.CDLL(os.path.join(ROOT, "structure_aware_grouped_amd", "librs_bench.so"))
    lib.rs_bench_sqrt_check.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    n, f = ctypes.c_uint64(), ctypes.c_uint32()
    assert lib.rs_bench_sqrt_check(lo, hi, ctypes.byref(n), ctypes.byref(f)) == 0
    return n.value, f.value


def test_short_square_root_on_every_value_of_its_range(gpu_lib):
    lo, hi = 0x0F800000, 0x7F7FFFFF          # 2^-96 .. FLT_MAX: 1,879,048,192 values
    bad, first = _check(lo, hi)
    assert bad == 0, f"{bad} values differ, the first 0x{first:08x}"


def test_the_range_bound_is_needed(gpu_lib):
    # below 2^-96 the hardware estimate is not within one ulp of every root (and subnormal
    # inputs are not handled at all), so the Adam step takes the general sequence there
    bad, first = _check(0x00800000, 0x0F7FFFFF)   # normal values below 2^-96
    assert bad > 0
    bad, first = _check(0x00000001, 0x007FFFFF)   # subnormal values
    assert bad > 0
