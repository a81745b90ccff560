"""The cache-policy store of the layout kernels (a buffer store with nt and sc1
set, addressed from the first active lane, else a global store), driven
through librs_bench.so's self-check along each of its paths and compared with
the expected buffer vector by vector: one buffer base per wave, the first
active lane at the highest address, lanes in two halves of a buffer (less
and more than 2 GiB apart) and waves with inactive lanes, lane 0 among them.
Vectors that no lane writes keep their prefilled bytes."""
import ctypes
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A5A5A5A


def _lib():
    lib = ctypes.CDLL(os.path.join(ROOT, "structure_aware_grouped_amd", "librs_bench.so"))
    lib.rs_bench_store_check.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    lib.rs_bench_store_check.restype = ctypes.c_int
    return lib


def _expected_source(nvec, mode, torch, dev):
    """v (the writing thread) for every vector t, and whether some lane writes t."""
    t = torch.arange(nvec, dtype=torch.int64, device=dev)
    written = torch.ones(nvec, dtype=torch.bool, device=dev)
    if mode == 0:
        v = t
    elif mode == 1:
        v = (t // 64) * 64 + 63 - t % 64
    elif mode == 2:
        half = nvec // 2
        lo = t < half
        u = torch.where(lo, t, t - half)
        v = (u // 32) * 64 + u % 32 + torch.where(lo, 0, 32)
    else:
        v = t
        written = (t % 64) % 3 != 0
    return v, written


@pytest.mark.parametrize("nvec,mode", [(128, 0), (1 << 20, 0), (1 << 20, 1), (1 << 20, 2), (1 << 20, 3),
                                       ((1 << 27) + 128, 2), (1 << 28, 2)])
def test_every_path_writes_exactly_its_vectors(gpu_lib, nvec, mode):
    # (1 << 27) + 128 vectors: the halves lie just over 1 GiB apart (buffer stores);
    # 1 << 28 vectors (4 GiB): they lie 2 GiB apart (global stores)
    import torch
    dev = torch.device("cuda:0")
    buf = torch.full((nvec, 4), SENTINEL, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    assert _lib().rs_bench_store_check(ctypes.c_void_p(buf.data_ptr()), ctypes.c_int64(nvec), ctypes.c_int(mode),
                                       ctypes.c_void_p(stream)) == 0
    torch.cuda.synchronize()
    v, written = _expected_source(nvec, mode, torch, dev)
    t = torch.arange(nvec, dtype=torch.int64, device=dev)
    got = buf.to(torch.int64) & 0xFFFFFFFF
    tag = 0xA5000000 | mode
    ok_w = (got[:, 0] == t) & (got[:, 1] == 0) & (got[:, 2] == v) & (got[:, 3] == tag)
    ok_u = (got == SENTINEL).all(dim=1)
    bad = torch.where(written, ~ok_w, ~ok_u)
    n_bad = int(bad.sum())
    assert n_bad == 0, f"{n_bad} vectors differ, the first at {int(torch.nonzero(bad)[0])}"
    del buf, got

