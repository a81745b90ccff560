"""librs_bench.so's streaming copy, the practical ceiling the benchmark times,
checked byte for byte: sizes that end inside a workgroup's 1 KiB and inside
the first 16 bytes, and destinations at offsets that are not multiples of the
workgroup's span."""
import ctypes
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,dst_off", [(16, 0), (1008, 16), (1024, 0), (5 * 1024 + 48, 272),
                                            ((3 << 20) + 16, 1024 + 528)])
def test_copy_is_exact(gpu_lib, nbytes, dst_off):
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "structure_aware_grouped_amd", "librs_bench.so"))
    lib.rs_bench_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.rs_bench_copy.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).to(dev)
    canary = 4096
    buf = torch.full((dst_off + nbytes + canary,), 0xA5, dtype=torch.uint8, device=dev)
    dst = buf[dst_off:dst_off + nbytes]
    stream = torch.cuda.current_stream().cuda_stream
    assert lib.rs_bench_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()),
                             ctypes.c_int64(nbytes), ctypes.c_void_p(stream)) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert bool((buf[:dst_off] == 0xA5).all()) and bool((buf[dst_off + nbytes:] == 0xA5).all())
