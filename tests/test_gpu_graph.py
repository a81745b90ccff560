"""HIP graphs: the transform calls captured once (after one eager call with
the same pointers) and replayed, with fresh inputs written by eager work and a
synchronisation between replays; every replay matches the oracle bit for bit.
A capture that would need a new pointer table is refused before it launches
anything."""
import numpy as np
import pytest
import torch

from oracle import transform as OT
from tests.gpu_util import garbage, tensor_bits, to_device_bits
from tests.test_gpu_parity import RAGGED, _plan, _values
from workloads import bf16_bits_from_f32, f32_from_bf16_bits

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _host_inputs(rng, plan, pdtype):
    """Flat parameter buffer (NaN padding), gradients, previous packed buffer."""
    total = plan.R_mat * plan.S
    flat = np.full(total, np.nan, dtype=np.float32)
    for sp, s in zip(plan.specs, plan.starts):
        flat[s: s + sp.rows * sp.cols] = _values(rng, sp.rows * sp.cols)
    grads = [_values(rng, sp.rows * sp.cols, scale=1e-3).reshape(sp.rows, sp.cols) for sp in plan.specs]
    if pdtype == torch.bfloat16:
        flat = f32_from_bf16_bits(bf16_bits_from_f32(flat))
        grads = [f32_from_bf16_bits(bf16_bits_from_f32(g)).reshape(g.shape) for g in grads]
    return flat, grads, _values(rng, total, scale=1e-3)


def _to_dev_flat(flat, pdtype):
    if pdtype == torch.bfloat16:
        bits = bf16_bits_from_f32(flat)
        bits[np.isnan(flat)] = 0x7FC1
        return to_device_bits(bits, torch.bfloat16, DEV)
    return torch.from_numpy(flat).to(DEV)


@pytest.mark.parametrize("pdtype", [torch.float32, torch.bfloat16])
def test_captured_step_replays_bit_exactly(gpu_lib, pdtype):
    import structure_aware_grouped_amd as rs
    specs, V = RAGGED, 6
    plan = _plan(rs, specs, V)
    R, S = plan.R_mat, plan.S
    total = R * S
    rng = np.random.default_rng(2024)

    # device buffers, fixed for the graph's lifetime
    flat, grads_h, prev_h = _host_inputs(rng, plan, pdtype)
    G = _to_dev_flat(flat, pdtype)
    grads = [torch.from_numpy(g).to(DEV).to(pdtype) for g in grads_h]
    prev = torch.from_numpy(prev_h).to(DEV)
    outs = [garbage(sp.rows * sp.cols, pdtype, DEV).view(sp.rows, sp.cols) for sp in specs]
    packed = garbage(total, torch.float32, DEV)
    q = garbage(total, torch.uint8, DEV)
    scales = garbage(plan.n_qblocks, torch.float32, DEV)
    deq = garbage(total, torch.float32, DEV)
    quantised = [sp.kind in ("TILE", "TILEMAJOR", "FLAT") for sp in specs]
    full = [garbage(sp.rows * sp.cols, pdtype, DEV).view(sp.rows, sp.cols) if qz else None
            for sp, qz in zip(specs, quantised)]

    def step():
        rs.rs_unpack_gathered(plan, G, outs)
        rs.rs_pack_scatter(plan, grads, packed, prev=prev)
        rs.rs_block_quant(plan, G, q, "e4m3", scales)
        rs.rs_block_dequant(plan, q, "e4m3", scales, deq)
        rs.rs_unpack_dequant(plan, q, "e4m3", scales, full)

    step()                        # uploads the pointer tables outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()

    sigma = OT.inv_v(V)
    tag = "bf16" if pdtype == torch.bfloat16 else "f32"
    for replay in range(3):
        # eager work between replays: new inputs in place, outputs poisoned again
        flat, grads_h, prev_h = _host_inputs(rng, plan, pdtype)
        G.copy_(_to_dev_flat(flat, pdtype))
        for g, gh in zip(grads, grads_h):
            g.copy_(torch.from_numpy(gh).to(DEV).to(pdtype))
        prev.copy_(torch.from_numpy(prev_h).to(DEV))
        for t in [*outs, packed, q, scales, deq, *[f for f in full if f is not None]]:
            t.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()

        for o, wv in zip(outs, OT.unpack(tensor_bits(G), specs, plan.starts)):
            assert np.array_equal(tensor_bits(o), wv), ("unpack", replay)
        want = OT.pack(grads_h, prev_h, specs, plan.starts, S, R, sigma, True)
        assert np.array_equal(tensor_bits(packed), want.view(np.uint32)), ("pack", replay)
        wq, ws = OT.block_quant(flat, specs, plan.starts, S, R, "e4m3")
        assert np.array_equal(tensor_bits(q), wq), ("quant", replay)
        assert np.array_equal(tensor_bits(scales), ws.view(np.uint32)), ("scales", replay)
        wd = OT.block_dequant(wq, ws, specs, plan.starts, S, R, "e4m3")
        assert np.array_equal(tensor_bits(deq), wd.view(np.uint32)), ("dequant", replay)
        for d, wv in zip(full, OT.unpack_dequant(wq, ws, specs, plan.starts, "e4m3", tag)):
            assert (d is None) == (wv is None)
            if d is not None:
                assert np.array_equal(tensor_bits(d), wv.view(np.uint32) if tag == "f32" else wv), ("gather", replay)
    del graph
    plan.close()


# the refused capture leaves an empty graph, which torch warns about
@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_capture_that_needs_a_new_pointer_table_is_refused(gpu_lib):
    import structure_aware_grouped_amd as rs
    from structure_aware_grouped_amd import binding
    specs, V = RAGGED, 3
    plan = _plan(rs, specs, V)
    G = torch.zeros(plan.R_mat * plan.S, device=DEV)
    outs_a = [torch.empty(sp.rows, sp.cols, device=DEV) for sp in specs]
    outs_b = [torch.empty(sp.rows, sp.cols, device=DEV) for sp in specs]
    rs.rs_unpack_gathered(plan, G, outs_a)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(binding.RsError) as ei:
        with torch.cuda.graph(graph):
            rs.rs_unpack_gathered(plan, G, outs_b)   # other pointers: refused, nothing launched
    assert ei.value.status == binding.RS_EINVAL and "captured" in str(ei.value)
    torch.cuda.synchronize()
    # outside a capture the same call goes through and uploads the new table
    G.fill_(1.0)
    rs.rs_unpack_gathered(plan, G, outs_b)
    torch.cuda.synchronize()
    assert all(bool((o == 1.0).all()) for o in outs_b)
    del graph
    plan.close()
