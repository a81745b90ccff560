"""HIP path vs the CPU oracle on the five workloads at full size, through the
same calls the bench times. Where the oracle would take minutes, whole tensors
are sampled (every element of a sampled tensor, tile or rank range is
compared) and properties are checked everywhere (padding is +0.0, codes
outside blocks are 0, every scale is a positive finite fp32)."""
import random

import numpy as np
import pytest
import torch

from oracle import plan as OP, transform as OT
from tests.gpu_util import Inputs, garbage, tensor_bits
from workloads import f32_from_bf16_bits, tile_major_variant, workload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _setup(rs, idx, tile_major=False):
    w = workload(idx)
    if tile_major:
        w = tile_major_variant(w)
    S, starts, _, _ = rs.rs_plan_build(list(w.specs), w.V)
    ref = OP.plan(w.specs, w.V)
    assert S == ref.S and starts == [int(s) for s in ref.starts]
    R = w.V if w.materialize_all_ranks else ref.R_used
    plan = rs.rs_plan_load(list(w.specs), w.V, S, starts, R, 0)
    return w, plan, Inputs(w, S, starts, R)


def _sample(n, k, seed):
    idx = list(range(n))
    if n <= k:
        return idx
    rng = random.Random(seed)
    return sorted(set([0, n - 1] + rng.sample(idx, k - 2)))


def _zero_everywhere(t: torch.Tensor, ranges):
    flat = t.view(torch.int32) if t.dtype == torch.float32 else t
    for b, e in ranges:
        assert bool((flat[b:e] == 0).all().item()), (b, e)


def _tensor_param_f32(inp, i):
    bits = inp.weight_bits(i)
    return f32_from_bf16_bits(bits) if bits.dtype == np.uint16 else bits.view(np.float32)


def _arrange(specs):
    """Row-major bits -> the order of the tensor's interval (the oracle's layout)."""
    def arrange(i, bits):
        if specs[i].kind != "TILEMAJOR":
            return bits
        out = np.empty_like(bits)
        out[OP.layout_offsets(specs[i])] = bits
        return out
    return arrange


@pytest.mark.parametrize("idx,tile_major", [(1, False), (2, False), (3, False), (1, True)])
def test_param_and_grad_workloads(gpu_lib, idx, tile_major):
    import structure_aware_grouped_amd as rs
    w, plan, inp = _setup(rs, idx, tile_major)
    R, S = plan.R_mat, plan.S
    specs = list(w.specs)
    print(f"workload {idx}{' (tile-major)' if tile_major else ''}: S={S} R_mat={R} tensors={len(specs)}",
          flush=True)

    G = inp.gathered(_arrange(specs))
    params = inp.empty_params()
    rs.rs_unpack_gathered(plan, G, params)
    print("  params uploaded and unpacked", flush=True)
    grads = inp.grads()
    prev = inp.prev()
    print("  grads and prev uploaded", flush=True)
    packed = garbage(R * S, torch.float32, DEV)
    rs.rs_pack_scatter(plan, grads, packed, prev=prev)
    q = scales = gathered = None
    if w.quant:
        q = garbage(R * S, torch.uint8, DEV, 0x3C)
        scales = garbage(plan.n_qblocks, torch.float32, DEV)
        rs.rs_block_quant(plan, G, q, w.quant, scales)
        # gather side: the codes and scales rebuild the quantised bf16 tensors
        gathered = [garbage(sp.rows * sp.cols, torch.bfloat16, DEV) if sp.kind in ("TILE", "TILEMAJOR", "FLAT") else None
                    for sp in specs]
        rs.rs_unpack_dequant(plan, q, w.quant, scales, gathered)
    torch.cuda.synchronize()

    print("  kernels done; checking against the oracle", flush=True)
    sample = _sample(len(specs), 12, idx)
    sigma = OT.inv_v(w.V)
    for i in sample:
        s, n = plan.starts[i], plan.numels[i]
        lay = OP.layout_offsets(specs[i]) if specs[i].kind == "TILEMAJOR" else slice(None)
        # unpack: T_i is the gathered slice
        assert np.array_equal(tensor_bits(params[i]).ravel(), inp.weight_bits(i)), f"unpack {i}"
        # pack: every element of the tensor's slice
        want = OT.pack_values(inp.grad(i).ravel(), inp.prev_range(s, s + n)[lay], sigma, True)
        assert np.array_equal(tensor_bits(packed[s: s + n])[lay], want.view(np.uint32)), f"pack {i}"
    pads = OP.padding_ranges(specs, plan.starts, S, R)
    _zero_everywhere(packed, pads)
    print(f"  unpack and pack match on tensors {sample}; padding zero", flush=True)
    if idx == 1 and not tile_major:
        # the same pack into a bf16 buffer (bf16 ReduceScatter): each fp32 result rounded once
        del packed
        packed_b = garbage(R * S, torch.bfloat16, DEV)
        rs.rs_pack_scatter(plan, grads, packed_b, prev=prev)
        torch.cuda.synchronize()
        for i in sample:
            s, n = plan.starts[i], plan.numels[i]
            want = OT.bf16_round(OT.pack_values(inp.grad(i).ravel(), inp.prev_range(s, s + n), sigma, True))
            assert np.array_equal(tensor_bits(packed_b[s: s + n]), want), f"bf16 pack {i}"
        _zero_everywhere(packed_b.view(torch.int16), pads)
        del packed_b
        print("  bf16 pack matches on the same tensors; padding zero", flush=True)

    if w.quant:
        first = [0]
        for sp in specs:
            first.append(first[-1] + OT.count_quant_blocks([sp]))
        sc_bits = tensor_bits(scales)
        for i in sample[: min(len(sample), 6)]:
            s, n = plan.starts[i], plan.numels[i]
            lay = OP.layout_offsets(specs[i])
            x = np.empty(n, np.float32)
            x[lay] = _tensor_param_f32(inp, i)           # the tensor's interval order
            elem = np.empty(n, np.int64)
            elem[lay] = np.arange(n)                     # interval position -> row-major element
            got_q = tensor_bits(q[s: s + n])
            got_g = tensor_bits(gathered[i]).ravel() if gathered[i] is not None else None
            for _, b, pos in OT.quant_blocks([specs[i]], [0]):
                c, sc = OT.quantize_block(x[pos], w.quant)
                assert np.array_equal(got_q[pos], c), f"quant {i} block {b}"
                assert sc_bits[first[i] + b] == np.float32(sc).view(np.uint32), f"scale {i} block {b}"
                want_g = OT.bf16_round(OT.dequant_values(c, sc, w.quant))
                assert np.array_equal(got_g[elem[pos]], want_g), f"unpack-dequant {i} block {b}"
        _zero_everywhere(q, OP.padding_ranges([sp for sp in specs if sp.kind in ("TILE", "TILEMAJOR", "FLAT")],
                                              [st for sp, st in zip(specs, plan.starts)
                                               if sp.kind in ("TILE", "TILEMAJOR", "FLAT")], S, R))
        sf = scales.float()
        assert bool(torch.isfinite(sf).all()) and bool((sf > 0).all())
    plan.close()


def test_adam_state_workload(gpu_lib):
    """Config 4 in full: pack m and v (scale 1, no accumulation), int8 / uint8 block
    quant, dequant; every element and every scale against the oracle."""
    import structure_aware_grouped_amd as rs
    w, plan, inp = _setup(rs, 4)
    R, S, specs = plan.R_mat, plan.S, list(w.specs)
    results = {}
    for which, fmt in (("m", "i8"), ("v", "u8")):
        states = inp.adam_states(which)
        packed = garbage(R * S, torch.float32, DEV)
        rs.rs_pack_scatter(plan, states, packed, scale=1.0)
        q = garbage(R * S, torch.uint8, DEV)
        sc = garbage(plan.n_qblocks, torch.float32, DEV)
        rs.rs_block_quant(plan, packed, q, fmt, sc)
        out = garbage(R * S, torch.float32, DEV)
        rs.rs_block_dequant(plan, q, fmt, sc, out)
        torch.cuda.synchronize()
        host = [s.cpu().numpy() for s in states]
        del states
        want_p = OT.pack(host, None, specs, plan.starts, S, R, np.float32(1.0), False)
        assert np.array_equal(tensor_bits(packed), want_p.view(np.uint32)), which
        wq, ws = OT.block_quant(want_p, specs, plan.starts, S, R, fmt)
        assert np.array_equal(tensor_bits(q), wq), which
        assert np.array_equal(tensor_bits(sc), ws.view(np.uint32)), which
        wd = OT.block_dequant(wq, ws, specs, plan.starts, S, R, fmt)
        got_d = tensor_bits(out)
        assert np.array_equal(got_d, wd.view(np.uint32)), which
        # round trip: within half a code step of each block's scale
        err = np.abs(got_d.view(np.float32).astype(np.float64) - want_p.astype(np.float64))
        for _, b, pos in OT.quant_blocks(specs[:2], plan.starts[:2]):
            assert np.all(err[pos] <= 0.5 * float(ws[b]) * (1 + 1e-5) + np.abs(want_p[pos]) * 2.0 ** -20)
        results[which] = True
    assert results == {"m": True, "v": True}
    plan.close()
