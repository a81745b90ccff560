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
from workloads import tile_major_variant, workload

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


def _arrange(specs):
    """Row-major bits -> the order of the tensor's interval (the oracle's layout)."""
    def arrange(i, bits):
        if specs[i].kind != "TILEMAJOR":
            return bits
        out = np.empty_like(bits)
        out[OP.layout_offsets(specs[i])] = bits
        return out
    return arrange


def _quant_bands(w, plan):
    """{tensor: [(r0, r1), ...]} of the tile bands whose codes, scales and rebuilt bf16
    rows are compared with the oracle at full size.
    Llama-3-8B layer (row-major or tile-major): every band of every quantised tensor,
    down (4096 x 14336, the widest) included.
    MoE layer: the router, the first and the last expert whole, and in every tensor that
    a rank boundary crosses, the band on each side of that boundary."""
    specs = list(w.specs)
    quantised = [i for i, sp in enumerate(specs) if sp.kind in ("TILE", "TILEMAJOR")]

    def all_bands(i):
        sp = specs[i]
        return [(r0, min(r0 + sp.p0, sp.rows)) for r0 in range(0, sp.rows, sp.p0)]

    if w.index == 1:
        return {i: all_bands(i) for i in quantised}
    names = {sp.name: i for i, sp in enumerate(specs)}
    whole = [names["router"], names["e0.gate_up"], names["e0.down"], names["e127.gate_up"], names["e127.down"]]
    wanted = {i: all_bands(i) for i in whole}
    S = plan.S
    for k in range(1, plan.R_mat):
        pos = k * S
        for i in quantised:
            s, sp = plan.starts[i], specs[i]
            if s < pos < s + sp.numel:
                e = pos - s
                assert e % (sp.p0 * sp.cols) == 0, "a rank boundary inside a tile band"
                row = e // sp.cols
                if i not in whole:
                    bands = wanted.setdefault(i, [])
                    for b in ((row - sp.p0, row), (row, min(row + sp.p0, sp.rows))):
                        if b not in bands:
                            bands.append(b)
    for i in wanted:
        wanted[i].sort()
    return wanted


def _check_quant_full_size(w, idx, tile_major, plan, q, scales, gathered):
    """Codes, scales and the fused gather side of the chosen bands (every tile of each band)
    against the oracle, computed band by band in worker processes."""
    from tests import oracle_pool
    specs = list(w.specs)
    first = [0]
    for sp in specs:
        first.append(first[-1] + OT.count_quant_blocks([sp]))
    sc_bits = tensor_bits(scales)
    wanted = _quant_bands(w, plan)
    n_tiles = sum(OT.count_quant_blocks([oracle_pool._band_spec(specs[i], r0, r1)])
                  for i, b in wanted.items() for r0, r1 in b)
    print(f"  quant: comparing {n_tiles} tiles of {len(wanted)} tensors with the oracle "
          f"({'all' if idx == 1 else 'stratified'})", flush=True)
    jobs = oracle_pool.band_jobs(idx, tile_major, w.quant, wanted)
    done = 0
    for i, results in oracle_pool.run(jobs):
        sp, s = specs[i], plan.starts[i]
        tpr = -(-sp.cols // sp.p1)
        g_rows = gathered[i].view(sp.rows, sp.cols)
        for r0, r1, want_q, want_sc, want_g in results:
            got_q = tensor_bits(q[s + r0 * sp.cols: s + r1 * sp.cols])
            assert np.array_equal(got_q, want_q), f"quant {sp.name} rows {r0}-{r1}"
            b0 = first[i] + (r0 // sp.p0) * tpr
            assert np.array_equal(sc_bits[b0: b0 + want_sc.size], want_sc), f"scales {sp.name} rows {r0}-{r1}"
            assert np.array_equal(tensor_bits(g_rows[r0:r1]), want_g), f"unpack-dequant {sp.name} rows {r0}-{r1}"
            done += OT.count_quant_blocks([oracle_pool._band_spec(sp, r0, r1)])
    assert done == n_tiles
    print(f"  quant, scales and unpack-dequant match on all {n_tiles} tiles", flush=True)


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
    if not tile_major:
        # every tensor, on the device: unpack is a copy of the tensor's slice of the gathered buffer,
        # and pack equals fl32(prev + fl32(g * sigma)) from torch's elementwise fp32 multiply and add
        sig = torch.tensor(sigma, dtype=torch.float32, device=DEV)
        for i in range(len(specs)):
            s, n = int(plan.starts[i]), int(plan.numels[i])
            assert torch.equal(params[i].reshape(-1).view(torch.int16 if params[i].element_size() == 2 else torch.int32),
                               G[s: s + n].view(torch.int16 if G.element_size() == 2 else torch.int32)), f"unpack {i}"
            y = torch.mul(grads[i].reshape(-1), sig)
            want = torch.add(prev[s: s + n], y)
            assert torch.equal(packed[s: s + n].view(torch.int32), want.view(torch.int32)), f"pack {i}"
        print(f"  unpack and pack of all {len(specs)} tensors match their slices and torch's fp32 ops", flush=True)
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
        _check_quant_full_size(w, idx, tile_major, plan, q, scales, gathered)
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
