"""HIP path vs the CPU oracle, element by element, on small groups that span
several tiles, ragged tails and the degenerate cases. Every call goes through
the C ABI (via the ctypes binding)."""
import os

import numpy as np
import pytest
import torch

from oracle import codes as OC, plan as OP, transform as OT
from tests.gpu_util import garbage, guard_intact, guarded, tensor_bits, to_device_bits
from workloads import TensorSpec, bf16_bits_from_f32, f32_from_bf16_bits, workload
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _rng(seed):
    return np.random.default_rng(seed)


def _plan(rs, specs, V, R_mat=None):
    S, starts, _, _ = rs.rs_plan_build(specs, V)
    ref = OP.plan(specs, V)
    assert S == ref.S and starts == [int(s) for s in ref.starts]
    return rs.rs_plan_load(specs, V, S, starts, V if R_mat is None else R_mat, 0)


def _values(rng, n, dist="normal", scale=1.0):
    if dist == "normal":
        return (rng.standard_normal(n) * scale).astype(np.float32)
    return (rng.random(n) * 2 - 1).astype(np.float32) * np.float32(scale)


def _flat_input(rng, plan, pdtype, scale=1.0, positive=False):
    """Flat buffer with tensor data at the plan's starts and NaN poison elsewhere.

    Returns (device tensor, fp32 host values of the flat buffer, per-tensor host values)."""
    total = plan.R_mat * plan.S
    host = np.full(total, np.nan, dtype=np.float32)
    per = []
    for spec, s in zip(plan.specs, plan.starts):
        v = _values(rng, spec.rows * spec.cols, scale=scale)
        if positive:
            v = np.abs(v)
        if pdtype == torch.bfloat16:
            v = f32_from_bf16_bits(bf16_bits_from_f32(v))
        host[s: s + v.size] = v
        per.append(v)
    if pdtype == torch.bfloat16:
        bits = bf16_bits_from_f32(host)
        bits[np.isnan(host)] = 0x7FC1
        dev = to_device_bits(bits, torch.bfloat16, DEV)
    else:
        dev = torch.from_numpy(host).to(DEV)
    return dev, host, per


def _full_check(rs, specs, V, pdtype, seed, fmts=("e4m3", "i8", "u8"), R_mat=None):
    rng = _rng(seed)
    plan = _plan(rs, specs, V, R_mat)
    R, S = plan.R_mat, plan.S
    total = R * S
    G, Gh, xs = _flat_input(rng, plan, pdtype)

    # unpack
    outs = [garbage(sp.rows * sp.cols, pdtype, DEV).view(sp.rows, sp.cols) for sp in specs]
    rs.rs_unpack_gathered(plan, G, outs)
    want = OT.unpack(tensor_bits(G), specs, plan.starts)
    for o, wv in zip(outs, want):
        assert np.array_equal(tensor_bits(o), wv)

    # pack, with and without accumulation, out of place and in place
    grads_h = [_values(rng, sp.rows * sp.cols, scale=1e-3).reshape(sp.rows, sp.cols) for sp in specs]
    gdt = pdtype
    if gdt == torch.bfloat16:
        grads_h = [f32_from_bf16_bits(bf16_bits_from_f32(g)).reshape(g.shape) for g in grads_h]
    grads = [torch.from_numpy(g).to(DEV).to(gdt) for g in grads_h]
    prev_h = _values(rng, total, scale=1e-3)
    prev = torch.from_numpy(prev_h).to(DEV)
    sigma = OT.inv_v(V)
    whole, packed = guarded(total, torch.float32, DEV)
    packed.view(torch.uint8).fill_(0xA5)
    rs.rs_pack_scatter(plan, grads, packed, prev=prev)
    want = OT.pack(grads_h, prev_h, specs, plan.starts, S, R, sigma, True)
    assert np.array_equal(tensor_bits(packed), want.view(np.uint32))
    assert guard_intact(whole, total)
    rs.rs_pack_scatter(plan, grads, packed)
    want0 = OT.pack(grads_h, None, specs, plan.starts, S, R, sigma, False)
    assert np.array_equal(tensor_bits(packed), want0.view(np.uint32))
    inplace = prev.clone()
    rs.rs_pack_scatter(plan, grads, inplace, prev=inplace, scale=0.75)
    want2 = OT.pack(grads_h, prev_h, specs, plan.starts, S, R, np.float32(0.75), True)
    assert np.array_equal(tensor_bits(inplace), want2.view(np.uint32))
    # a bf16 packed buffer (bf16 ReduceScatter): each fp32 result rounded once to nearest even
    for acc in (True, False):
        bwhole, pb = guarded(total, torch.bfloat16, DEV)
        pb.view(torch.uint8).fill_(0xA5)
        rs.rs_pack_scatter(plan, grads, pb, prev=prev if acc else None)
        want_b = OT.pack_to_bf16(grads_h, prev_h if acc else None, specs, plan.starts, S, R, sigma, acc)
        assert np.array_equal(tensor_bits(pb), want_b), acc
        assert guard_intact(bwhole, total)

    # quant and dequant of the flat parameter buffer
    for fmt in fmts:
        src_dev, src_h = G, Gh
        if fmt == "u8":   # unsigned codes take non-negative values (Adam's v)
            src_dev, src_h, _ = _flat_input(rng, plan, pdtype, positive=True)
        qwhole, q = guarded(total, torch.uint8, DEV)
        q.fill_(0x5A)
        swhole, scales = guarded(max(plan.n_qblocks, 1), torch.float32, DEV)
        rs.rs_block_quant(plan, src_dev, q, fmt, scales)
        wq, ws = OT.block_quant(src_h, specs, plan.starts, S, R, fmt)
        assert np.array_equal(tensor_bits(q), wq), fmt
        assert np.array_equal(tensor_bits(scales)[: plan.n_qblocks], ws.view(np.uint32)), fmt
        assert guard_intact(qwhole, total) and guard_intact(swhole, max(plan.n_qblocks, 1))
        owhole, out = guarded(total, torch.float32, DEV)
        out.view(torch.uint8).fill_(0x77)
        rs.rs_block_dequant(plan, q, fmt, scales, out)
        wd = OT.block_dequant(wq, ws, specs, plan.starts, S, R, fmt)
        assert np.array_equal(tensor_bits(out), wd.view(np.uint32)), fmt
        assert guard_intact(owhole, total)
        # unpack of a 1-byte buffer: the gathered codes, tensor by tensor
        cdst = [garbage(sp.rows * sp.cols, torch.uint8, DEV, 0x99).view(sp.rows, sp.cols) for sp in specs]
        rs.rs_unpack_gathered(plan, q, cdst)
        for d, wv in zip(cdst, OT.unpack(wq, specs, plan.starts)):
            assert np.array_equal(tensor_bits(d), wv), fmt
        # gather side: gathered codes + scales -> the quantised full tensors
        for out_dt, tag in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
            quantised = [sp.kind in ("TILE", "TILEMAJOR", "FLAT") for sp in specs]
            dsts = [garbage(sp.rows * sp.cols, out_dt, DEV).view(sp.rows, sp.cols) if qz else None
                    for sp, qz in zip(specs, quantised)]
            rs.rs_unpack_dequant(plan, q, fmt, scales, dsts)
            want = OT.unpack_dequant(wq, ws, specs, plan.starts, fmt, tag)
            for d, wv in zip(dsts, want):
                assert (d is None) == (wv is None)
                if d is not None:
                    assert np.array_equal(tensor_bits(d), wv.view(np.uint32) if tag == "f32" else wv), (fmt, tag)
    plan.close()


def test_tiny_workload(gpu_lib):
    import structure_aware_grouped_amd as rs
    w = workload(0)
    _full_check(rs, list(w.specs), w.V, torch.float32, 0)


@pytest.mark.parametrize("V", [1, 2, 3, 5, 7, 8])
@pytest.mark.parametrize("pdtype", [torch.float32, torch.bfloat16])
def test_tiny_shapes_other_rank_counts(gpu_lib, V, pdtype):
    import structure_aware_grouped_amd as rs
    _full_check(rs, list(workload(0).specs), V, pdtype, 100 + V)


RAGGED = [
    TensorSpec("tile_partial", 37, 20, "TILE", 8, 6),     # partial tiles, unaligned columns
    TensorSpec("tile_vec", 130, 64, "TILE", 16, 16),      # vector path, partial last band
    TensorSpec("flat_tail", 1, 4099, "FLAT", 256),         # partial last flat block
    TensorSpec("flat_big", 2048, 3, "FLAT", 2048),
    TensorSpec("elem", 7, 130, "ELEM"),
    TensorSpec("rows3", 10, 10, "ROWS", 3),
    TensorSpec("whole", 5, 5, "WHOLE"),
    TensorSpec("tile_wide", 33, 520, "TILE", 32, 128),    # 128-wide tiles and a 8-wide edge
    TensorSpec("norm", 4096, 1, "ROWS", 1),
]


@pytest.mark.parametrize("encoder", ["sw", "hw"])
@pytest.mark.parametrize("V", [1, 3, 6, 16])
@pytest.mark.parametrize("pdtype", [torch.float32, torch.bfloat16])
def test_ragged_group(gpu_lib, V, pdtype, encoder, monkeypatch):
    import structure_aware_grouped_amd as rs
    monkeypatch.setenv("RS_E4M3_ENCODER", encoder)
    _full_check(rs, RAGGED, V, pdtype, 7 * V)


@pytest.mark.parametrize("encoder", ["sw", "hw"])
@pytest.mark.parametrize("pdtype", [torch.float32, torch.bfloat16])
def test_e4m3_amax_overshoot(gpu_lib, encoder, pdtype, monkeypatch):
    """Block maxima whose scaled value rounds just above 448 (fl32(amax * fl32(448/amax)) >
    448) must saturate to 0x7E / 0xFE, like every other value of the block."""
    import structure_aware_grouped_amd as rs
    monkeypatch.setenv("RS_E4M3_ENCODER", encoder)
    rng = _rng(21)
    a = (rng.random(200_000) * 100).astype(np.float32) + np.float32(1e-3)
    if pdtype == torch.bfloat16:
        a = f32_from_bf16_bits(bf16_bits_from_f32(a))
    r = (448.0 / a.astype(np.float64)).astype(np.float32)
    over = a[(a.astype(np.float64) * r.astype(np.float64)).astype(np.float32) > 448][:1024]
    assert over.size >= 256
    b = 64
    blocks = np.empty((over.size, b), dtype=np.float32)
    blocks[:] = (rng.random((over.size, b)) * 2 - 1) * over[:, None] * np.float32(0.99)
    blocks[:, 3] = over
    blocks[:, 40] = -over
    if pdtype == torch.bfloat16:
        blocks = f32_from_bf16_bits(bf16_bits_from_f32(blocks)).reshape(blocks.shape)
    data = blocks.ravel()
    spec = [TensorSpec("o", over.size, b, "FLAT", b)]
    plan = rs.rs_plan_load(spec, 1, data.size, [0], 1, 0)
    src = torch.from_numpy(data).to(DEV).to(pdtype)
    q = torch.empty(data.size, dtype=torch.uint8, device=DEV)
    sc = torch.empty(over.size, dtype=torch.float32, device=DEV)
    rs.rs_block_quant(plan, src, q, "e4m3", sc)
    wq, ws = OT.block_quant(data, spec, [0], data.size, 1, "e4m3")
    got = tensor_bits(q)
    assert np.array_equal(got, wq)
    assert np.all(got.reshape(-1, b)[:, 3] == 0x7E) and np.all(got.reshape(-1, b)[:, 40] == 0xFE)
    assert np.array_equal(tensor_bits(sc), ws.view(np.uint32))
    plan.close()


TILE_MAJOR = [
    TensorSpec("tm32", 64, 96, "TILEMAJOR", 32, 32),
    TensorSpec("tm_wide", 32, 2048, "TILEMAJOR", 16, 128),  # strips split by the LDS budget
    TensorSpec("tm_odd", 32, 12, "TILEMAJOR", 16, 3),        # runs not a multiple of 16 bytes
    TensorSpec("rows", 10, 10, "ROWS", 1),
    TensorSpec("tile_rm", 48, 64, "TILE", 16, 16),
    TensorSpec("flat", 1, 1000, "FLAT", 256),
]


@pytest.mark.parametrize("V", [1, 3, 8])
@pytest.mark.parametrize("pdtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("tm_kernel", ["direct", "lds"])
def test_tile_major_group(gpu_lib, V, pdtype, tm_kernel, monkeypatch):
    """Tile-major tensors through unpack / pack (direct reorder, or staged through LDS),
    quant, dequant and the fused unpack-dequant, next to row-major ones."""
    import structure_aware_grouped_amd as rs
    monkeypatch.setenv("RS_TM_KERNEL", tm_kernel)
    _full_check(rs, TILE_MAJOR, V, pdtype, 40 + V)


# Big enough that each split or XCD-grouped launch runs whole rounds plus a
# ragged tail. Pack: more than 2048 pieces of 512 outputs. Row-run gather: more
# than 1024 pieces. Tile kernels: more than 32 tiles. It also holds partial
# tiles on unaligned columns, a partial flat block and tile-major tiles.
MID = [
    TensorSpec("tiles32", 1024, 1024, "TILE", 32, 32),
    TensorSpec("tiles64_ragged", 300, 1000, "TILE", 64, 64),
    TensorSpec("flat2048", 1, 300001, "FLAT", 2048),
    TensorSpec("tm32x64", 256, 512, "TILEMAJOR", 32, 64),
    TensorSpec("rows3", 777, 33, "ROWS", 3),
    TensorSpec("elem", 5000, 1, "ELEM"),
]


@pytest.mark.parametrize("pdtype", [torch.float32, torch.bfloat16])
def test_mid_size_group(gpu_lib, pdtype):
    import structure_aware_grouped_amd as rs
    S, _, _, _ = rs.rs_plan_build(MID, 7)
    pieces = 7 * S // 4096 * 8                  # pack pieces: a whole round of 2048 and a tail
    assert pieces > 2048 and pieces % 2048 != 0
    _full_check(rs, MID, 7, pdtype, 77)


# Blocks larger than the register paths hold (a tile of more than 16384
# elements, a flat block of more than 2048 fp32 / 4096 bf16 elements), so the
# kernels take their two-pass element paths; plus a flat block size that is not
# a multiple of 16 (per-block gather), tile-major tiles of 32768 elements and
# tile-major tiles of the widest allowed shape (8192 columns).
BIG_BLOCKS = [
    TensorSpec("tile_big", 300, 520, "TILE", 256, 128),
    TensorSpec("flat_big", 1, 20000, "FLAT", 6000),
    TensorSpec("tm_big", 512, 256, "TILEMAJOR", 256, 128),
    TensorSpec("flat_odd", 1, 3001, "FLAT", 1000),
    TensorSpec("norm", 300, 1, "ROWS", 1),
    TensorSpec("tm_widest", 4, 16384, "TILEMAJOR", 2, 8192),   # 8192-column tiles: one-row strips
]


@pytest.mark.parametrize("V", [1, 3])
@pytest.mark.parametrize("pdtype", [torch.float32, torch.bfloat16])
def test_blocks_beyond_the_register_paths(gpu_lib, V, pdtype):
    import structure_aware_grouped_amd as rs
    _full_check(rs, BIG_BLOCKS, V, pdtype, 90 + V)


@pytest.mark.parametrize("tm_kernel", ["direct", "lds"])
def test_launches_that_loop_over_work_items(gpu_lib, tm_kernel, monkeypatch):
    """RS_MAX_GRID=24 caps every launch at 24 workgroups, so each workgroup loops
    over many work items (and reuses its LDS between tiles): the results must not
    change."""
    import structure_aware_grouped_amd as rs
    monkeypatch.setenv("RS_MAX_GRID", "24")
    monkeypatch.setenv("RS_TM_KERNEL", tm_kernel)
    _full_check(rs, MID, 7, torch.bfloat16, 78)
    _full_check(rs, TILE_MAJOR, 3, torch.float32, 79)


@pytest.mark.parametrize("max_grid", [None, "24"])
@pytest.mark.parametrize("vec", ["2", "4"])
@pytest.mark.parametrize("pdtype", [torch.float32, torch.bfloat16])
def test_row_run_gather_at_both_vector_counts(gpu_lib, vec, pdtype, max_grid, monkeypatch):
    """The row-run gather with 2 and 4 vectors per thread (RS_GATHER_VEC forces the count; a
    plan takes 4 below 2^29 row-run elements, so every small group here would take 4), on the
    ragged and mid-size groups, with and without launches that loop over their runs."""
    import structure_aware_grouped_amd as rs
    monkeypatch.setenv("RS_GATHER_VEC", vec)
    if max_grid:
        monkeypatch.setenv("RS_MAX_GRID", max_grid)
    _full_check(rs, RAGGED, 6, pdtype, 41)
    _full_check(rs, MID, 7, pdtype, 42)


def test_trailing_padding_ranks(gpu_lib):
    """R_mat > R_used: ranks holding only padding come out zero."""
    import structure_aware_grouped_amd as rs
    specs = [TensorSpec("a", 64, 64, "TILE", 32, 32), TensorSpec("b", 100, 1, "ELEM")]
    _full_check(rs, specs, 16, torch.bfloat16, 3)


def test_bf16_pack_keeps_nan_and_overflows_to_infinity(gpu_lib):
    """A bf16 packed buffer from gradients holding NaN payloads that the rounding add would
    carry into the exponent (0x7FFFFFFF, 0xFFFFFFFF) and other NaNs: every NaN stays NaN
    (checked position by position against the oracle). Values past bf16's overflow midpoint
    come out as infinities, bit for bit, as do all finite values."""
    import structure_aware_grouped_amd as rs
    specs = [TensorSpec("a", 40, 48, "ROWS", 1), TensorSpec("b", 300, 1, "ELEM")]
    plan = _plan(rs, specs, 4)
    R, S = plan.R_mat, plan.S
    rng = _rng(77)
    specials = np.array([0x7FFFFFFF, 0xFFFFFFFF, 0x7FC00000, 0xFFC00001, 0x7FBFFFFF, 0x7F7FFFFF, 0xFF7FFFFF,
                         0x7F7F8000, 0x7F7F7FFF, 0x7F800000, 0xFF800000], dtype=np.uint32).view(np.float32)
    grads_h = []
    for sp in specs:
        g = _values(rng, sp.rows * sp.cols, scale=1e-3)
        pos = rng.choice(g.size, size=4 * specials.size, replace=False)
        g[pos] = np.tile(specials, 4)
        grads_h.append(g.reshape(sp.rows, sp.cols))
    grads = [torch.from_numpy(g).to(DEV) for g in grads_h]
    prev_h = _values(rng, R * S, scale=1e-3)
    prev = torch.from_numpy(prev_h).to(DEV)
    for acc in (False, True):
        whole, pb = guarded(R * S, torch.bfloat16, DEV)
        pb.view(torch.uint8).fill_(0xA5)
        rs.rs_pack_scatter(plan, grads, pb, prev=prev if acc else None, scale=1.0)
        torch.cuda.synchronize()
        want = OT.pack_to_bf16(grads_h, prev_h if acc else None, specs, plan.starts, S, R, np.float32(1.0), acc)
        got = tensor_bits(pb)
        as_f32 = lambda b: (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
        nan_w, nan_g = np.isnan(as_f32(want)), np.isnan(as_f32(got))
        assert nan_w.sum() >= 4 * 5 * len(specs) and np.array_equal(nan_w, nan_g), acc
        assert np.array_equal(got[~nan_w], want[~nan_w]), acc
        assert np.isinf(as_f32(got)).sum() >= 4 * 5 * len(specs), acc
        assert guard_intact(whole, R * S)
    plan.close()


def test_single_element_group(gpu_lib):
    import structure_aware_grouped_amd as rs
    _full_check(rs, [TensorSpec("x", 1, 1, "FLAT", 1)], 1, torch.float32, 5)
    _full_check(rs, [TensorSpec("x", 1, 1, "TILE", 1, 1)], 3, torch.bfloat16, 6)


@pytest.mark.parametrize("encoder", ["sw", "hw"])
def test_e4m3_encoder_every_mantissa(gpu_lib, encoder, monkeypatch):
    """Every fp32 value of magnitude in [2^-20, 448), both signs (all 2^23 mantissas of each
    binade), plus signed zeros and subnormals, through rs_block_quant with a 448 pivot at
    the head of each 2048-element block (so r = 1 and y = x). Everything below 2^-20 lies
    under half the smallest E4M3 subnormal and must encode as a signed zero."""
    import structure_aware_grouped_amd as rs
    monkeypatch.setenv("RS_E4M3_ENCODER", encoder)
    b = 2047
    per = 2 * (1 << 23)
    nblk = -(-per // b)
    spec = [TensorSpec("sweep", nblk, 2048, "FLAT", 2048)]
    plan = rs.rs_plan_load(spec, 1, nblk * 2048, [0], 1, 0)
    q = torch.empty(nblk * 2048, dtype=torch.uint8, device=DEV)
    sc = torch.empty(nblk, dtype=torch.float32, device=DEV)
    m = np.arange(1 << 23, dtype=np.uint32)
    tiny = np.float32([0.0, -0.0, 2.0 ** -149, -(2.0 ** -149), 2.0 ** -127, 2.0 ** -21, -(2.0 ** -21)])
    for e in range(-20, 9):
        x = (np.uint32((e + 127) << 23) | m).view(np.float32)
        x = x[x < 448]
        x = np.concatenate([x, -x, tiny])
        data = np.zeros((nblk, 2048), dtype=np.float32)
        data[:, 0] = 448.0
        flat = np.zeros(nblk * b, dtype=np.float32)
        flat[: x.size] = x
        data[:, 1:] = flat.reshape(nblk, b)
        rs.rs_block_quant(plan, torch.from_numpy(data.ravel()).to(DEV), q, "e4m3", sc)
        got = tensor_bits(q).reshape(nblk, 2048)
        assert np.all(tensor_bits(sc) == np.float32(1.0).view(np.uint32)), e
        assert np.all(got[:, 0] == 0x7E), e
        assert np.array_equal(got[:, 1:].ravel()[: x.size], OC.e4m3_encode(x)), e
    # decode of every code through dequant with unit scales
    codes_all = np.tile(np.arange(256, dtype=np.uint8), 8)
    spec2 = [TensorSpec("codes", 1, 2048, "FLAT", 2048)]
    plan2 = rs.rs_plan_load(spec2, 1, 2048, [0], 1, 0)
    out = torch.empty(2048, dtype=torch.float32, device=DEV)
    rs.rs_block_dequant(plan2, torch.from_numpy(codes_all).to(DEV), "e4m3",
                        torch.ones(1, dtype=torch.float32, device=DEV), out)
    dec = out.cpu().numpy().astype(np.float64)
    ref = OC.e4m3_decode(codes_all)
    assert np.all(((dec == ref) & (np.signbit(dec) == np.signbit(ref))) | (np.isnan(dec) & np.isnan(ref)))
    plan.close()
    plan2.close()


@pytest.mark.parametrize("fmt,encoder", [("e4m3", "sw"), ("e4m3", "hw"), ("i8", "sw"), ("u8", "sw")])
def test_special_blocks(gpu_lib, fmt, encoder, monkeypatch):
    """All-zero, subnormal-amax, constant, single-outlier and signed-zero blocks, and blocks that
    hold a NaN (quiet, signalling, negative) or an infinity: codes and scales bit for bit; the
    dequantised values bit for bit, NaN where the oracle has NaN (a NaN's sign and payload carry
    no meaning: 0 x inf gives the platform's default NaN)."""
    import structure_aware_grouped_amd as rs
    monkeypatch.setenv("RS_E4M3_ENCODER", encoder)
    b = 256
    blocks = [
        np.zeros(b, np.float32),
        np.full(b, 1e-41, np.float32) * np.sign(np.arange(b) % 3 - 1).astype(np.float32),
        np.full(b, 3.25, np.float32),
        np.where(np.arange(b) == 17, 1e4, 1e-3).astype(np.float32),
        np.where(np.arange(b) % 2 == 0, -0.0, 0.5).astype(np.float32),
        (np.random.default_rng(1).standard_normal(b) * 1e-30).astype(np.float32),
        np.float32(np.random.default_rng(2).standard_normal(b) * 1e30),
    ]
    for k, bad in enumerate([0x7FC00000, 0x7F800001, 0xFFC00000, 0x7F800000, 0xFF800000]):
        x = np.random.default_rng(10 + k).standard_normal(b).astype(np.float32)
        x[(37 * k) % b] = np.uint32(bad).view(np.float32)
        blocks.append(x)
    x = np.random.default_rng(20).standard_normal(b).astype(np.float32)   # a NaN and an infinity
    x[5], x[200] = np.inf, np.nan
    blocks.append(x)
    data = np.concatenate(blocks)
    if fmt == "u8":
        data = np.abs(data)
    spec = [TensorSpec("s", 1, data.size, "FLAT", b)]
    plan = rs.rs_plan_load(spec, 1, data.size, [0], 1, 0)
    q = torch.empty(data.size, dtype=torch.uint8, device=DEV)
    sc = torch.empty(len(blocks), dtype=torch.float32, device=DEV)
    rs.rs_block_quant(plan, torch.from_numpy(data).to(DEV), q, fmt, sc)
    wq, ws = OT.block_quant(data, spec, [0], data.size, 1, fmt)
    assert np.array_equal(tensor_bits(q), wq)
    assert np.array_equal(tensor_bits(sc), ws.view(np.uint32))
    out = torch.empty(data.size, dtype=torch.float32, device=DEV)
    rs.rs_block_dequant(plan, q, fmt, sc, out)
    want = OT.block_dequant(wq, ws, spec, [0], data.size, 1, fmt)
    got = out.cpu().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 6 * b
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))
    full = torch.empty(1, data.size, dtype=torch.float32, device=DEV)      # the gather side
    rs.rs_unpack_dequant(plan, q, fmt, sc, [full])
    got = full.cpu().numpy().ravel()
    assert np.array_equal(np.isnan(got), nan) and np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))
    plan.close()


def test_pointer_table_refresh(gpu_lib):
    """New destination / source tensors on a later call are picked up."""
    import structure_aware_grouped_amd as rs
    specs = RAGGED[:4]
    plan = _plan(rs, specs, 4)
    rng = _rng(9)
    G, Gh, xs = _flat_input(rng, plan, torch.float32)
    for _ in range(3):
        outs = [torch.zeros(sp.rows, sp.cols, device=DEV) for sp in specs]
        rs.rs_unpack_gathered(plan, G, outs)
        for o, x in zip(outs, xs):
            assert np.array_equal(tensor_bits(o).ravel(), x.view(np.uint32))
    for k in range(3):
        grads_h = [_values(rng, sp.rows * sp.cols) for sp in specs]
        packed = torch.empty(plan.R_mat * plan.S, device=DEV)
        rs.rs_pack_scatter(plan, [torch.from_numpy(g).to(DEV) for g in grads_h], packed)
        want = OT.pack(grads_h, None, specs, plan.starts, plan.S, plan.R_mat, OT.inv_v(4), False)
        assert np.array_equal(tensor_bits(packed), want.view(np.uint32))
    plan.close()


def test_calls_on_a_side_stream(gpu_lib):
    """Every call runs on torch's current stream: on a side stream (default
    priority) the results, including a changed pointer table, arrive in order."""
    import structure_aware_grouped_amd as rs
    specs = RAGGED
    plan = _plan(rs, specs, 3)
    rng = _rng(21)
    G, Gh, xs = _flat_input(rng, plan, torch.bfloat16)
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        for k in range(2):   # the second round brings new tensors, so a new pointer table
            outs = [garbage(sp.rows * sp.cols, torch.bfloat16, DEV).view(sp.rows, sp.cols) for sp in specs]
            rs.rs_unpack_gathered(plan, G, outs)
            q = garbage(plan.R_mat * plan.S, torch.uint8, DEV)
            scales = garbage(max(plan.n_qblocks, 1), torch.float32, DEV)
            rs.rs_block_quant(plan, G, q, "e4m3", scales)
    side.synchronize()
    want = OT.unpack(tensor_bits(G), specs, plan.starts)
    for o, wv in zip(outs, want):
        assert np.array_equal(tensor_bits(o), wv)
    wq, ws = OT.block_quant(Gh, specs, plan.starts, plan.S, plan.R_mat, "e4m3")
    assert np.array_equal(tensor_bits(q), wq)
    assert np.array_equal(tensor_bits(scales)[: plan.n_qblocks], ws.view(np.uint32))
    plan.close()


def test_bad_arguments_launch_nothing(gpu_lib):
    import structure_aware_grouped_amd as rs
    from structure_aware_grouped_amd import binding as b
    specs = [TensorSpec("a", 64, 64, "TILE", 16, 16)]
    plan = _plan(rs, specs, 2)
    total = plan.R_mat * plan.S
    G = torch.zeros(total + 4, device=DEV)
    dst = [torch.full((64, 64), 7.0, device=DEV)]
    lib = b.load()
    st = lib.rs_unpack_gathered(plan.handle, G[1:].data_ptr(), b.RS_F32, b._ptrs(dst),
                                b._stream(0))
    assert st == b.RS_EALIGN
    st = lib.rs_unpack_gathered(plan.handle, G.data_ptr(), 9, b._ptrs(dst), b._stream(0))
    assert st == b.RS_EDTYPE
    q = torch.full((total,), 3, dtype=torch.uint8, device=DEV)
    sc = torch.empty(plan.n_qblocks, device=DEV)
    st = lib.rs_block_quant(plan.handle, G.data_ptr(), b.RS_F32, q.data_ptr(), b.RS_F32,
                            sc.data_ptr(), b._stream(0))
    assert st == b.RS_EDTYPE
    st = lib.rs_pack_scatter(plan.handle, b._ptrs([dst[0]]), b.RS_E4M3, None, G.data_ptr(), b.RS_F32, 0,
                             0.0, b._stream(0))
    assert st == b.RS_EDTYPE
    st = lib.rs_pack_scatter(plan.handle, b._ptrs([dst[0]]), b.RS_F32, None, G.data_ptr(), b.RS_E4M3, 0,
                             0.0, b._stream(0))
    assert st == b.RS_EDTYPE
    # a bf16 packed buffer cannot also be the fp32 accumulator
    st = lib.rs_pack_scatter(plan.handle, b._ptrs([dst[0]]), b.RS_F32, G.data_ptr(), G.data_ptr(), b.RS_BF16, 0,
                             0.0, b._stream(0))
    assert st == b.RS_EINVAL
    torch.cuda.synchronize()
    assert bool((dst[0] == 7.0).all()) and bool((q == 3).all()) and bool((G == 0).all())
    plan.close()


def test_plan_reloaded_from_json(gpu_lib):
    """A plan saved as JSON and loaded again drives the kernels exactly like the original."""
    import structure_aware_grouped_amd as rs
    rng = _rng(2024)
    V = 6
    a = _plan(rs, RAGGED, V)
    specs, V2, S, starts, R = rs.plan_from_json(a.to_json())
    b = rs.rs_plan_load(specs, V2, S, starts, R, 0)
    assert (b.S, b.starts, b.R_mat, b.n_qblocks, b.padding) == (a.S, a.starts, a.R_mat, a.n_qblocks, a.padding)
    G, _, _ = _flat_input(rng, a, torch.bfloat16)
    grads = [torch.from_numpy(_values(rng, sp.rows * sp.cols, scale=1e-3)).to(DEV).view(sp.rows, sp.cols)
             for sp in RAGGED]
    prev = torch.from_numpy(_values(rng, a.R_mat * a.S, scale=1e-3)).to(DEV)
    res = []
    for plan in (a, b):
        outs = [garbage(sp.rows * sp.cols, torch.bfloat16, DEV).view(sp.rows, sp.cols) for sp in RAGGED]
        rs.rs_unpack_gathered(plan, G, outs)
        packed = garbage(plan.R_mat * plan.S, torch.float32, DEV)
        rs.rs_pack_scatter(plan, grads, packed, prev=prev)
        q = garbage(plan.R_mat * plan.S, torch.uint8, DEV)
        scales = garbage(plan.n_qblocks, torch.float32, DEV)
        rs.rs_block_quant(plan, G, q, "e4m3", scales)
        torch.cuda.synchronize()
        res.append([tensor_bits(t) for t in (*outs, packed, q, scales)])
    assert all(np.array_equal(x, y) for x, y in zip(*res))
    a.close()
    b.close()


# Tensors whose tile rows start inside 128-byte lines of codes, so neighbouring tiles (run by
# different workgroups) write the two halves of a line: 2880-wide rows of 128x128 tiles (the
# MoE layer's shape, 22 full tiles and a 64-wide edge tile a band, a partial last band), 8.5
# tiles of 64x128, 256-wide tiles, 64-wide tiles, and a tile-major, a flat and a row tensor in
# the same plan.
SPLIT_LINES = [
    TensorSpec("moe_like", 300, 2880, "TILE", 128, 128),
    TensorSpec("eight_and_half", 130, 1088, "TILE", 64, 128),
    TensorSpec("wide_tiles", 200, 1344, "TILE", 128, 256),
    TensorSpec("narrow_tiles", 70, 200, "TILE", 32, 64),
    TensorSpec("tm", 64, 128, "TILEMAJOR", 32, 32),
    TensorSpec("flat", 1, 10000, "FLAT", 2048),
    TensorSpec("norm", 2880, 1, "ROWS", 1),
]


@pytest.mark.parametrize("max_grid", [None, "16"])
@pytest.mark.parametrize("pdtype", [torch.float32, torch.bfloat16])
def test_quant_of_tiles_that_share_lines_of_codes(gpu_lib, max_grid, pdtype, monkeypatch):
    """Codes and scales bit for bit against the oracle in every format when neighbouring
    tiles share 128-byte lines of codes (the MoE-shaped band, the partial last band, the
    edge tiles); RS_MAX_GRID=16 once, so workgroups loop over tiles."""
    import structure_aware_grouped_amd as rs
    if max_grid:
        monkeypatch.setenv("RS_MAX_GRID", max_grid)
    V = 5
    plan = _plan(rs, SPLIT_LINES, V)
    R, S = plan.R_mat, plan.S
    total = R * S
    rng = _rng(300 + (16 if max_grid else 0) + (1 if pdtype == torch.bfloat16 else 0))
    for fmt in ("e4m3", "i8", "u8"):
        src_dev, src_h, _ = _flat_input(rng, plan, pdtype, scale=0.3, positive=(fmt == "u8"))
        qwhole, q = guarded(total, torch.uint8, DEV)
        q.fill_(0x5A)
        swhole, scales = guarded(plan.n_qblocks, torch.float32, DEV)
        rs.rs_block_quant(plan, src_dev, q, fmt, scales)
        torch.cuda.synchronize()
        wq, ws = OT.block_quant(src_h, SPLIT_LINES, plan.starts, S, R, fmt)
        assert np.array_equal(tensor_bits(q), wq), fmt
        assert np.array_equal(tensor_bits(scales), ws.view(np.uint32)), fmt
        assert guard_intact(qwhole, total) and guard_intact(swhole, plan.n_qblocks)
    plan.close()
