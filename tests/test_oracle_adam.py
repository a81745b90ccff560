"""Pins of the 8-bit Adam step oracle.

  * every fp32 operation against exact rationals rounded by IEEE's definition
    (square root by exact comparison of squares);
  * torch.optim.AdamW (an independent implementation) on the same fp32
    states, to a few ulps (torch fuses and orders some operations
    differently, so this is a tolerance check of the formula, not of the
    roundings);
  * closed forms: zero gradient and state leave p * decay; zero weight decay
    and zero gradient leave p;
  * a planted mistake (no bias correction) fails the torch comparison.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import adam as A, plan as P, transform as T
from tests import exact
from workloads import TensorSpec


def _f(x):
    return Fraction(float(x))


def _r(q):
    return exact.round_f32(q)


def _exact_update(p, g, m0, v0, k):
    m1 = _r(_f(_r(_f(k["b1"]) * _f(m0))) + _f(_r(_f(k["c1"]) * _f(g))))
    gg = _r(_f(g) * _f(g))
    v1 = _r(_f(_r(_f(k["b2"]) * _f(v0))) + _f(_r(_f(k["c2"]) * _f(gg))))
    sq = exact.sqrt_f32(float(np.float32(v1)))
    den = _r(_f(_r(_f(sq) * _f(k["inv_bc2_sqrt"]))) + _f(k["eps"]))
    upd = _r(_f(m1) / _f(den))
    p1 = _r(_f(_r(_f(p) * _f(k["decay"]))) - _f(_r(_f(k["step_size"]) * _f(upd))))
    return p1, m1, v1


HYPERS = [A.AdamHyper(1e-3, 0.9, 0.999, 1e-8, 0.01, 1), A.AdamHyper(3e-4, 0.95, 0.98, 1e-6, 0.1, 17),
          A.AdamHyper(1e-2, 0.8, 0.9999, 1e-8, 0.0, 1000)]


@pytest.mark.parametrize("h", HYPERS)
def test_update_against_exact_rationals(h):
    rng = np.random.default_rng(h.step)
    n = 300
    p = rng.standard_normal(n).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    m0 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v0 = ((rng.standard_normal(n) * 1e-3) ** 2).astype(np.float32)
    g[:3] = 0.0
    k = A.host_scalars(h)
    p1, m1, v1 = A.update_values(p, g, m0, v0, k)
    for i in range(n):
        ep, em, ev = _exact_update(p[i], g[i], m0[i], v0[i], k)
        assert (p1[i], m1[i], v1[i]) == (np.float32(ep), np.float32(em), np.float32(ev)), i


def test_host_scalars_closed_form():
    k = A.host_scalars(A.AdamHyper(0.5, 0.5, 0.75, 0.0, 0.5, 1))
    assert k["step_size"] == np.float32(1.0)          # 0.5 / (1 - 0.5)
    assert k["inv_bc2_sqrt"] == np.float32(2.0)       # 1 / sqrt(1 - 0.75)
    assert k["decay"] == np.float32(0.75)             # 1 - 0.5 * 0.5
    assert k["c1"] == np.float32(0.5) and k["c2"] == np.float32(0.25)


def _torch_adamw(p, g, m0, v0, h):
    pt = torch.nn.Parameter(torch.from_numpy(p.copy()))
    opt = torch.optim.AdamW([pt], lr=float(np.float32(h.lr)), betas=(float(np.float32(h.beta1)), float(np.float32(h.beta2))),
                            eps=float(np.float32(h.eps)), weight_decay=float(np.float32(h.weight_decay)),
                            foreach=False, fused=False)
    pt.grad = torch.from_numpy(g.copy())
    st = opt.state[pt]
    st["step"] = torch.tensor(float(h.step - 1))
    st["exp_avg"] = torch.from_numpy(m0.copy())
    st["exp_avg_sq"] = torch.from_numpy(v0.copy())
    opt.step()
    return pt.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


@pytest.mark.parametrize("h", HYPERS)
def test_update_agrees_with_torch_adamw(h):
    rng = np.random.default_rng(100 + h.step)
    n = 20000
    p = rng.standard_normal(n).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    m0 = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    v0 = ((rng.standard_normal(n) * 1e-2) ** 2).astype(np.float32)
    p1, m1, v1 = A.update_values(p, g, m0, v0, A.host_scalars(h))
    tp, tm, tv = _torch_adamw(p, g, m0, v0, h)
    # a few ulps of the operands (torch forms m by lerp, v by a fused multiply-add)
    ulp_m = np.spacing(np.maximum.reduce([np.abs(m0), np.abs(g), np.abs(m1)]))
    ulp_v = np.spacing(np.maximum(np.abs(v0), np.abs(g * g)))
    assert np.all(np.abs(m1 - tm) <= 4 * ulp_m)
    assert np.all(np.abs(v1 - tv) <= 4 * ulp_v)
    # the parameter moves by step_size * m/den; compare the moves to a few ulps of the move
    np.testing.assert_allclose(p1 - p, tp - p, rtol=1e-5, atol=np.abs(p).max() * 2.0 ** -22)


def test_closed_forms():
    h = A.AdamHyper(1e-3, 0.9, 0.999, 1e-8, 0.01, 5)
    k = A.host_scalars(h)
    p = np.float32([1.5, -2.0, 3e-5])
    z = np.zeros(3, np.float32)
    p1, m1, v1 = A.update_values(p, z, z, z, k)
    assert np.array_equal(p1, T.f32(p.astype(np.float64) * float(k["decay"]))) and not m1.any() and not v1.any()
    k0 = A.host_scalars(A.AdamHyper(1e-3, 0.9, 0.999, 1e-8, 0.0, 5))
    assert np.array_equal(A.update_values(p, z, z, z, k0)[0], p)


def test_step_quantises_each_block_and_leaves_the_rest():
    specs = [TensorSpec("a", 64, 32, "TILE", 16, 16), TensorSpec("n", 7, 1, "ROWS", 1),
             TensorSpec("f", 1, 3000, "FLAT", 512)]
    V = 4
    p = P.plan(specs, V)
    rng = np.random.default_rng(3)
    total = V * p.S
    param = rng.standard_normal(total).astype(np.float32)
    grad = (rng.standard_normal(total) * 1e-3).astype(np.float32)
    m = (rng.standard_normal(total) * 1e-3).astype(np.float32)
    v = ((rng.standard_normal(total) * 1e-3) ** 2).astype(np.float32)
    qm, sm = T.block_quant(m, specs, p.starts, p.S, V, "i8")
    qv, sv = T.block_quant(v, specs, p.starts, p.S, V, "u8")
    h = HYPERS[0]
    p1, qm1, sm1, qv1, sv1 = A.adam8_step(param, grad, qm, sm, qv, sv, specs, p.starts, h)
    inside = np.zeros(total, bool)
    for _, b, pos in T.quant_blocks(specs, p.starts):
        inside[pos] = True
        m0 = T.dequant_values(qm[pos], sm[b], "i8")
        v0 = T.dequant_values(qv[pos], sv[b], "u8")
        want_p, want_m, want_v = A.update_values(param[pos], grad[pos], m0, v0, A.host_scalars(h))
        assert np.array_equal(p1[pos], want_p)
        c, s = T.quantize_block(want_m, "i8")
        assert np.array_equal(qm1[pos], c) and sm1[b] == s
    assert np.array_equal(p1[~inside], param[~inside]) and np.array_equal(qm1[~inside], qm[~inside])


def test_a_nan_gradient_blanks_its_blocks_only():
    """Reading (non-finite blocks): a NaN gradient makes that element's m1, v1 and parameter NaN;
    its m and v blocks get NaN scales and all-zero codes, so the next step reads NaN state for the
    whole block; every other block steps as without the NaN."""
    specs = [TensorSpec("f", 1, 2048, "FLAT", 512)]
    rng = np.random.default_rng(5)
    param = rng.standard_normal(2048).astype(np.float32)
    grad = (rng.standard_normal(2048) * 1e-3).astype(np.float32)
    m = (rng.standard_normal(2048) * 1e-3).astype(np.float32)
    v = ((rng.standard_normal(2048) * 1e-3) ** 2).astype(np.float32)
    qm, sm = T.block_quant(m, specs, [0], 2048, 1, "i8")
    qv, sv = T.block_quant(v, specs, [0], 2048, 1, "u8")
    h = HYPERS[0]
    clean = A.adam8_step(param, grad, qm, sm, qv, sv, specs, [0], h)
    g2 = grad.copy()
    g2[700] = np.nan                                            # block 1 (elements 512..1023)
    with np.errstate(invalid="ignore"):
        p1, qm1, sm1, qv1, sv1 = A.adam8_step(param, g2, qm, sm, qv, sv, specs, [0], h)
    blk = slice(512, 1024)
    assert np.isnan(p1[700]) and np.isnan(p1).sum() == 1
    assert not qm1[blk].any() and not qv1[blk].any()
    assert sm1.view(np.uint32)[1] == 0x7FC00000 and sv1.view(np.uint32)[1] == 0x7FC00000
    for k in (0, 2, 3):
        rest = slice(512 * k, 512 * (k + 1))
        assert np.array_equal(p1[rest], clean[0][rest]) and np.array_equal(qm1[rest], clean[1][rest])
        assert sm1[k] == clean[2][k] and sv1[k] == clean[4][k]
    with np.errstate(invalid="ignore"):                        # the next step: the whole block is NaN
        p2 = A.adam8_step(p1, grad, qm1, sm1, qv1, sv1, specs, [0], h)[0]
    assert np.isnan(p2[blk]).all() and not np.isnan(p2[:512]).any()


def test_pin_catches_a_missing_bias_correction(monkeypatch):
    orig = A.host_scalars

    def no_bc(h):
        k = orig(h)
        k["step_size"] = np.float32(h.lr)
        k["inv_bc2_sqrt"] = np.float32(1.0)
        return k

    monkeypatch.setattr(A, "host_scalars", no_bc)
    with pytest.raises(AssertionError):
        test_update_agrees_with_torch_adamw(HYPERS[1])
