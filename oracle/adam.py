"""One 8-bit Adam step on block-quantised optimizer state, by definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages run 8-bit Adam on RaggedShard ([walk], 8-bit Adam paragraph:
optimizer statistics quantised in blocks that stay whole on their device, so
no device needs another device's block scales to requantise its part) but
give no update formula. Reading: the decoupled-weight-decay Adam update
(AdamW), applied to every element of every quantisation block of the plan,
with the state kept as block-quantised codes:

  host scalars (float64 from the fp32 hyper-parameters, then one rounding):
    c1 = fl32(1 - b1),  c2 = fl32(1 - b2)
    step_size    = fl32(lr / (1 - b1**t))
    inv_bc2_sqrt = fl32(1 / sqrt(1 - b2**t))
    decay        = fl32(1 - lr * wd)
  per element, every operation one fp32 round-to-nearest-even step:
    m0 = dec(qm) * sm,  v0 = dec(qv) * sv
    m1 = b1*m0 + c1*g
    v1 = b2*v0 + c2*(g*g)
    den = sqrt(v1) * inv_bc2_sqrt + eps
    p1 = p*decay - step_size*(m1 / den)
  per block: m1 requantised to int8 (signed), v1 to uint8, by the block
  quantisation rule (amax, scale = amax/Q, codes of x * min(Q/amax, FLT_MAX)).

Elements outside quantisation blocks (padding, unquantised tensors) are not
touched.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from .transform import dequant_values, f32, quant_blocks, quantize_block


@dataclass
class AdamHyper:
    lr: float
    beta1: float
    beta2: float
    eps: float
    weight_decay: float
    step: int


def host_scalars(h: AdamHyper):
    """The fp32 scalars of one step (each computed in float64, rounded once)."""
    b1, b2 = float(np.float32(h.beta1)), float(np.float32(h.beta2))
    lr, wd = float(np.float32(h.lr)), float(np.float32(h.weight_decay))
    return dict(
        b1=np.float32(b1), b2=np.float32(b2), eps=np.float32(h.eps),
        c1=np.float32(1.0 - b1), c2=np.float32(1.0 - b2),
        step_size=np.float32(lr / (1.0 - b1 ** int(h.step))),
        inv_bc2_sqrt=np.float32(1.0 / math.sqrt(1.0 - b2 ** int(h.step))),
        decay=np.float32(1.0 - lr * wd),
    )


def _mul(a, b):
    return f32(np.asarray(a, np.float32).astype(np.float64) * np.asarray(b, np.float32).astype(np.float64))


def _add(a, b):
    return f32(np.asarray(a, np.float32).astype(np.float64) + np.asarray(b, np.float32).astype(np.float64))


def _sub(a, b):
    return f32(np.asarray(a, np.float32).astype(np.float64) - np.asarray(b, np.float32).astype(np.float64))


def _div(a, b):
    return f32(np.asarray(a, np.float32).astype(np.float64) / np.asarray(b, np.float32).astype(np.float64))


def _sqrt(a):
    return f32(np.sqrt(np.asarray(a, np.float32).astype(np.float64)))


def update_values(p, g, m0, v0, k):
    """(p1, m1, v1) of the element-wise update with host scalars k."""
    m1 = _add(_mul(k["b1"], m0), _mul(k["c1"], g))
    v1 = _add(_mul(k["b2"], v0), _mul(k["c2"], _mul(g, g)))
    den = _add(_mul(_sqrt(v1), k["inv_bc2_sqrt"]), k["eps"])
    p1 = _sub(_mul(p, k["decay"]), _mul(k["step_size"], _div(m1, den)))
    return p1, m1, v1


def adam8_step(param, grad, qm, sm, qv, sv, specs, starts, h: AdamHyper):
    """New (param, qm, sm, qv, sv) as copies; inputs are flat buffers and scale arrays."""
    k = host_scalars(h)
    p_out, qm_out, qv_out = param.copy(), qm.copy(), qv.copy()
    sm_out, sv_out = np.array(sm, np.float32), np.array(sv, np.float32)
    for _, b, pos in quant_blocks(specs, starts):
        m0 = dequant_values(qm[pos], sm[b], "i8")
        v0 = dequant_values(qv[pos], sv[b], "u8")
        p1, m1, v1 = update_values(param[pos], grad[pos], m0, v0, k)
        p_out[pos] = p1
        qm_out[pos], sm_out[b] = quantize_block(m1, "i8")
        qv_out[pos], sv_out[b] = quantize_block(v1, "u8")
    return p_out, qm_out, sm_out, qv_out, sv_out
