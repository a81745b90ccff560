"""Layer shapes for the planner padding study (shapes only; no values).

One FSDP group per decoder layer, from the public architectures the pages
evaluate padding on (walkthrough, the ablation paragraph on planner padding:
GPT-OSS-120B and DeepSeek-V3-671B, at 1x / 16x / 128x row granularity):

* GPT-OSS-120B: hidden 2880, 64 query heads and 8 key-value heads of width
  64, attention projections with biases, learned attention sinks, 128 experts
  whose gate/up (2 x 2880) and down projections are stored fused into one
  tensor each, as that model ships them, with their biases, and a 128-way
  router.
* DeepSeek-V3-671B (an MoE layer): hidden 7168, multi-head latent attention
  (q rank 1536, kv rank 512, 128 heads of 128 + 64 rope dims, value width 128),
  256 routed experts and one shared expert of width 2048, a 256-way router
  with its score-correction bias.

Beside them, the bench's own groups with the same block convention: the
Llama-3-8B layer and the 128-expert MoE layer, per-expert and with each
projection of all experts fused into one tensor.

A 2-D tensor gets ROWS(k) atomic blocks (k = the row granularity); a 1-D
tensor (norm, bias, sink) gets one-element blocks.
"""
from __future__ import annotations

from typing import List

from .configs import TensorSpec


def _mat(name, rows, cols, k):
    return TensorSpec(name, rows, cols, "ROWS", k)


def _vec(name, n):
    return TensorSpec(name, n, 1, "ROWS", 1)


def gpt_oss_120b_layer(k: int, fused_experts: bool = True) -> List[TensorSpec]:
    h, e, inter, hd, nq, nkv = 2880, 128, 2880, 64, 64, 8
    specs = [
        _vec("input_norm", h),
        _mat("q_proj", nq * hd, h, k), _vec("q_bias", nq * hd),
        _mat("k_proj", nkv * hd, h, k), _vec("k_bias", nkv * hd),
        _mat("v_proj", nkv * hd, h, k), _vec("v_bias", nkv * hd),
        _mat("o_proj", h, nq * hd, k), _vec("o_bias", h),
        _vec("sinks", nq),
        _vec("post_attn_norm", h),
        _mat("router", e, h, k), _vec("router_bias", e),
    ]
    if fused_experts:
        specs += [
            _mat("experts.gate_up", e * h, 2 * inter, k),
            _mat("experts.gate_up_bias", e, 2 * inter, k),
            _mat("experts.down", e * inter, h, k),
            _mat("experts.down_bias", e, h, k),
        ]
    else:
        for x in range(e):
            specs += [_mat(f"e{x}.gate_up", h, 2 * inter, k), _vec(f"e{x}.gate_up_bias", 2 * inter),
                      _mat(f"e{x}.down", inter, h, k), _vec(f"e{x}.down_bias", h)]
    return specs


def deepseek_v3_layer(k: int) -> List[TensorSpec]:
    h, heads, qr, kvr, nope, rope, vd, e, inter = 7168, 128, 1536, 512, 128, 64, 128, 256, 2048
    specs = [
        _vec("input_norm", h),
        _mat("q_a_proj", qr, h, k), _vec("q_a_norm", qr),
        _mat("q_b_proj", heads * (nope + rope), qr, k),
        _mat("kv_a_proj", kvr + rope, h, k), _vec("kv_a_norm", kvr),
        _mat("kv_b_proj", heads * (nope + vd), kvr, k),
        _mat("o_proj", h, heads * vd, k),
        _vec("post_attn_norm", h),
        _mat("gate", e, h, k), _vec("gate_bias", e),
    ]
    for x in range(e):
        specs += [_mat(f"e{x}.gate", inter, h, k), _mat(f"e{x}.up", inter, h, k), _mat(f"e{x}.down", h, inter, k)]
    specs += [_mat("shared.gate", inter, h, k), _mat("shared.up", inter, h, k), _mat("shared.down", h, inter, k)]
    return specs


def llama3_8b_layer(k: int) -> List[TensorSpec]:
    """The Llama-3-8B decoder layer of the bench (hidden 4096, 8 key-value heads of 128,
    FFN 14336), with k-row blocks instead of its 128x128 tiles."""
    h, kv, ffn = 4096, 1024, 14336
    return [_mat("wq", h, h, k), _mat("wk", kv, h, k), _mat("wv", kv, h, k), _mat("wo", h, h, k),
            _mat("gate", ffn, h, k), _mat("up", ffn, h, k), _mat("down", h, ffn, k),
            _vec("attn_norm", h), _vec("mlp_norm", h)]


def moe128_layer(k: int, fused_experts: bool = False) -> List[TensorSpec]:
    """The bench's MoE layer (128 experts of gate_up 5760x2880 and down 2880x2880, a
    128x2880 router) with k-row blocks: per-expert tensors as the bench stores them, or
    each projection of all experts fused into one tensor (128*5760 x 2880 and
    128*2880 x 2880)."""
    e, h, inter = 128, 2880, 2880
    if fused_experts:
        specs = [_mat("experts.gate_up", e * 2 * inter, h, k), _mat("experts.down", e * inter, h, k)]
    else:
        specs = []
        for x in range(e):
            specs += [_mat(f"e{x}.gate_up", 2 * inter, h, k), _mat(f"e{x}.down", inter, h, k)]
    return specs + [_mat("router", e, h, k)]


STUDY_LAYERS = {
    "gpt_oss_120b": lambda k: gpt_oss_120b_layer(k, fused_experts=True),
    "gpt_oss_120b_unfused": lambda k: gpt_oss_120b_layer(k, fused_experts=False),
    "deepseek_v3": deepseek_v3_layer,
    "llama3_8b": llama3_8b_layer,
    "moe128": lambda k: moe128_layer(k, fused_experts=False),
    "moe128_fused": lambda k: moe128_layer(k, fused_experts=True),
}
STUDY_GRANULARITIES = (1, 16, 128)
STUDY_FSDP_SIZES = (8, 16, 32, 64, 96, 128, 192, 256, 384, 512, 768, 1024)
