"""GPU parity of the decode-stack configuration at full layer shape.

Each stack layer is one forward call with 4 tokens: 256 routed experts top-8 (INT4,
or INT8 on the 8-bit layers), one INT8 shared expert (2048 -> 512 -> 2048) with
weight 1, and the layer input added back as the residual.  The check is
teacher-forced: the oracle evaluates layer l on the GPU's own bf16 output of layer
l - 1, from its own quantization of the same seeded fp32 weights.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_int4_rtn_amd as w4
from gpu_util import OracleExperts, bf16_from_dev, bf16_to_dev, check_ffn, f32_to_dev, gpu_layer, say

pytestmark = pytest.mark.gpu

CFG = synth.CONFIGS["stack40"]


def _layer(layer):
    bits = 8 if layer in CFG.int8_layers else 4
    routed = gpu_layer(CFG.group, layer, CFG.E, CFG.H, CFG.I, bits)
    shared = gpu_layer(CFG.group, layer, 1, CFG.H, CFG.shared_I, 8, shared=True)
    ref = OracleExperts(CFG.group, layer, CFG.H, CFG.I, bits)
    sref = OracleExperts(CFG.group, layer, CFG.H, CFG.shared_I, 8, shared=True)
    return bits, routed, shared, ref, sref


def _forward(h_bits, layer, bits, routed, shared):
    logits = synth.router_logits(synth.CONFIG_INDEX["stack40"], CFG.T, CFG.E, layer=layer)
    h = bf16_to_dev(h_bits)
    w13, s13, w2, s2 = routed
    y = w4.moe_w4a16_forward(h, w13, s13, w2, s2, top_k=CFG.k, bits=bits, router_logits=f32_to_dev(logits),
                             shared=shared, residual=h)
    torch.cuda.synchronize()
    return y, logits


def test_stack_chain_teacher_forced():
    """Layers 6 (INT4 experts) and 7 (INT8 experts), each with the INT8 shared expert."""
    h = synth.activations_bf16(synth.CONFIG_INDEX["stack40"], CFG.T, CFG.H)
    for layer in (6, 7):
        say(f"stack layer {layer}")
        bits, routed, shared, ref, sref = _layer(layer)
        y, logits = _forward(h, layer, bits, routed, shared)
        y_ref, _ = oracle.moe_layer(h, logits, CFG.k, *ref.as_args(), bits, shared=sref.shared_dict(),
                                    residual_bits=h)
        check_ffn(y, y_ref, f"stack layer {layer} (bits {bits})")
        # the layer's own contribution, against the oracle's, beside the bf16 rounding of h
        delta = oracle.f32_from_bf16_bits(bf16_from_dev(y)).astype(np.float64) - \
            oracle.f32_from_bf16_bits(h).astype(np.float64)
        delta_ref = y_ref - oracle.f32_from_bf16_bits(h).astype(np.float64)
        ulp = np.abs(y_ref).max() * 2.0 ** -8
        assert np.abs(delta - delta_ref).max() <= ulp + 2e-2 * np.abs(delta_ref).max()
        h = bf16_from_dev(y)


@pytest.mark.parametrize("layer", [0, 13])
def test_stack_layer_in_place_residual(layer):
    """The output may overwrite the residual buffer (the stack's in-place update)."""
    say(f"stack layer {layer} in place")
    h = synth.activations_bf16(90 + layer, CFG.T, CFG.H)
    bits, routed, shared, ref, sref = _layer(layer)
    logits = synth.router_logits(synth.CONFIG_INDEX["stack40"], CFG.T, CFG.E, layer=layer)
    x = bf16_to_dev(h)
    res = bf16_to_dev(h)
    w13, s13, w2, s2 = routed
    w4.moe_w4a16_forward(x, w13, s13, w2, s2, top_k=CFG.k, bits=bits, router_logits=f32_to_dev(logits),
                         shared=shared, residual=res, out=res)
    torch.cuda.synchronize()
    y_ref, _ = oracle.moe_layer(h, logits, CFG.k, *ref.as_args(), bits, shared=sref.shared_dict(), residual_bits=h)
    check_ffn(res, y_ref, f"layer {layer} in place")
