"""GPU parity of the decode-stack configuration at full layer shape.

Each stack layer is one forward call with 4 tokens: 256 routed experts top-8 (INT4,
or INT8 on the 8-bit layers), one INT8 shared expert (2048 -> 512 -> 2048) with
weight 1, and the layer input added back as the residual.  The check is
teacher-forced: the oracle evaluates layer l on the GPU's own bf16 output of layer
l - 1, from its own quantization of the same seeded fp32 weights.
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_int4_rtn_amd as w4
from gpu_util import DEV, OracleExperts, bf16_from_dev, bf16_to_dev, check_ffn, f32_to_dev, gpu_layer, say

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


def _rms_normed(h_bits):
    """A layer's input: the residual stream divided by its per-token RMS (no weight), as a
    decoder's norm before each block gives it; the same host function serves both chains."""
    h = oracle.f32_from_bf16_bits(h_bits).astype(np.float64)
    r = np.sqrt(np.mean(h * h, axis=1, keepdims=True) + 1e-6)
    return oracle.bf16_bits_from_f32((h / r).astype(np.float32))


def test_stack_forty_layer_drift():
    """End-to-end drift of the 40-layer stack (information, with a loose guard).

    Each layer: y = h + MoE(norm(h)) with the INT8 shared expert, norm the per-token RMS
    normalization above (without one the synthetic residual stream grows until it
    overflows).  The GPU chain feeds each layer's bf16 output on; the oracle runs its own
    chain, each layer in fp64 from its own quantization of the same seeded weights, its
    output rounded to bf16 (through fp32) as the next layer's input.  Routing comes from
    given logits, so the two chains route alike and the difference is the arithmetic's
    alone.  Only the experts a layer's 4 tokens use are generated (the other experts'
    weights are zeros, which no kernel reads).
    """
    T, H, I, E, k = CFG.T, CFG.H, CFG.I, CFG.E, CFG.k
    h0 = synth.activations_bf16(synth.CONFIG_INDEX["stack40"], T, H)
    h_gpu = bf16_to_dev(h0)
    h_ref = h0
    worst = 0.0
    for layer in range(CFG.layers):
        bits = 8 if layer in CFG.int8_layers else 4
        logits = synth.router_logits(synth.CONFIG_INDEX["stack40"], T, E, layer=layer)
        used = sorted(set(int(e) for e in oracle.route(logits, k)[0].ravel() if e >= 0))
        w13 = torch.zeros((E, 2 * I, H * bits // 32), dtype=torch.int32, device=DEV)
        s13 = torch.zeros((E, 2 * I, H // 128), dtype=torch.bfloat16, device=DEV)
        w2 = torch.zeros((E, H, I * bits // 32), dtype=torch.int32, device=DEV)
        s2 = torch.zeros((E, H, I // 128), dtype=torch.bfloat16, device=DEV)
        ref = OracleExperts(CFG.group, layer, H, I, bits)

        def prep(e, layer=layer, bits=bits):   # the seeded fp32 weights and the oracle's codes
            f13 = synth.expert_w13(CFG.group, layer, e, H, I)
            f2 = synth.expert_w2(CFG.group, layer, e, H, I)
            return e, f13, f2, oracle.quantize_pack(f13, bits) + oracle.quantize_pack(f2, bits)

        with ThreadPoolExecutor(8) as ex:
            for e, f13, f2, q in ex.map(prep, used):
                w4.rtn_quantize_pack(f32_to_dev(f13[None]), bits, packed=w13[e:e + 1], scales=s13[e:e + 1])
                w4.rtn_quantize_pack(f32_to_dev(f2[None]), bits, packed=w2[e:e + 1], scales=s2[e:e + 1])
                ref.cache[e] = q
        shared = gpu_layer(CFG.group, layer, 1, H, CFG.shared_I, 8, shared=True)
        sref = OracleExperts(CFG.group, layer, H, CFG.shared_I, 8, shared=True)
        x_gpu = bf16_to_dev(_rms_normed(bf16_from_dev(h_gpu)))
        y = w4.moe_w4a16_forward(x_gpu, w13, s13, w2, s2, top_k=k, bits=bits, router_logits=f32_to_dev(logits),
                                 shared=shared, residual=h_gpu)
        torch.cuda.synchronize()
        y_ref, _ = oracle.moe_layer(_rms_normed(h_ref), logits, k, *ref.as_args(), bits, shared=sref.shared_dict(),
                                    residual_bits=h_ref)
        y64 = oracle.f32_from_bf16_bits(bf16_from_dev(y)).astype(np.float64)
        rel = np.abs(y64 - y_ref).max() / np.abs(y_ref).max()
        worst = max(worst, rel)
        say(f"  layer {layer:2d} (bits {bits}): max|d|/max|ref| = {rel:.3e}")
        h_gpu = y
        h_ref = oracle.bf16_bits_from_f32(y_ref.astype(np.float32))
        del w13, s13, w2, s2, shared
    say(f"stack drift after {CFG.layers} layers: max|d|/max|ref| = {rel:.3e} (worst layer {worst:.3e})")
    assert np.isfinite(worst) and worst <= 0.1
