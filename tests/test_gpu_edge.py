"""Edge cases of the expert FFN against the CPU oracle through the C ABI.

* Skewed routing at prefill sizes: every token's logits favour the same few experts, so
  those experts hold several 128-row tiles (one of them ragged) while most experts receive
  no token at all.
* The single-launch path (T * k <= 16) with every combination of routed code width,
  shared-expert width (none, 4-bit, 8-bit) and a residual, each checking that the
  single-launch kernel is the one that ran.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_int4_rtn_amd as w4
from gpu_util import OracleExperts, bf16_to_dev, check_ffn, f32_to_dev, gpu_layer, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,E,k,hot", [(600, 64, 4, 4), (300, 32, 8, 8), (257, 16, 2, 1)])
def test_prefill_skewed_routing(T, E, k, hot):
    """`hot` experts receive every token (the others none): hot <= k, so each hot expert
    holds T rows in ceil(T / 128) tiles."""
    say(f"prefill skewed T={T} E={E} k={k} hot={hot}")
    H, I, bits = 512, 256, 4
    w13, s13, w2, s2 = gpu_layer(61, 0, E, H, I, bits)
    ref = OracleExperts(61, 0, H, I, bits)
    x = synth.activations_bf16(900 + T, T, H)
    logits = synth.router_logits(900 + T, T, E)
    logits[:, :hot] += 20.0   # the hot experts win every token
    y, timings = w4.moe_w4a16_forward_timed(bf16_to_dev(x), w13, s13, w2, s2, top_k=k, bits=bits,
                                            router_logits=f32_to_dev(logits))
    names = [n for n, _ in timings]
    assert "gk_prefill" in names and "dk_prefill" in names, timings
    counts = oracle.route(logits, k)[2]
    assert (counts[:hot] == T).all() and counts.sum() == T * k
    y_ref, _ = oracle.moe_layer(x, logits, k, *ref.as_args(), bits)
    check_ffn(y, y_ref, f"skewed T={T}")


@pytest.mark.parametrize("T", [1, 2])
@pytest.mark.parametrize("bits,sbits", [(4, 0), (4, 4), (4, 8), (8, 0), (8, 4), (8, 8)])
def test_tiny_code_widths_shared_and_residual(T, bits, sbits):
    say(f"tiny T={T} routed bits={bits} shared bits={sbits}")
    E, H, I, k = 64, 1024, 256, 8
    routed = gpu_layer(71, 0, E, H, I, bits)
    ref = OracleExperts(71, 0, H, I, bits)
    sh_gpu = sh_ref = None
    if sbits:
        sh_gpu = gpu_layer(71, 1, 1, H, I, sbits, shared=True)
        sh_ref = OracleExperts(71, 1, H, I, sbits, shared=True).shared_dict()
    x = synth.activations_bf16(950 + T, T, H)
    res = synth.activations_bf16(960 + T, T, H)
    logits = synth.router_logits(950 + T + bits + sbits, T, E)
    y, timings = w4.moe_w4a16_forward_timed(bf16_to_dev(x), *routed, top_k=k, bits=bits,
                                            router_logits=f32_to_dev(logits), shared=sh_gpu,
                                            residual=bf16_to_dev(res))
    assert [n for n, _ in timings] == ["tiny_decode"], timings
    y_ref, _ = oracle.moe_layer(x, logits, k, *ref.as_args(), bits, shared=sh_ref, residual_bits=res)
    check_ffn(y, y_ref, f"tiny T={T} bits={bits} sbits={sbits}")
