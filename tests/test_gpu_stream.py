"""The streaming gate/up and down kernels of the small-batch path (T <= 64 tokens outside the
single-launch path, hidden size an even number of 128-column groups from 1280 to 2048), against the CPU oracle through the C ABI.

The cases cover M-tiles whose activation rows go through LDS (at most 4 rows) and larger
ones loaded straight into registers, experts with more than 16 rows (several M-tiles),
a hidden size whose second K chunk holds two groups, a small intermediate size,
8-bit routed experts, and a shared expert of either width (16-token tiles plus a ragged
one).  Each case also checks that the streaming kernels are the ones that ran and that
two calls agree bitwise.
"""

import pytest
import torch

import oracle
import synth
import weight_only_int4_rtn_amd as w4
from gpu_util import DEV, OracleExperts, bf16_to_dev, check_ffn, f32_to_dev, gpu_layer, say

pytestmark = pytest.mark.gpu

CASES = [
    # T, E, H, I, k, routed bits, shared bits
    (3, 32, 2048, 512, 8, 4, 0),
    (17, 32, 2048, 384, 4, 4, 0),
    (64, 8, 2048, 256, 4, 4, 0),
    (40, 16, 1280, 128, 2, 4, 0),
    (9, 32, 2048, 256, 4, 8, 0),
    (4, 32, 2048, 512, 8, 4, 8),
    (20, 32, 2048, 256, 4, 4, 8),
    (33, 32, 2048, 256, 4, 8, 4),
]


@pytest.mark.parametrize("T,E,H,I,k,bits,sbits", CASES)
def test_stream_gate_up(T, E, H, I, k, bits, sbits):
    say(f"stream T={T} E={E} H={H} I={I} k={k} bits={bits} shared={sbits}")
    group = 40 + T
    routed = gpu_layer(group, 0, E, H, I, bits)
    ref = OracleExperts(group, 0, H, I, bits)
    sh_gpu = sh_ref = None
    if sbits:
        sh_gpu = gpu_layer(group, 1, 1, H, I, sbits, shared=True)
        sh_ref = OracleExperts(group, 1, H, I, sbits, shared=True).shared_dict()
    x = synth.activations_bf16(500 + T, T, H)
    logits = synth.router_logits(500 + T, T, E)
    y, timings = w4.moe_w4a16_forward_timed(bf16_to_dev(x), *routed, top_k=k, bits=bits,
                                            router_logits=f32_to_dev(logits), shared=sh_gpu)
    names = [name for name, _ in timings]
    assert "gk_stream" in names and "dk_stream" in names, timings
    y_ref, _ = oracle.moe_layer(x, logits, k, *ref.as_args(), bits, shared=sh_ref)
    check_ffn(y, y_ref, f"stream T={T}")
    y2 = w4.moe_w4a16_forward(bf16_to_dev(x), *routed, top_k=k, bits=bits, router_logits=f32_to_dev(logits),
                              shared=sh_gpu)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "streaming result not bitwise reproducible"
