"""W4A16_FLAG_NO_COOPERATIVE: with it, 1- and 2-token batches leave the single-launch kernel
(whose gate/up and down workgroups wait for each other) for the multi-launch streaming
path; both are held to the oracle, and unknown flag bits are rejected before any launch."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_int4_rtn_amd as w4
from gpu_util import DEV, OracleExperts, bf16_to_dev, check_ffn, f32_to_dev, gpu_layer, say

pytestmark = pytest.mark.gpu

H, I, K, E = 2048, 512, 8, 64


@pytest.mark.parametrize("T,shared_bits", [(1, 0), (2, 8)])
def test_no_cooperative_takes_the_stream(T, shared_bits):
    say(f"flags T={T} shared={shared_bits}")
    routed = gpu_layer(95, 0, E, H, I, 4)
    ref = OracleExperts(95, 0, H, I, 4)
    sh = gpu_layer(95, 0, 1, H, 512, shared_bits, shared=True) if shared_bits else None
    sh_ref = OracleExperts(95, 0, H, 512, shared_bits, shared=True).shared_dict() if shared_bits else None
    x = synth.activations_bf16(1000 + T, T, H)
    logits = synth.router_logits(1000 + T, T, E)
    ids, wts, *_ = oracle.route(logits, K)
    y_ref = oracle.moe_ffn(x, ids, wts, *ref.as_args(), 4, shared=sh_ref)
    ws = w4.new_workspace(w4.moe_w4a16_workspace_size(T, H, I, E, K, shared_bits, 512 if shared_bits else 0), DEV)
    for coop in (True, False, True):   # the single-launch path still works on the workspace afterwards
        y, tk = w4.moe_w4a16_forward_timed(bf16_to_dev(x), *routed, top_k=K, router_logits=f32_to_dev(logits),
                                           shared=sh, workspace=ws, cooperative=coop)
        names = [n for n, _ in tk]
        if coop:
            assert names == ["tiny_decode"], names
        else:
            assert "tiny_decode" not in names and "dk_stream" in names, names
        check_ffn(y, y_ref, f"T={T} cooperative={coop}")
    assert not w4.moe_w4a16_workspace_check(ws)


def test_unknown_flags_rejected():
    T, Es, Hs = 4, 16, 256
    lay = tuple(torch.zeros(s, dtype=d, device=DEV) for s, d in
                (((Es, 256, 32), torch.int32), ((Es, 256, 2), torch.bfloat16), ((Es, Hs, 16), torch.int32),
                 ((Es, Hs, 1), torch.bfloat16)))
    x = bf16_to_dev(synth.activations_bf16(1, T, Hs))
    logits = f32_to_dev(synth.router_logits(1, T, Es))
    a = w4._args(x, *lay, 2, 4, logits, None, None, None, None, torch.empty_like(x), None, None, None,
                 torch.zeros(1 << 20, dtype=torch.uint8, device=DEV))
    a.flags = 6   # bit 2 is not a flag
    assert w4._lib.lib().moe_w4a16_forward(ctypes.byref(a), None) == w4._lib.W4A16_ERR_INVALID_ARG
    assert "flags" in w4._lib.last_error()
