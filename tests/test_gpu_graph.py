"""The forward call under HIP graph capture: replays, interleaved with eager work and
synchronisations, must reproduce the eager result bitwise (every path is deterministic:
no atomics take part in any sum)."""

import numpy as np
import pytest
import torch

import synth
import weight_only_int4_rtn_amd as w4
from gpu_util import DEV, bf16_to_dev, f32_to_dev, gpu_layer, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,E,H,I", [(1, 64, 512, 256), (32, 64, 512, 256), (300, 64, 512, 256),
                                     # pair mode of the stream; the split routing launch (its
                                     # arrival counter resets on every replay) and the stream
                                     (4, 256, 2048, 512), (32, 256, 2048, 512)])
def test_graph_replay_matches_eager(T, E, H, I):
    say(f"graph replay T={T} E={E} H={H}")
    k = 8
    w13, s13, w2, s2 = gpu_layer(21, 0, E, H, I, 4)
    x = bf16_to_dev(synth.activations_bf16(70 + T, T, H))
    logits = f32_to_dev(synth.router_logits(70 + T, T, E))
    ws = w4.new_workspace(w4.moe_w4a16_workspace_size(T, H, I, E, k), DEV)
    call = w4.MoeCall(x, w13, s13, w2, s2, top_k=k, workspace=ws)
    eager = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    call(x, eager, router_logits=logits)
    torch.cuda.synchronize()

    out = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(x, out, router_logits=logits)
    for rep in range(4):
        out.zero_()
        junk = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
        call(x, junk, router_logits=f32_to_dev(synth.router_logits(80 + rep, T, E)))   # eager work between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep} differs"
