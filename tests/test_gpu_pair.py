"""Pair mode of the streaming gate/up (T * top_k <= 64 pairs, at least twice as many experts
as pairs, outside the single-launch path), against the CPU oracle through the C ABI.

Workgroup 0 of the gate/up launch routes the batch and writes the routing outputs; the
routed tiles of every other workgroup's range are (token, rank) pairs, whose experts it
finds with a top-k that stops at the pair's rank, and it writes each pair's a row, which
the streaming down kernel finds through the pair indices of its tile records.
The cases cover the 40-layer stack's shapes (4 tokens, INT4 or INT8 routed experts and an
INT8 shared expert), the 64-pair boundary, a shared expert spanning two M-tiles (one of
them ragged), a hidden size of 1280, experts chosen by several tokens, and caller-supplied
ids with dropped pairs.  Each case checks that the pair kernel is the one that ran, the
routing outputs bit for bit, and that two calls agree bitwise.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_int4_rtn_amd as w4
from gpu_util import DEV, OracleExperts, bf16_to_dev, check_ffn, f32_to_dev, gpu_layer, say

pytestmark = pytest.mark.gpu

CASES = [
    # T, E, H, I, k, routed bits, shared bits
    (4, 256, 2048, 512, 8, 4, 8),
    (4, 256, 2048, 512, 8, 8, 8),
    (3, 64, 2048, 512, 8, 4, 0),
    (8, 256, 2048, 512, 8, 4, 4),
    (20, 128, 2048, 256, 3, 4, 8),
    (5, 64, 1280, 128, 4, 4, 0),
]


def _names(timings):
    return [name for name, _ in timings]


@pytest.mark.parametrize("T,E,H,I,k,bits,sbits", CASES)
def test_pair_gate_up(T, E, H, I, k, bits, sbits):
    say(f"pair T={T} E={E} H={H} I={I} k={k} bits={bits} shared={sbits}")
    group = 70 + T
    routed = gpu_layer(group, 0, E, H, I, bits)
    ref = OracleExperts(group, 0, H, I, bits)
    sh_gpu = sh_ref = None
    if sbits:
        sh_gpu = gpu_layer(group, 1, 1, H, I, sbits, shared=True)
        sh_ref = OracleExperts(group, 1, H, I, sbits, shared=True).shared_dict()
    x = synth.activations_bf16(700 + T, T, H)
    logits = synth.router_logits(700 + T, T, E)
    if T >= 3:   # tokens that share experts: identical logits for tokens 1 and 2
        logits[2] = logits[1]
    (y, r), timings = w4.moe_w4a16_forward_timed(bf16_to_dev(x), *routed, top_k=k, bits=bits,
                                                 router_logits=f32_to_dev(logits), shared=sh_gpu, routing_out=True)
    names = _names(timings)
    assert "gk_pair_stream" in names and "dk_stream" in names and "gk_stream" not in names, timings
    ids, w, counts, offsets, pairs = oracle.route(logits, k)
    assert np.array_equal(r["ids"].cpu().numpy(), ids)
    assert np.array_equal(r["counts"].cpu().numpy(), counts)
    assert np.array_equal(r["offsets"].cpu().numpy(), offsets)
    assert np.array_equal(r["sorted_pairs"].cpu().numpy(), pairs)
    assert np.abs(r["w"].cpu().numpy() - w).max() <= 1e-6
    y_ref, _ = oracle.moe_layer(x, logits, k, *ref.as_args(), bits, shared=sh_ref)
    check_ffn(y, y_ref, f"pair T={T}")
    y2 = w4.moe_w4a16_forward(bf16_to_dev(x), *routed, top_k=k, bits=bits, router_logits=f32_to_dev(logits),
                              shared=sh_gpu)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "pair result not bitwise reproducible"


def test_pair_given_ids_with_dropped_pairs():
    """Caller-supplied ids: out-of-range ids and repeats within a token contribute
    nothing, and an expert picked by every token is read once per pair."""
    E, H, I, k, T = 64, 2048, 256, 4, 6
    say("pair given ids with dropped pairs")
    routed = gpu_layer(79, 0, E, H, I, 4)
    ref = OracleExperts(79, 0, H, I, 4)
    x = synth.activations_bf16(790, T, H)
    ids = np.array([[3, 7, 7, 1], [63, -1, 2, 0], [5, 64, 9, 5], [3, 11, 12, 13], [3, 40, 41, 42],
                    [3, 50, 51, 52]], dtype=np.int32)
    rng = np.random.default_rng(791)
    w = rng.uniform(0.05, 0.5, size=(T, k)).astype(np.float32)
    y, timings = w4.moe_w4a16_forward_timed(bf16_to_dev(x), *routed, top_k=k,
                                            topk_ids=torch.from_numpy(ids).to(DEV), topk_w=torch.from_numpy(w).to(DEV))
    assert "gk_pair_stream" in _names(timings), timings
    keep = np.ones_like(ids, dtype=bool)
    for t in range(T):
        seen = set()
        for j in range(k):
            e = int(ids[t, j])
            if e < 0 or e >= E or e in seen:
                keep[t, j] = False
            else:
                seen.add(e)
    ids_ok = np.where(keep, ids, 0)
    w_ok = np.where(keep, w, 0.0).astype(np.float32)
    y_ref = oracle.moe_ffn(x, ids_ok, w_ok, *ref.as_args(), 4)
    check_ffn(y, y_ref, "pair given ids")


def _tied_logits(seed, T, E):
    """Router logits whose top ranks are full of exact ties: the 12 largest of each token
    take only three distinct values, one token's top values are +0 and -0 among negatives,
    and some logits are -inf."""
    logits = synth.router_logits(seed, T, E)
    for t in range(T):
        top = np.argsort(-logits[t], kind="stable")[:12]
        logits[t, top] = np.array([3.0, 3.0, 3.0, 2.5, 2.5, 2.5, 2.5, 2.5, 1.0, 1.0, 1.0, 1.0],
                                  dtype=np.float32)[np.arange(12) % 12]
    t = T - 1
    logits[t] = -np.abs(logits[t]) - 1.0
    logits[t, [5, 9, 40, 41, 200]] = np.array([0.0, -0.0, 0.0, -0.0, -0.0], dtype=np.float32)
    logits[t, [1, 2]] = -np.inf
    return logits


@pytest.mark.parametrize("T,path", [(1, "tiny_decode"), (2, "tiny_decode"), (4, "gk_pair_stream")])
def test_rank_expert_with_ties(T, path):
    """Each gate/up workgroup runs its pair's top-k only up to the pair's rank; with exact
    ties, signed zeros and -inf among the top ranks the experts it finds (and so y) must
    still be those of the oracle's order (larger logit first, lower index first)."""
    E, H, I, k = 256, 2048, 512, 8
    say(f"rank ties T={T}")
    routed = gpu_layer(81, 0, E, H, I, 4)
    ref = OracleExperts(81, 0, H, I, 4)
    x = synth.activations_bf16(810 + T, T, H)
    logits = _tied_logits(820 + T, T, E)
    (y, r), timings = w4.moe_w4a16_forward_timed(bf16_to_dev(x), *routed, top_k=k,
                                                 router_logits=f32_to_dev(logits), routing_out=True)
    assert path in _names(timings), timings
    ids, w, _, _, _ = oracle.route(logits, k)
    assert np.array_equal(r["ids"].cpu().numpy(), ids)
    y_ref, _ = oracle.moe_layer(x, logits, k, *ref.as_args(), 4)
    check_ffn(y, y_ref, f"rank ties T={T}")
