"""The single-launch path for tiny batches (T * top_k <= 16, H <= 4096).

Gate/up workgroups hand the intermediate rows to the down workgroups of the same kernel
through the workspace head: each value is written with the epoch of its call, and the
last down workgroup resets the exit counters and advances the epoch (clearing the tagged
values when the epoch wraps).  These tests run many calls with changing shapes and
routing on one workspace, check every output against the oracle, and read the head back.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_int4_rtn_amd as w4
from gpu_util import DEV, OracleExperts, bf16_to_dev, check_ffn, f32_to_dev, gpu_layer, say

pytestmark = pytest.mark.gpu

SYNC_BYTES = 16384                       # counters, one per 128-byte line
HEAD_BYTES = w4._lib.WORKSPACE_HEAD_BYTES  # counters, then the tagged values
GROUP0, TOP, ERROR, EPOCH = 80, 100, 101, 102
EPOCHS = 65535


def _words(ws):
    return ws[:SYNC_BYTES].cpu().numpy().view(np.uint32)[::32]


def _counters_reset(ws):
    """Every exit counter back at zero and no wait timed out."""
    w = _words(ws)
    return not w[GROUP0:ERROR + 1].any()


def _epoch_word(ws):
    return int(_words(ws)[EPOCH])


def _set_epoch_word(ws, v):
    ws[EPOCH * 128:EPOCH * 128 + 4] = torch.from_numpy(np.array([v], dtype=np.uint32).view(np.uint8)).to(ws.device)


def test_tiny_calls_share_one_workspace():
    E, H, I, k = 64, 512, 256, 2
    routed = {b: gpu_layer(31, 0, E, H, I, b) for b in (4, 8)}
    refs = {b: OracleExperts(31, 0, H, I, b) for b in (4, 8)}
    sI = 384   # shared intermediate differs from the routed one: some row blocks are idle
    sh_gpu = gpu_layer(31, 1, 1, H, sI, 8, shared=True)
    sh_ref = OracleExperts(31, 1, H, sI, 8, shared=True)
    need = max(w4.moe_w4a16_workspace_size(T, H, I, E, k, 8, sI) for T in (1, 8))
    ws = w4.new_workspace(need, DEV)
    assert _epoch_word(ws) == 0
    plan = [(1, 4, False), (8, 4, True), (3, 8, False), (1, 8, True), (8, 8, False), (5, 4, True),
            (2, 4, False), (8, 4, False), (1, 4, True), (7, 8, True)]
    for i, (T, bits, with_shared) in enumerate(plan):
        say(f"tiny call {i}: T={T} bits={bits} shared={with_shared}")
        x = synth.activations_bf16(200 + i, T, H)
        res = synth.activations_bf16(300 + i, T, H)
        logits = synth.router_logits(200 + i, T, E)
        y = w4.moe_w4a16_forward(bf16_to_dev(x), *routed[bits], top_k=k, bits=bits,
                                 router_logits=f32_to_dev(logits), shared=sh_gpu if with_shared else None,
                                 residual=bf16_to_dev(res), workspace=ws)
        torch.cuda.synchronize()
        y_ref, _ = oracle.moe_layer(x, logits, k, *refs[bits].as_args(), bits,
                                    shared=sh_ref.shared_dict() if with_shared else None, residual_bits=res)
        check_ffn(y, y_ref, f"call {i}")
        assert _counters_reset(ws), f"counters not reset after call {i}"
        assert _epoch_word(ws) == i + 1, f"epoch not advanced by call {i}"


@pytest.mark.parametrize("H", [4096, 4224])
def test_tiny_boundary_hidden_sizes(H):
    """H = 4096 is the widest hidden size on the single-launch path (256 down
    workgroups); 4224 takes the routing-kernel path.  Both must agree with the oracle."""
    E, I, k, T = 16, 128, 8, 2   # T * k = 16: the largest tiny batch
    say(f"tiny boundary H={H}")
    routed = gpu_layer(32, 0, E, H, I, 4)
    ref = OracleExperts(32, 0, H, I, 4)
    x = synth.activations_bf16(400, T, H)
    logits = synth.router_logits(400, T, E)
    ws = w4.new_workspace(w4.moe_w4a16_workspace_size(T, H, I, E, k), DEV)
    for rep in range(3):
        y = w4.moe_w4a16_forward(bf16_to_dev(x), *routed, top_k=k, router_logits=f32_to_dev(logits), workspace=ws)
        torch.cuda.synchronize()
        y_ref, _ = oracle.moe_layer(x, logits, k, *ref.as_args(), 4)
        check_ffn(y, y_ref, f"H={H} rep {rep}")
    assert _counters_reset(ws)


def test_tiny_given_ids_with_dropped_pairs():
    """Caller-supplied ids: an out-of-range id and a repeat within a token contribute
    nothing; the rest must match the oracle on the remaining pairs."""
    E, H, I, k, T = 16, 256, 128, 4, 3
    say("tiny given ids with dropped pairs")
    routed = gpu_layer(33, 0, E, H, I, 4)
    ref = OracleExperts(33, 0, H, I, 4)
    x = synth.activations_bf16(500, T, H)
    ids = np.array([[3, 7, 7, 1], [15, -1, 2, 0], [5, 16, 9, 5]], dtype=np.int32)
    w = np.array([[0.4, 0.3, 0.2, 0.1], [0.25, 0.25, 0.25, 0.25], [0.1, 0.2, 0.3, 0.4]], dtype=np.float32)
    y = w4.moe_w4a16_forward(bf16_to_dev(x), *routed, top_k=k, topk_ids=torch.from_numpy(ids).to(DEV),
                             topk_w=torch.from_numpy(w).to(DEV))
    torch.cuda.synchronize()
    # the oracle's FFN on the surviving pairs (dropped ones get weight 0 and any valid id)
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
    check_ffn(y, y_ref, "given ids")


def test_tiny_epoch_wrap():
    """Calls across the wrap of the epoch (65535 -> 1): the call at the last epoch clears
    every tagged value, so values left with tag 1 from long ago are never taken as new.
    Words carrying epoch 1 are planted before two one-token calls (which write rows 0-7
    only); the two-token call after the wrap reads rows 8-15 and must not take them."""
    E, H, I, k = 16, 256, 128, 8
    routed = gpu_layer(34, 0, E, H, I, 4)
    ref = OracleExperts(34, 0, H, I, 4)
    ws = w4.new_workspace(w4.moe_w4a16_workspace_size(2, H, I, E, k), DEV)
    # stale values tagged with epoch 1 in every tag word (value bits: bf16 1.0)
    stale = np.full(((HEAD_BYTES - SYNC_BYTES) // 4,), (1 << 16) | 0x3F80, dtype=np.uint32)
    _set_epoch_word(ws, EPOCHS - 3)                 # next calls: epochs 65533, 65534, 65535, 1, 2
    for i, T in enumerate((2, 1, 1, 2, 1)):
        say(f"tiny epoch wrap call {i}: T={T} epoch word {_epoch_word(ws)}")
        if i == 1:
            ws[SYNC_BYTES:HEAD_BYTES] = torch.from_numpy(stale.view(np.uint8)).to(DEV)
        x = synth.activations_bf16(600 + i, T, H)
        logits = synth.router_logits(600 + i, T, E)
        y = w4.moe_w4a16_forward(bf16_to_dev(x), *routed, top_k=k, router_logits=f32_to_dev(logits), workspace=ws)
        torch.cuda.synchronize()
        y_ref, _ = oracle.moe_layer(x, logits, k, *ref.as_args(), 4)
        check_ffn(y, y_ref, f"wrap call {i}")
        assert _counters_reset(ws)
        assert _epoch_word(ws) == (EPOCHS - 3 + i + 1) % EPOCHS
        if i == 2:   # the call at epoch 65535 cleared the tag area on its way out
            assert not ws[SYNC_BYTES:HEAD_BYTES].cpu().numpy().any()
