"""The boundary's failure reporting and ordering, on the GPU, through the C ABI.

* The single-launch path's sticky time-out word: planted from the host (no wait is made
  to time out), it turns every later single-launch output into NaN rows, and
  ``moe_w4a16_workspace_check`` reports it as W4A16_ERR_TIMEOUT and resets the head, after
  which calls are correct again.
* Calls on a side stream (``stream=s`` not the current stream): every tensor the binding
  allocates is ordered before the kernels on ``s``; results match the current-stream ones
  bit for bit on all three launch paths (single launch, streaming decode, prefill).
* Shape mismatches the C ABI cannot see (raw pointers) raise ValueError in the binding
  before anything is enqueued.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_int4_rtn_amd as w4
from gpu_util import DEV, OracleExperts, bf16_to_dev, check_ffn, f32_to_dev, gpu_layer, say

pytestmark = pytest.mark.gpu

ERR_WORD = w4._lib.WORKSPACE_ERROR_OFFSET // 4


def test_planted_timeout_word_poisons_outputs_until_checked():
    E, H, I, k, T = 16, 512, 256, 4, 2   # T * k = 8: the single-launch path
    say("planted time-out word")
    w13, s13, w2, s2 = gpu_layer(41, 0, E, H, I, 4)
    ref = OracleExperts(41, 0, H, I, 4)
    x = synth.activations_bf16(41, T, H)
    logits = synth.router_logits(41, T, E)
    ws = w4.new_workspace(w4.moe_w4a16_workspace_size(T, H, I, E, k), DEV)
    call = w4.MoeCall(bf16_to_dev(x), w13, s13, w2, s2, top_k=k, workspace=ws)
    xd, ld = bf16_to_dev(x), f32_to_dev(logits)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    y_ref, _ = oracle.moe_layer(x, logits, k, *ref.as_args(), 4)

    call(xd, out, router_logits=ld)
    assert not w4.moe_w4a16_workspace_check(ws)          # synchronises; nothing timed out
    check_ffn(out, y_ref, "before")
    good = out.clone()

    ws.view(torch.int32)[ERR_WORD] = 1                     # as a timed-out wait leaves it
    for _ in range(2):
        out.zero_()
        call(xd, out, router_logits=ld)
        torch.cuda.synchronize()
        assert torch.isnan(out.float()).all(), "a set time-out word must give NaN rows"
    assert int(ws.view(torch.int32)[ERR_WORD].item()) == 1

    assert w4.moe_w4a16_workspace_check(ws)               # reported once, head reset
    assert not ws[:w4._lib.WORKSPACE_HEAD_BYTES].any()
    assert not w4.moe_w4a16_workspace_check(ws)
    call(xd, out, router_logits=ld)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), good.view(torch.int16))


@pytest.mark.parametrize("T", [1, 32, 300])
def test_side_stream_matches_current_stream(T):
    E, H, I, k = 64, 512, 256, 8
    say(f"side stream T={T}")
    w13, s13, w2, s2 = gpu_layer(42, 0, E, H, I, 4)
    sh = gpu_layer(42, 0, 1, H, 256, 8, shared=True)
    x = bf16_to_dev(synth.activations_bf16(42 + T, T, H))
    logits = f32_to_dev(synth.router_logits(42 + T, T, E))
    y0, r0 = w4.moe_w4a16_forward(x, w13, s13, w2, s2, top_k=k, router_logits=logits, shared=sh, routing_out=True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream(DEV)
    s.wait_stream(torch.cuda.current_stream(DEV))
    # a long kernel queued on the current stream first: the side stream must not depend on it
    busy = torch.randn((2048, 2048), device=DEV)
    for _ in range(4):
        busy = busy @ busy * 1e-3
    y1, r1 = w4.moe_w4a16_forward(x, w13, s13, w2, s2, top_k=k, router_logits=logits, shared=sh,
                                  routing_out=True, stream=s)
    call = w4.MoeCall(x, w13, s13, w2, s2, top_k=k, shared=sh, stream=s)
    with torch.cuda.stream(s):
        out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    y2 = call(x, out, router_logits=logits)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    assert torch.equal(y0.view(torch.int16), y2.view(torch.int16))
    for name in ("ids", "counts", "offsets", "sorted_pairs"):
        assert torch.equal(r0[name], r1[name]), name


def test_binding_rejects_mismatched_shapes():
    E, H, I, k, T = 8, 256, 128, 2, 4
    say("binding shape checks")
    w13, s13, w2, s2 = gpu_layer(43, 0, E, H, I, 4)
    x = bf16_to_dev(synth.activations_bf16(43, T, H))
    logits = f32_to_dev(synth.router_logits(43, T, E))
    fwd = lambda **kw: w4.moe_w4a16_forward(**{**dict(x=x, w13=w13, s13=s13, w2=w2, s2=s2, top_k=k,   # noqa: E731
                                                      router_logits=logits), **kw})
    torch.cuda.synchronize()
    cases = {
        "8-bit codes for a 4-bit bank": dict(bits=8),
        "short out": dict(out=torch.empty((T - 1, H), dtype=torch.bfloat16, device=DEV)),
        "wide out": dict(out=torch.empty((T, H + 128), dtype=torch.bfloat16, device=DEV)),
        "logits of another E": dict(router_logits=f32_to_dev(synth.router_logits(43, T, E + 1))),
        "ids of another k": dict(router_logits=None, topk_ids=torch.zeros((T, k + 1), dtype=torch.int32, device=DEV),
                                 topk_w=torch.zeros((T, k + 1), device=DEV)),
        "residual of another T": dict(residual=torch.zeros((T + 1, H), dtype=torch.bfloat16, device=DEV)),
        "scales of another I": dict(s2=torch.zeros((E, H, 2), dtype=torch.bfloat16, device=DEV)),
        "small workspace": dict(workspace=torch.zeros((1024,), dtype=torch.uint8, device=DEV)),
        "top_k > E": dict(top_k=E + 1),
    }
    for what, kw in cases.items():
        with pytest.raises(ValueError):
            fwd(**kw)
        say(f"  rejected: {what}")
    bad_shared = gpu_layer(43, 0, 1, H, I, 8, shared=True)
    bad_shared["bits"] = 4     # 8-bit packed tensors declared as 4-bit
    with pytest.raises(ValueError):
        fwd(shared=bad_shared)
    w = torch.zeros((2, 16, 256), device=DEV)
    with pytest.raises(ValueError):
        w4.rtn_quantize_pack(w, 4, packed=torch.empty((2, 16, 16), dtype=torch.int32, device=DEV))
    with pytest.raises(ValueError):
        w4.rtn_quantize_pack(w, 4, scales=torch.empty((2, 16, 1), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError):
        w4.MoeCall(x, w13, s13, w2, s2, top_k=k)(x[:T - 1], torch.empty((T - 1, H), dtype=torch.bfloat16,
                                                                         device=DEV), router_logits=logits)
    torch.cuda.synchronize()
    # nothing above reached a kernel: the stream is idle and a correct call still works
    y = fwd()
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all()


@pytest.mark.parametrize("n_words", [4, 64, 4 * 1000 + 4, 1 << 22])
def test_stream_read_xor(n_words):
    """The measurement aid's fold of every word read (a ragged tail past the 4-vector loop)."""
    import numpy as np
    rng = np.random.default_rng(n_words)
    host = rng.integers(0, 2 ** 32, size=n_words, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to("cuda:0")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    w4.stream_read(buf, sink)
    w4.stream_read(buf, sink)   # twice: the fold cancels
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    w4.stream_read(buf, sink)
    torch.cuda.synchronize()
    assert np.uint32(sink.cpu().numpy().view(np.uint32)[0]) == np.bitwise_xor.reduce(host)


def test_stream_read_argument_rules():
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    with pytest.raises(Exception):
        w4.stream_read(torch.zeros(5, dtype=torch.int32, device="cuda:0"), sink)   # 20 bytes
