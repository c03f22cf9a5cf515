"""The allocation-free entry point ``moe_w4a16_forward_noalloc`` (static per-GPU scratch),
called through the C ABI, against ``moe_w4a16_forward`` on the same inputs: two calls in a
row on the one shared array, the second with a smaller input, then shapes beyond the
array's size rejected on the host.  Outputs are held to the FFN acceptance tolerance
against the caller-workspace entry point, and must match it bit for bit where both take
the same kernels (T * top_k > 16).
"""

import ctypes as C

import pytest
import torch

import synth
import weight_only_int4_rtn_amd as w4
from weight_only_int4_rtn_amd import _lib
from gpu_util import DEV, bf16_to_dev, check_ffn, f32_to_dev, gpu_layer, say

pytestmark = pytest.mark.gpu


def _noalloc(x, layer, k, logits, shared=None, residual=None):
    """One call of moe_w4a16_forward_noalloc: the caller allocates the output beforehand;
    no workspace is passed."""
    w13, s13, w2, s2 = layer
    T, H = x.shape
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    torch.cuda.synchronize()
    a = w4._args(x, w13, s13, w2, s2, k, 4, logits, None, None, shared, residual, out, None, None, None, None)
    st = _lib.lib().moe_w4a16_forward_noalloc(C.byref(a), C.c_void_p(torch.cuda.current_stream(DEV).cuda_stream))
    _lib.check(st, "moe_w4a16_forward_noalloc")
    return out


def test_noalloc_matches_workspace_entry_point_twice_then_smaller():
    E, H, I, k = 64, 512, 256, 8
    layer = gpu_layer(51, 0, E, H, I, 4)
    sh = gpu_layer(51, 0, 1, H, 256, 8, shared=True)
    # first a prefill-sized call (the larger layout), then a decode-sized one in the same array,
    # then a single token (which the caller-workspace entry point runs as one launch)
    for i, T in enumerate((300, 24, 1)):
        say(f"noalloc call {i}: T={T}")
        x = bf16_to_dev(synth.activations_bf16(51 + T, T, H))
        res = bf16_to_dev(synth.activations_bf16(52 + T, T, H))
        logits = f32_to_dev(synth.router_logits(51 + T, T, E))
        y_ref = w4.moe_w4a16_forward(x, *layer, top_k=k, router_logits=logits, shared=sh, residual=res)
        y = _noalloc(x, layer, k, logits, shared=sh, residual=res)
        torch.cuda.synchronize()
        ref64 = y_ref.double().cpu().numpy()
        check_ffn(y, ref64, f"noalloc T={T} vs workspace entry point")
        if T * k > 16:
            assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), f"T={T}: not bitwise equal"


def test_noalloc_rejects_shapes_beyond_the_scratch():
    E, H, I, k, T = 256, 2048, 512, 8, 8192   # about 356 MiB of workspace
    assert w4.moe_w4a16_workspace_size(T, H, I, E, k) > _lib.NOALLOC_SCRATCH_BYTES
    a = _lib.MoeArgs()
    a.T, a.H, a.I, a.E, a.top_k, a.bits, a.group = T, H, I, E, k, 4, 128
    for i, f in enumerate(("x", "router_logits", "w13", "s13", "w2", "s2", "y")):
        setattr(a, f, 0x100000 + 0x1000 * i)   # never dereferenced: rejected on the host
    assert _lib.lib().moe_w4a16_forward_noalloc(C.byref(a), None) == _lib.W4A16_ERR_UNSUPPORTED
    assert "scratch" in _lib.last_error()
