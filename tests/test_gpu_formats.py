"""GPU parity of the FP8 E4M3 per-channel and MXFP4 expert formats, through the C ABI.

Bar: codes and scales of fp8_quantize_pack / mxfp4_quantize_pack (both exponent choices)
bit-exact against the oracle, including rounding ties, zero rows and blocks and lossless
grids; the MoE forward with routed experts in either format within the FFN tolerance of
``gpu_util.check_ffn`` against the oracle's own quantization of the same seeded weights,
on the decode path (1 and 32 tokens of the full 256-expert layer, with and without a
shared expert, the router and the residual) and the prefill grouped GEMM (ragged tiles,
workgroups walking several items).
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_int4_rtn_amd as w4
from oracle import formats as FM
from gpu_util import DEV, bf16_to_dev, check_ffn, f32_to_dev, gpu_layer, say

pytestmark = pytest.mark.gpu

BITS = {"fp8": 8, "mxfp4": 4}


def _gpu_quant(fmt, w_dev, method="mse"):
    if fmt == "fp8":
        return w4.fp8_quantize_pack(w_dev)
    return w4.mxfp4_quantize_pack(w_dev, method)


def _ref_quant(fmt, w, method="mse"):
    if fmt == "fp8":
        return FM.fp8_quantize_pack(w)
    return FM.mxfp4_quantize_pack(w, method)


def _as_np(t):
    return t.cpu().numpy()


# ------------------------------------------------------------------ quantizers

@pytest.mark.parametrize("fmt,method", [("fp8", None), ("mxfp4", "mse"), ("mxfp4", "rtn")])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(8, 256, 256), (3, 5, 384), (1, 1, 128), (2, 64, 2048)])
def test_format_quantizers_bitexact(fmt, method, dtype, shape):
    say(f"quantize {fmt} {method} {dtype} {shape}")
    rng = np.random.default_rng(hash((fmt, method, dtype, shape)) % 2 ** 32)
    w = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    if dtype == "bf16":
        wb = oracle.bf16_bits_from_f32(w)
        w = oracle.f32_from_bf16_bits(wb)
        dev_w = bf16_to_dev(wb)
    else:
        dev_w = f32_to_dev(w)
    p, s = _gpu_quant(fmt, dev_w, method)
    torch.cuda.synchronize()
    p_ref, s_ref = _ref_quant(fmt, w, method)
    assert np.array_equal(_as_np(s), s_ref)
    assert np.array_equal(_as_np(p), p_ref)


def test_fp8_quantizer_edge_rows_bitexact():
    say("fp8 edge rows")
    grid = FM.e4m3_decode(np.arange(0, 127)).astype(np.float64)
    mids = (grid[:-1] + grid[1:]) / 2
    rows = []
    r = np.zeros(256)
    r[0] = 448.0                         # scale exactly 1: every value is its own ratio
    r[1:1 + len(mids[:200])] = mids[:200]   # ties between neighbouring E4M3 values
    rows.append(r)
    r = np.zeros(256)
    r[0] = -448.0
    r[1:1 + len(mids[200:])] = -mids[200:]
    rows.append(r)
    rows.append(np.zeros(256))                                   # all-zero channel
    rng = np.random.default_rng(11)
    rows.append(rng.standard_normal(256) * 1e-30)                # tiny
    rows.append(rng.standard_normal(256) * 3e30)                 # huge
    r = np.full(256, -0.0)
    r[5] = 2.0
    rows.append(r)                                               # signed zeros
    w = np.stack(rows).astype(np.float32)
    p, s = w4.fp8_quantize_pack(f32_to_dev(w))
    torch.cuda.synchronize()
    p_ref, s_ref = FM.fp8_quantize_pack(w)
    assert np.array_equal(_as_np(s), s_ref)
    assert np.array_equal(_as_np(p), p_ref)


@pytest.mark.parametrize("method", ["mse", "rtn"])
def test_mxfp4_quantizer_edge_blocks_bitexact(method):
    say(f"mxfp4 edge blocks {method}")
    rng = np.random.default_rng(12)
    blocks = []
    g = FM.E2M1_VALUES[rng.integers(0, 8, 32)] * np.where(rng.random(32) < 0.5, -1, 1)
    g[:2] = [6, -6]
    blocks.append(g * 2.0 ** -7)                                 # lossless grid
    blocks.append(np.zeros(32))                                  # zero block
    blocks.append(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4) * 2.0 ** -3)   # ties
    t = rng.standard_normal(32) * 0.01
    t[3] = 0.5                                                   # one outlier: clipping vs resolution
    blocks.append(t)
    t = np.full(32, 0.02)
    t[0] = -0.0
    blocks.append(t)                                             # equal magnitudes, a signed zero
    blocks.append(rng.standard_t(2, 32) * 0.01)                  # heavy tails
    blocks.append(rng.standard_normal(32) * 1e-20)
    w = np.concatenate(blocks)[None, :].astype(np.float32)       # one row of 7 blocks, padded to 256
    w = np.concatenate([w, np.zeros((1, 256 - w.shape[1]), np.float32)], axis=1)
    p, s = w4.mxfp4_quantize_pack(f32_to_dev(w), method)
    torch.cuda.synchronize()
    p_ref, s_ref = FM.mxfp4_quantize_pack(w, method)
    assert np.array_equal(_as_np(s), s_ref)
    assert np.array_equal(_as_np(p), p_ref)


# --------------------------------------------------------------------- FFN

class FmtExperts:
    """The oracle's own packed experts in format `fmt`, from the seeds, on demand."""

    def __init__(self, fmt, group, layer, H, I):
        self.fmt, self.args, self.cache = fmt, (group, layer, H, I), {}

    def get(self, e):
        if e not in self.cache:
            group, layer, H, I = self.args
            self.cache[e] = (*_ref_quant(self.fmt, synth.expert_w13(group, layer, e, H, I)),
                             *_ref_quant(self.fmt, synth.expert_w2(group, layer, e, H, I)))
        return self.cache[e]

    def prefetch(self, experts):
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(8) as ex:
            list(ex.map(self.get, [int(e) for e in experts if int(e) not in self.cache]))

    def as_args(self):
        parent = self

        class _V:
            def __init__(self, i):
                self.i = i

            def __getitem__(self, e):
                return parent.get(int(e))[self.i]
        return _V(0), _V(1), _V(2), _V(3)


def fmt_layer(fmt, group, layer, E, H, I):
    """All experts of a layer from the seeds, quantized on the GPU by the library."""
    bits = BITS[fmt]
    w13 = torch.empty((E, 2 * I, H * bits // 32), dtype=torch.int32, device=DEV)
    w2 = torch.empty((E, H, I * bits // 32), dtype=torch.int32, device=DEV)
    if fmt == "fp8":
        s13 = torch.empty((E, 2 * I), dtype=torch.float32, device=DEV)
        s2 = torch.empty((E, H), dtype=torch.float32, device=DEV)
    else:
        s13 = torch.empty((E, 2 * I, H // 32), dtype=torch.uint8, device=DEV)
        s2 = torch.empty((E, H, I // 32), dtype=torch.uint8, device=DEV)
    for e0 in range(0, E, 16):
        es = range(e0, min(E, e0 + 16))
        f13 = f32_to_dev(np.stack([synth.expert_w13(group, layer, e, H, I) for e in es]))
        f2 = f32_to_dev(np.stack([synth.expert_w2(group, layer, e, H, I) for e in es]))
        sl = slice(e0, e0 + len(es))
        if fmt == "fp8":
            w4.fp8_quantize_pack(f13, packed=w13[sl], scales=s13[sl])
            w4.fp8_quantize_pack(f2, packed=w2[sl], scales=s2[sl])
        else:
            w4.mxfp4_quantize_pack(f13, "mse", packed=w13[sl], scales=s13[sl])
            w4.mxfp4_quantize_pack(f2, "mse", packed=w2[sl], scales=s2[sl])
    torch.cuda.synchronize()
    return w13, s13, w2, s2


@pytest.fixture(scope="module", params=["fp8", "mxfp4"])
def full_fmt_layer(request):
    fmt = request.param
    say(f"full 256-expert layer in {fmt}")
    return fmt, fmt_layer(fmt, 1, 0, 256, 2048, 512)


def test_full_layer_quantized_experts_match(full_fmt_layer):
    fmt, (w13, s13, w2, s2) = full_fmt_layer
    ref = FmtExperts(fmt, 1, 0, 2048, 512)
    for e in (0, 131, 255):
        p13, q13, p2, q2 = ref.get(e)
        assert np.array_equal(_as_np(w13[e]), p13) and np.array_equal(_as_np(s13[e]), q13)
        assert np.array_equal(_as_np(w2[e]), p2) and np.array_equal(_as_np(s2[e]), q2)


@pytest.mark.parametrize("T", [1, 32])
@pytest.mark.parametrize("with_shared", [False, True])
def test_full_layer_decode(full_fmt_layer, T, with_shared):
    fmt, layer = full_fmt_layer
    say(f"{fmt} decode T={T} shared={with_shared}")
    ref = FmtExperts(fmt, 1, 0, 2048, 512)
    x = synth.activations_bf16(500 + T, T, 2048)
    logits = synth.router_logits(500 + T, T, 256)
    res = synth.activations_bf16(501 + T, T, 2048)
    kw = {}
    sh_ref = None
    if with_shared:
        kw = dict(shared=gpu_layer(5, 0, 1, 2048, 512, 8, shared=True), residual=bf16_to_dev(res))
        from gpu_util import OracleExperts
        sh_ref = OracleExperts(5, 0, 2048, 512, 8, shared=True).shared_dict()
    y, r = w4.moe_w4a16_forward(bf16_to_dev(x), *layer, top_k=8, bits=BITS[fmt], weight_format=fmt,
                                router_logits=f32_to_dev(logits), routing_out=True, **kw)
    torch.cuda.synchronize()
    ids, wts, *_ = oracle.route(logits, 8)
    assert np.array_equal(_as_np(r["ids"]), ids)
    ref.prefetch(np.unique(ids))
    y_ref = oracle.moe_ffn(x, ids, wts, *ref.as_args(), BITS[fmt], weight_format=fmt, shared=sh_ref,
                           residual_bits=res if with_shared else None)
    check_ffn(y, y_ref, f"{fmt} T={T} shared={with_shared}")


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("T,E,H,I,k", [(4, 8, 256, 128, 2), (65, 16, 512, 256, 4), (300, 32, 512, 256, 4),
                                       (2048, 32, 1024, 512, 8)])
def test_ffn_shapes(fmt, T, E, H, I, k):
    """Tiny layer, the first prefill batch size, ragged tiles, and a batch whose prefill
    workgroups walk several items; with an INT8 shared expert, its gate and the router."""
    say(f"{fmt} ffn T={T} E={E} H={H} I={I} k={k}")
    group = 70 + T % 7
    layer = fmt_layer(fmt, group, 0, E, H, I)
    ref = FmtExperts(fmt, group, 0, H, I)
    sh = gpu_layer(group, 0, 1, H, I, 8, shared=True)
    from gpu_util import OracleExperts
    sh_ref = OracleExperts(group, 0, H, I, 8, shared=True).shared_dict()
    x = synth.activations_bf16(600 + T, T, H)
    res = synth.activations_bf16(601 + T, T, H)
    wr = synth.router_weight_bf16(group, 0, E, H)
    wg = synth.shared_gate_weight_bf16(group, 0, H)
    y, r = w4.moe_w4a16_forward(bf16_to_dev(x), *layer, top_k=k, bits=BITS[fmt], weight_format=fmt,
                                router_w=bf16_to_dev(wr), shared=sh, shared_gate_w=bf16_to_dev(wg),
                                residual=bf16_to_dev(res), routing_out=True)
    torch.cuda.synchronize()
    ids, wts = _as_np(r["ids"]), _as_np(r["w"])
    assert np.array_equal(ids, oracle.route(_as_np(r["logits"]), k)[0])
    y_ref = oracle.moe_ffn(x, ids, wts, *ref.as_args(), BITS[fmt], weight_format=fmt, shared=sh_ref,
                           residual_bits=res, shared_gate=oracle.shared_gate(x, wg))
    check_ffn(y, y_ref, f"{fmt} T={T}")
    # without the residual and shared expert, so the routed experts alone are compared
    y0 = w4.moe_w4a16_forward(bf16_to_dev(x), *layer, top_k=k, bits=BITS[fmt], weight_format=fmt,
                              topk_ids=r["ids"], topk_w=r["w"])
    torch.cuda.synchronize()
    y0_ref = oracle.moe_ffn(x, ids, wts, *ref.as_args(), BITS[fmt], weight_format=fmt)
    check_ffn(y0, y0_ref, f"{fmt} T={T} routed only")


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("T,shared_bits", [(1, 0), (2, 4), (2, 8)])
def test_single_launch_formats(fmt, T, shared_bits):
    """One- and two-token layers of the float formats take the single-launch kernel (routing,
    gate/up and down in one launch), with or without an INT shared expert; three calls in a
    row on one workspace (the launch epoch advances between them)."""
    from gpu_util import OracleExperts
    E, H, I, k = 64, 1024, 256, 8
    layer = fmt_layer(fmt, 81, 0, E, H, I)
    ref = FmtExperts(fmt, 81, 0, H, I)
    kw, sh_ref, sI = {}, None, 0
    if shared_bits:
        sI = 512
        kw = dict(shared=gpu_layer(81, 0, 1, H, sI, shared_bits, shared=True))
        sh_ref = OracleExperts(81, 0, H, sI, shared_bits, shared=True).shared_dict()
    say(f"{fmt} single launch T={T} shared={shared_bits}")
    ws = w4.new_workspace(w4.moe_w4a16_workspace_size(T, H, I, E, k, shared_bits, sI), DEV)
    for it in range(3):
        x = synth.activations_bf16(700 + 10 * T + it, T, H)
        logits = synth.router_logits(700 + 10 * T + it, T, E)
        y, tk = w4.moe_w4a16_forward_timed(bf16_to_dev(x), *layer, top_k=k, bits=BITS[fmt], weight_format=fmt,
                                           router_logits=f32_to_dev(logits), workspace=ws, **kw)
        assert [nm for nm, _ in tk] == ["tiny_decode"], tk
        ids, wts, *_ = oracle.route(logits, k)
        ref.prefetch(np.unique(ids))
        y_ref = oracle.moe_ffn(x, ids, wts, *ref.as_args(), BITS[fmt], weight_format=fmt, shared=sh_ref)
        check_ffn(y, y_ref, f"{fmt} single launch T={T} shared={shared_bits} call {it}")


@pytest.fixture(scope="module", params=["fp8", "mxfp4"])
def stream_fmt_layer(request):
    fmt = request.param
    return fmt, fmt_layer(fmt, 83, 0, 64, 2048, 256), FmtExperts(fmt, 83, 0, 2048, 256)


@pytest.mark.parametrize("T,shared_bits", [(3, 8), (4, 0), (8, 0), (16, 4), (24, 4), (40, 8), (64, 0), (64, 8)])
def test_stream_formats(stream_fmt_layer, T, shared_bits):
    """Small batches of the float formats on the streaming kernels: pair mode (3, 4 tokens of
    64 experts), routing fused into the gate/up kernel (8..24) and routing in its own launch
    (40, 64), with or without an INT shared expert; two calls on one workspace."""
    from gpu_util import OracleExperts
    fmt, layer, ref = stream_fmt_layer
    E, H, I, k = 64, 2048, 256, 8
    kw, sh_ref, sI = {}, None, 0
    if shared_bits:
        sI = 512
        kw = dict(shared=gpu_layer(83, 0, 1, H, sI, shared_bits, shared=True))
        sh_ref = OracleExperts(83, 0, H, sI, shared_bits, shared=True).shared_dict()
    say(f"{fmt} stream T={T} shared={shared_bits}")
    ws = w4.new_workspace(w4.moe_w4a16_workspace_size(T, H, I, E, k, shared_bits, sI), DEV)
    for it in range(2):
        x = synth.activations_bf16(800 + 10 * T + it, T, H)
        logits = synth.router_logits(800 + 10 * T + it, T, E)
        y, tk = w4.moe_w4a16_forward_timed(bf16_to_dev(x), *layer, top_k=k, bits=BITS[fmt], weight_format=fmt,
                                           router_logits=f32_to_dev(logits), workspace=ws, **kw)
        names = [nm for nm, _ in tk]
        assert ("gk_stream" in names or "gk_pair_stream" in names) and "dk_stream" in names, names
        ids, wts, *_ = oracle.route(logits, k)
        ref.prefetch(np.unique(ids))
        y_ref = oracle.moe_ffn(x, ids, wts, *ref.as_args(), BITS[fmt], weight_format=fmt, shared=sh_ref)
        check_ffn(y, y_ref, f"{fmt} stream T={T} shared={shared_bits} call {it}")


def test_full_layer_prefill_sampled(full_fmt_layer):
    """The 8192-token step over the full 256-expert layer in each float format.  The first
    1024 tokens route only among every fourth expert (their other logits are -inf); the
    other tokens route freely, so all experts are active and every one of those 64 experts'
    M-tiles mixes compared and uncompared rows.  Every output row of the 1024 tokens is
    compared, against the oracle quantizing just those 64 experts."""
    fmt, layer = full_fmt_layer
    T, E, k, H, I = 8192, 256, 8, 2048, 512
    say(f"{fmt} prefill 8192 sampled")
    x = synth.activations_bf16(520, T, H)
    logits = synth.router_logits(520, T, E)
    subset = np.arange(0, E, 4)
    n_cmp = 1024
    logits[:n_cmp, np.setdiff1d(np.arange(E), subset)] = -np.inf
    y, tk = w4.moe_w4a16_forward_timed(bf16_to_dev(x), *layer, top_k=k, bits=BITS[fmt], weight_format=fmt,
                                       router_logits=f32_to_dev(logits))
    assert "gk_prefill" in [n for n, _ in tk], tk
    ids, wts, counts, *_ = oracle.route(logits, k)
    assert np.all(counts > 0) and np.all(np.isin(ids[:n_cmp], subset))
    assert np.any(counts[subset] % 128 != 0)   # ragged last tiles among the compared experts
    tokens = np.arange(n_cmp)
    ref = FmtExperts(fmt, 1, 0, H, I)
    ref.prefetch(np.unique(ids[tokens]))
    y_ref = oracle.moe_ffn(x, ids, wts, *ref.as_args(), BITS[fmt], weight_format=fmt, tokens=tokens)
    check_ffn(y[:n_cmp], y_ref, f"{fmt} prefill 8192, {n_cmp} tokens")
