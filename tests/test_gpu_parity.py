"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bar: packed codes, scales and routing (ids, counts, offsets, sorted pairs) bit-exact;
routing weights within 1e-6; FFN outputs within the acceptance tolerance of
``gpu_util.check_ffn``.  Sizes span several tiles and ragged tails; the full layer
shape (256 experts, top-8, hidden 2048, intermediate 512) runs at 1, 32 and 8192
tokens, the last one checked on every token routed to any of 16 experts.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_int4_rtn_amd as w4
from gpu_util import (DEV, OracleExperts, bf16_from_dev, bf16_to_dev, check_ffn, f32_to_dev, gpu_layer, say)

pytestmark = pytest.mark.gpu

FULL = synth.CONFIGS["decode1"]


# ------------------------------------------------------------------ quantizer

@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(8, 256, 256), (3, 5, 384), (1, 1, 128), (2, 64, 2048)])
def test_quantize_bitexact(bits, dtype, shape):
    say(f"quantize bits={bits} dtype={dtype} shape={shape}")
    rng = np.random.default_rng(hash((bits, dtype, shape)) % 2 ** 32)
    w = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    if dtype == "bf16":
        wb = oracle.bf16_bits_from_f32(w)
        w = oracle.f32_from_bf16_bits(wb)
        dev_w = bf16_to_dev(wb)
    else:
        dev_w = f32_to_dev(w)
    p_ref, s_ref = oracle.quantize_pack(w, bits)
    p, s = w4.rtn_quantize_pack(dev_w, bits)
    torch.cuda.synchronize()
    assert np.array_equal(p.cpu().numpy(), p_ref)
    assert np.array_equal(bf16_from_dev(s), s_ref)


@pytest.mark.parametrize("bits", [4, 8])
def test_quantize_edge_cases_bitexact(bits):
    say(f"quantize edge cases bits={bits}")
    qmax = oracle.QMAX[bits]
    rows = []
    u = 2.0 ** -7
    r = np.zeros(128)
    r[:6] = np.array([qmax, 0.5, 1.5, 2.5, -2.5, 3.5]) * u            # ties
    rows.append(r)
    rows.append(np.zeros(128))                                        # all-zero group
    rng = np.random.default_rng(1)
    g = rng.integers(-qmax, qmax + 1, 128).astype(np.float64)
    g[7] = -qmax
    rows.append(g * 2.0 ** -9)                                        # lossless grid
    rows.append(rng.standard_normal(128) * 1e-30)                     # tiny normals
    rows.append(rng.standard_normal(128) * 3e30)                      # huge values
    r = rng.standard_normal(128) * 0.02
    r[::2] = -r[1::2]                                                 # +-x pairs
    rows.append(r)
    r = np.full(128, -0.0)
    r[3] = 1.0
    rows.append(r)
    w = np.stack(rows).astype(np.float32)
    p_ref, s_ref = oracle.quantize_pack(w, bits)
    p, s = w4.rtn_quantize_pack(f32_to_dev(w), bits)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_from_dev(s), s_ref)
    assert np.array_equal(p.cpu().numpy(), p_ref)


@pytest.fixture(scope="module")
def full_layer():
    say("generating and quantizing the full 256-expert layer on the GPU")
    return gpu_layer(FULL.group, 0, FULL.E, FULL.H, FULL.I, 4)


def test_quantize_full_layer_sampled_experts(full_layer):
    w13, s13, w2, s2 = full_layer
    ref = OracleExperts(FULL.group, 0, FULL.H, FULL.I, 4)
    for e in (0, 1, 77, 128, 200, 255):
        say(f"  expert {e}")
        p13, q13, p2, q2 = ref.get(e)
        assert np.array_equal(w13[e].cpu().numpy(), p13)
        assert np.array_equal(bf16_from_dev(s13[e]), q13)
        assert np.array_equal(w2[e].cpu().numpy(), p2)
        assert np.array_equal(bf16_from_dev(s2[e]), q2)


# -------------------------------------------------------------------- routing

def _run_route(logits, k, E, H=256, I=128):
    """Routing outputs of a forward call on a small zero layer."""
    T = logits.shape[0]
    x = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    w13 = torch.zeros((E, 2 * I, H // 8), dtype=torch.int32, device=DEV)
    s13 = torch.zeros((E, 2 * I, H // 128), dtype=torch.bfloat16, device=DEV)
    w2 = torch.zeros((E, H, I // 8), dtype=torch.int32, device=DEV)
    s2 = torch.zeros((E, H, I // 128), dtype=torch.bfloat16, device=DEV)
    y, r = w4.moe_w4a16_forward(x, w13, s13, w2, s2, top_k=k, router_logits=f32_to_dev(logits), routing_out=True)
    torch.cuda.synchronize()
    return y, {n: t.cpu().numpy() for n, t in r.items()}


@pytest.mark.parametrize("T,E,k", [(4, 8, 2), (1, 256, 8), (32, 256, 8), (64, 256, 8), (65, 256, 8),
                                   (300, 64, 6), (8192, 256, 8), (7, 1024, 16), (5, 3, 3),
                                   # the split routing launch (25..64 tokens): its smallest and
                                   # largest workgroup counts, 8 and 16 logits per lane
                                   (25, 512, 4), (40, 1024, 16), (64, 128, 1)])
def test_route_bitexact(T, E, k):
    say(f"route T={T} E={E} k={k}")
    logits = synth.router_logits(50 + T, T, E)
    if T > 2:   # exact ties inside a token and identical tokens
        logits[0, 1] = logits[0, 2]
        logits[2] = logits[1]
    y, r = _run_route(logits, k, E)
    ids, w, counts, offsets, pairs = oracle.route(logits, k)
    assert np.array_equal(r["ids"], ids)
    assert np.array_equal(r["counts"], counts)
    assert np.array_equal(r["offsets"], offsets)
    assert np.array_equal(r["sorted_pairs"], pairs)
    assert np.abs(r["w"] - w).max() <= 1e-6
    assert np.all(bf16_from_dev(y) == 0)        # zero weights give zero output


@pytest.mark.parametrize("T,E,k", [(1, 256, 8), (8, 256, 8), (33, 256, 8), (200, 256, 8), (6, 512, 8),
                                   (70, 1024, 16), (3, 20, 5)])
def test_route_heavy_ties_bitexact(T, E, k):
    """Logits drawn from a handful of values (including -0.0, +0.0 and -inf), so most
    top-k choices are decided by the lower-index rule."""
    say(f"route heavy ties T={T} E={E} k={k}")
    rng = np.random.default_rng(1000 + T * 7 + E)
    vals = np.array([1.5, 0.75, 0.0, -0.0, -0.5, -np.inf], dtype=np.float32)
    logits = vals[rng.integers(0, len(vals), size=(T, E))]
    logits[0, :k + 3] = 0.0          # the first token: a tie of more than k values
    logits[0, 1] = -0.0
    y, r = _run_route(logits, k, E)
    ids, w, counts, offsets, pairs = oracle.route(logits, k)
    assert np.array_equal(r["ids"], ids)
    assert np.array_equal(r["counts"], counts)
    assert np.array_equal(r["offsets"], offsets)
    assert np.array_equal(r["sorted_pairs"], pairs)
    assert np.abs(r["w"] - w).max() <= 1e-6


@pytest.mark.parametrize("T", [3, 100])
def test_route_from_given_ids(T):
    say(f"route from given ids T={T}")
    E, k, H, I = 16, 4, 256, 128
    rng = np.random.default_rng(T)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ids[0, 3] = ids[0, 1]     # repeated id: the later slot contributes nothing
    ids[1, 2] = E + 5         # out of range: contributes nothing
    wts = rng.random((T, k)).astype(np.float32)
    x = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    w13 = torch.zeros((E, 2 * I, H // 8), dtype=torch.int32, device=DEV)
    s13 = torch.zeros((E, 2 * I, H // 128), dtype=torch.bfloat16, device=DEV)
    w2 = torch.zeros((E, H, I // 8), dtype=torch.int32, device=DEV)
    s2 = torch.zeros((E, H, I // 128), dtype=torch.bfloat16, device=DEV)
    _, r = w4.moe_w4a16_forward(x, w13, s13, w2, s2, top_k=k, topk_ids=torch.from_numpy(ids).to(DEV),
                                topk_w=f32_to_dev(wts), routing_out=True)
    torch.cuda.synchronize()
    valid = ids.copy()
    valid[0, 3] = -1
    valid[1, 2] = -1
    flat = valid.reshape(-1)
    counts = np.bincount(flat[flat >= 0], minlength=E)
    assert np.array_equal(r["counts"].cpu().numpy(), counts)
    assert np.array_equal(r["offsets"].cpu().numpy()[1:], np.cumsum(counts))
    good = np.nonzero(flat >= 0)[0]
    order = good[np.lexsort((good, flat[good]))]
    assert np.array_equal(r["sorted_pairs"].cpu().numpy()[:len(order)], order)


# ------------------------------------------------------------------------ FFN

def _small_layer(E, H, I, bits, group=7, layer=0):
    return gpu_layer(group, layer, E, H, I, bits), OracleExperts(group, layer, H, I, bits)


@pytest.mark.parametrize("bits", [4, 8])
def test_ffn_tiny(bits):
    cfg = synth.CONFIGS["tiny"]
    say(f"ffn tiny bits={bits}")
    (w13, s13, w2, s2), ref = _small_layer(cfg.E, cfg.H, cfg.I, bits, group=cfg.group)
    x = synth.activations_bf16(0, cfg.T, cfg.H)
    logits = synth.router_logits(0, cfg.T, cfg.E)
    y = w4.moe_w4a16_forward(bf16_to_dev(x), w13, s13, w2, s2, top_k=cfg.k, bits=bits, router_logits=f32_to_dev(logits))
    torch.cuda.synchronize()
    y_ref, _ = oracle.moe_layer(x, logits, cfg.k, *ref.as_args(), bits)
    check_ffn(y, y_ref, f"tiny bits={bits}")


@pytest.mark.parametrize("T,E,H,I,k", [(2, 16, 256, 256, 4), (5, 32, 512, 384, 4), (63, 32, 512, 256, 4),
                                       (64, 16, 256, 128, 8), (65, 32, 512, 256, 4), (200, 32, 512, 256, 4),
                                       (513, 8, 384, 256, 2)])
def test_ffn_ragged(T, E, H, I, k):
    say(f"ffn ragged T={T} E={E} H={H} I={I} k={k}")
    (w13, s13, w2, s2), ref = _small_layer(E, H, I, 4, group=11)
    x = synth.activations_bf16(20 + T, T, H)
    logits = synth.router_logits(20 + T, T, E)
    y = w4.moe_w4a16_forward(bf16_to_dev(x), w13, s13, w2, s2, top_k=k, router_logits=f32_to_dev(logits))
    torch.cuda.synchronize()
    y_ref, _ = oracle.moe_layer(x, logits, k, *ref.as_args(), 4)
    check_ffn(y, y_ref, f"T={T}")


@pytest.mark.parametrize("cfg_name", ["decode1", "decode32"])
def test_ffn_full_layer_decode(full_layer, cfg_name):
    cfg = synth.CONFIGS[cfg_name]
    say(f"ffn {cfg_name}")
    w13, s13, w2, s2 = full_layer
    ref = OracleExperts(FULL.group, 0, FULL.H, FULL.I, 4)
    ci = synth.CONFIG_INDEX[cfg_name]
    x = synth.activations_bf16(ci, cfg.T, cfg.H)
    logits = synth.router_logits(ci, cfg.T, cfg.E)
    y, r = w4.moe_w4a16_forward(bf16_to_dev(x), w13, s13, w2, s2, top_k=cfg.k, router_logits=f32_to_dev(logits),
                                routing_out=True)
    torch.cuda.synchronize()
    y_ref, (ids, *_ ) = oracle.moe_layer(x, logits, cfg.k, *ref.as_args(), 4)
    assert np.array_equal(r["ids"].cpu().numpy(), ids)
    check_ffn(y, y_ref, cfg_name)
    y2 = w4.moe_w4a16_forward(bf16_to_dev(x), w13, s13, w2, s2, top_k=cfg.k, router_logits=f32_to_dev(logits))
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "decode result not bitwise reproducible"


def test_ffn_full_layer_prefill_sixteen_experts(full_layer):
    """8192 tokens over the full layer: every output row of every token routed to any of
    16 experts spread over the bank (about 40 % of the tokens), so each of those experts'
    M-tiles, the ragged last one included, is compared in full."""
    cfg = synth.CONFIGS["prefill8192"]
    say("ffn prefill8192 (all tokens of 16 experts)")
    w13, s13, w2, s2 = full_layer
    ref = OracleExperts(FULL.group, 0, FULL.H, FULL.I, 4)
    x = synth.activations_bf16(3, cfg.T, cfg.H)
    logits = synth.router_logits(3, cfg.T, cfg.E)
    y = w4.moe_w4a16_forward(bf16_to_dev(x), w13, s13, w2, s2, top_k=cfg.k, router_logits=f32_to_dev(logits))
    torch.cuda.synchronize()
    ids, wts, counts, *_ = oracle.route(logits, cfg.k)
    chosen = np.arange(0, 256, 17)
    assert len(chosen) == 16 and np.any(counts[chosen] % 128 != 0)
    tokens = np.nonzero(np.isin(ids, chosen).any(axis=1))[0]
    say(f"  {len(tokens)} tokens")
    ref.prefetch(np.unique(ids[tokens]))
    y_ref = oracle.moe_ffn(x, ids, wts, *ref.as_args(), 4, tokens=tokens)
    check_ffn(y[torch.from_numpy(tokens).to(DEV)], y_ref, "prefill8192, 16 experts' tokens")
    y2 = w4.moe_w4a16_forward(bf16_to_dev(x), w13, s13, w2, s2, top_k=cfg.k, router_logits=f32_to_dev(logits))
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "prefill result not bitwise reproducible"


@pytest.mark.parametrize("T", [4, 100])
@pytest.mark.parametrize("routed_bits", [4, 8])
def test_ffn_shared_expert_and_residual(T, routed_bits):
    say(f"ffn shared+residual T={T} routed_bits={routed_bits}")
    E, H, I, k = 32, 512, 256, 4
    (w13, s13, w2, s2), ref = _small_layer(E, H, I, routed_bits, group=13)
    sh_gpu = gpu_layer(13, 0, 1, H, I, 8, shared=True)
    sh_ref = OracleExperts(13, 0, H, I, 8, shared=True)
    x = synth.activations_bf16(30 + T, T, H)
    res = synth.activations_bf16(31 + T, T, H)
    logits = synth.router_logits(30 + T, T, E)
    res_dev = bf16_to_dev(res)
    y = w4.moe_w4a16_forward(bf16_to_dev(x), w13, s13, w2, s2, top_k=k, bits=routed_bits,
                             router_logits=f32_to_dev(logits), shared=sh_gpu, residual=res_dev)
    torch.cuda.synchronize()
    y_ref, _ = oracle.moe_layer(x, logits, k, *ref.as_args(), routed_bits, shared=sh_ref.shared_dict(),
                                residual_bits=res)
    check_ffn(y, y_ref, f"shared T={T}")
    # in place: y aliases the residual
    y2 = w4.moe_w4a16_forward(bf16_to_dev(x), w13, s13, w2, s2, top_k=k, bits=routed_bits,
                              router_logits=f32_to_dev(logits), shared=sh_gpu, residual=res_dev, out=res_dev)
    torch.cuda.synchronize()
    check_ffn(y2, y_ref, f"shared in-place T={T}")


def test_ffn_given_ids_matches_logits_path():
    say("ffn given ids == logits path")
    E, H, I, k, T = 16, 256, 256, 4, 9
    (w13, s13, w2, s2), ref = _small_layer(E, H, I, 4, group=17)
    x = bf16_to_dev(synth.activations_bf16(40, T, H))
    logits = f32_to_dev(synth.router_logits(40, T, E))
    y1, r = w4.moe_w4a16_forward(x, w13, s13, w2, s2, top_k=k, router_logits=logits, routing_out=True)
    y2 = w4.moe_w4a16_forward(x, w13, s13, w2, s2, top_k=k, topk_ids=r["ids"], topk_w=r["w"])
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_output_guard_bands_untouched(full_layer):
    say("guard bands")
    w13, s13, w2, s2 = full_layer
    for T in (1, 32, 300):
        x = bf16_to_dev(synth.activations_bf16(60, T, FULL.H))
        logits = f32_to_dev(synth.router_logits(60, T, FULL.E))
        pad = 4096
        buf = torch.full((T * FULL.H + 2 * pad,), 0x5A5A, dtype=torch.int16, device=DEV)
        out = buf[pad:pad + T * FULL.H].view(T, FULL.H).view(torch.bfloat16)
        w4.moe_w4a16_forward(x, w13, s13, w2, s2, top_k=8, router_logits=logits, out=out)
        torch.cuda.synchronize()
        assert torch.all(buf[:pad] == 0x5A5A) and torch.all(buf[-pad:] == 0x5A5A)
        assert not torch.any(buf[pad:-pad] == 0x5A5A)


def test_zero_tokens():
    E, H, I = 8, 256, 128
    x = torch.zeros((0, H), dtype=torch.bfloat16, device=DEV)
    w13 = torch.zeros((E, 2 * I, H // 8), dtype=torch.int32, device=DEV)
    s13 = torch.zeros((E, 2 * I, H // 128), dtype=torch.bfloat16, device=DEV)
    w2 = torch.zeros((E, H, I // 8), dtype=torch.int32, device=DEV)
    s2 = torch.zeros((E, H, I // 128), dtype=torch.bfloat16, device=DEV)
    y = w4.moe_w4a16_forward(x, w13, s13, w2, s2, top_k=2, router_logits=torch.zeros((0, E), device=DEV))
    torch.cuda.synchronize()
    assert y.shape == (0, H)
