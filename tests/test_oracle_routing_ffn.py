"""Pins for the oracle's routing and expert MLP (CPU only).

Routing is pinned by brute-force Python sorting, by SciPy's softmax and by
invariants; the MLP by ``torch.nn.functional`` on a one-expert layer, by a
dense mixture over every expert that involves no routing permutation, and by
invariants (zero input, linear scaling, batch and permutation behaviour).
"""

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
import synth


# ------------------------------------------------------------------ routing

def _brute_route(logits, k):
    T, E = logits.shape
    ids = [sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k] for t in range(T)]
    pairs = sorted(range(T * k), key=lambda p: (ids[p // k][p % k], p // k))
    return np.array(ids), np.array(pairs)


@pytest.mark.parametrize("T,E,k", [(1, 256, 8), (5, 8, 2), (32, 64, 8), (7, 16, 16)])
def test_route_against_brute_force(T, E, k):
    logits = synth.router_logits(99, T, E)
    if T > 1:   # plant exact ties between experts of one token and across tokens
        logits[0, 3] = logits[0, 5]
        logits[1, :] = logits[0, :]
    ids, w, counts, offsets, pairs = oracle.route(logits, k)
    bids, bpairs = _brute_route(logits, k)
    assert np.array_equal(ids, bids)
    assert np.array_equal(pairs, bpairs)
    assert np.array_equal(counts, np.bincount(bids.ravel(), minlength=E))
    assert offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(np.diff(offsets), counts)
    # weights: softmax of the chosen logits, summing to one, non-increasing
    sel = np.take_along_axis(logits.astype(np.float64), ids, 1)
    assert np.allclose(w, scipy.special.softmax(sel, axis=1), rtol=0, atol=1e-7)
    assert np.allclose(w.astype(np.float64).sum(1), 1.0, atol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_route_tie_goes_to_lower_index():
    logits = np.zeros((2, 6), np.float32)
    logits[0, [1, 4]] = 2.0
    logits[1, :] = -0.0
    logits[1, 5] = 0.0
    ids, w, *_ = oracle.route(logits, 3)
    assert list(ids[0]) == [1, 4, 0]
    assert list(ids[1]) == [0, 1, 2]          # -0.0 and 0.0 compare equal
    assert np.allclose(w[1], 1 / 3)


def test_route_full_and_single():
    logits = synth.router_logits(98, 6, 32)
    ids, w, *_ = oracle.route(logits, 32)
    full = scipy.special.softmax(logits.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(full, ids, 1), atol=1e-7)
    ids1, w1, *_ = oracle.route(logits, 1)
    assert np.all(w1 == 1.0) and np.array_equal(ids1[:, 0], logits.argmax(1))


def test_route_prefill_distribution():
    """8192 tokens, top-8 of 256: every expert gets about 256 +- 16 tokens."""
    logits = synth.router_logits(3, 8192, 256)
    _, _, counts, _, _ = oracle.route(logits, 8)
    assert counts.sum() == 65536 and counts.min() > 150 and counts.max() < 360


# ---------------------------------------------------------------- expert MLP

def _tiny_layer(E=8, H=256, I=128, bits=4, seed_group=0):
    w13 = np.stack([synth.expert_w13(seed_group, 0, e, H, I) for e in range(E)])
    w2 = np.stack([synth.expert_w2(seed_group, 0, e, H, I) for e in range(E)])
    p13, s13 = oracle.quantize_pack(w13, bits)
    p2, s2 = oracle.quantize_pack(w2, bits)
    return p13, s13, p2, s2


@pytest.mark.parametrize("bits", [4, 8])
def test_single_expert_matches_torch_functional(bits):
    """E = 1, k = 1 is a dense gated MLP on the dequantized weights."""
    p13, s13, p2, s2 = _tiny_layer(E=1, bits=bits)
    x_bits = synth.activations_bf16(0, 4, 256)
    ids = np.zeros((4, 1), np.int32)
    w = np.ones((4, 1), np.float32)
    y = oracle.moe_ffn(x_bits, ids, w, p13, s13, p2, s2, bits)
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).double()
    W13 = torch.from_numpy(oracle.dequantize(p13[0], s13[0], bits)).double()
    W2 = torch.from_numpy(oracle.dequantize(p2[0], s2[0], bits)).double()
    gate, up = W13[:128], W13[128:]
    ref = F.linear(F.silu(F.linear(x, gate)) * F.linear(x, up), W2)
    assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_dense_mixture_identity():
    """Tiny layer: the routed sum equals a dense sum over all experts with
    weight w if chosen and 0 otherwise (no permutation code involved)."""
    cfg = synth.CONFIGS["tiny"]
    p13, s13, p2, s2 = _tiny_layer()
    x_bits = synth.activations_bf16(0, cfg.T, cfg.H)
    logits = synth.router_logits(0, cfg.T, cfg.E)
    y, (ids, w, *_) = oracle.moe_layer(x_bits, logits, cfg.k, p13, s13, p2, s2, 4)
    x = oracle.f32_from_bf16_bits(x_bits).astype(np.float64)
    dense = np.zeros_like(y)
    for t in range(cfg.T):
        for e in range(cfg.E):
            gate = float(w[t][list(ids[t]).index(e)]) if e in ids[t] else 0.0
            W13 = oracle.dequantize(p13[e], s13[e], 4).astype(np.float64)
            W2 = oracle.dequantize(p2[e], s2[e], 4).astype(np.float64)
            dense[t] += gate * oracle.expert_ffn(x[t], W13, W2)
    assert np.allclose(y, dense, rtol=1e-12, atol=1e-14)


def test_ffn_invariants():
    cfg = synth.CONFIGS["tiny"]
    p13, s13, p2, s2 = _tiny_layer()
    x_bits = synth.activations_bf16(0, cfg.T, cfg.H)
    logits = synth.router_logits(0, cfg.T, cfg.E)
    ids, w, *_ = oracle.route(logits, cfg.k)
    y = oracle.moe_ffn(x_bits, ids, w, p13, s13, p2, s2, 4)
    # zero input -> exactly zero output
    assert np.all(oracle.moe_ffn(np.zeros_like(x_bits), ids, w, p13, s13, p2, s2, 4) == 0)
    # all-zero down scales -> zero output; doubled down scales -> doubled output
    assert np.all(oracle.moe_ffn(x_bits, ids, w, p13, s13, p2, np.zeros_like(s2), 4) == 0)
    s2x2 = oracle.bf16_bits_from_f32(2 * oracle.f32_from_bf16_bits(s2))
    assert np.allclose(oracle.moe_ffn(x_bits, ids, w, p13, s13, p2, s2x2, 4), 2 * y, rtol=1e-12, atol=0)
    # batch invariance: a token alone gives the same row (up to the fp64 summation order
    # of a matrix product against a vector product)
    for t in range(cfg.T):
        yt = oracle.moe_ffn(x_bits[t:t + 1], ids[t:t + 1], w[t:t + 1], p13, s13, p2, s2, 4)
        assert np.allclose(yt[0], y[t], rtol=1e-12, atol=1e-15)
    # token permutation equivariance, and the token-subset argument
    perm = np.array([2, 0, 3, 1])
    yp = oracle.moe_ffn(x_bits[perm], ids[perm], w[perm], p13, s13, p2, s2, 4)
    assert np.allclose(yp, y[perm], rtol=1e-12, atol=1e-15)
    ys = oracle.moe_ffn(x_bits, ids, w, p13, s13, p2, s2, 4, tokens=[3, 1])
    assert np.allclose(ys, y[[3, 1]], rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("shared_bits", [4, 8])
def test_shared_expert_and_residual_against_torch_functional(shared_bits):
    """The shared expert (weight 1) and the bf16 residual, pinned by an independent
    evaluation: torch.nn.functional's linear and silu in fp64 on the dequantized shared
    weights, the routed experts as a dense mixture over every expert (no routing code),
    and the residual widened by torch's own bf16 -> fp64 conversion."""
    cfg = synth.CONFIGS["tiny"]
    H, I = cfg.H, cfg.I
    p13, s13, p2, s2 = _tiny_layer()
    sp13, ss13 = oracle.quantize_pack(synth.expert_w13(0, 0, 0, H, I, shared=True), shared_bits)
    sp2, ss2 = oracle.quantize_pack(synth.expert_w2(0, 0, 0, H, I, shared=True), shared_bits)
    shared = dict(w13=sp13, s13=ss13, w2=sp2, s2=ss2, bits=shared_bits)
    x_bits = synth.activations_bf16(0, cfg.T, H)
    res_bits = synth.activations_bf16(0, cfg.T, H, stream=12)
    ids, w, *_ = oracle.route(synth.router_logits(0, cfg.T, cfg.E), cfg.k)
    ys = oracle.moe_ffn(x_bits, ids, w, p13, s13, p2, s2, 4, shared=shared, residual_bits=res_bits)

    def as_torch_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double()

    def mlp(x, W13, W2):
        W13 = torch.from_numpy(W13).double()
        W2 = torch.from_numpy(W2).double()
        return F.linear(F.silu(F.linear(x, W13[:I])) * F.linear(x, W13[I:]), W2)

    x = as_torch_bf16(x_bits)
    ref = torch.zeros((cfg.T, H), dtype=torch.float64)
    for e in range(cfg.E):   # dense mixture: weight of e for each token, 0 when not chosen
        ge = torch.zeros(cfg.T, dtype=torch.float64)
        for t in range(cfg.T):
            hit = np.nonzero(ids[t] == e)[0]
            if len(hit):
                ge[t] = float(w[t, hit[0]])
        ref += ge[:, None] * mlp(x, oracle.dequantize(p13[e], s13[e], 4), oracle.dequantize(p2[e], s2[e], 4))
    ref += mlp(x, oracle.dequantize(sp13, ss13, shared_bits), oracle.dequantize(sp2, ss2, shared_bits))
    ref += as_torch_bf16(res_bits)
    assert np.allclose(ys, ref.numpy(), rtol=1e-12, atol=1e-12)
    # the shared term is really there: dropping it moves the result by far more than rounding
    no_shared = oracle.moe_ffn(x_bits, ids, w, p13, s13, p2, s2, 4, residual_bits=res_bits)
    assert np.abs(no_shared - ys).max() > 1e-3


# ------------------------------------------------------------ dense projections

@pytest.mark.parametrize("bits", [8, 4])
def test_linear_against_torch_functional(bits):
    """y = x W_hat^T (+ residual) against torch.nn.functional.linear in fp64."""
    T, K, N = 5, 384, 256
    w = synth.expert_weight(12, 0, 0, 6, N, K)
    p, s = oracle.quantize_pack(w, bits)
    x_bits = synth.activations_bf16(12, T, K)
    r_bits = synth.activations_bf16(13, T, N)
    y = oracle.linear(x_bits, p, s, bits, residual_bits=r_bits)
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).double()
    r = torch.from_numpy(r_bits.view(np.int16)).view(torch.bfloat16).double()
    ref = F.linear(x, torch.from_numpy(oracle.dequantize(p, s, bits)).double()) + r
    assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_linear_closed_form_on_a_lossless_grid():
    """W = q * 2^-7 with one code 127 per group: y = (x . q^T) * 2^-7 exactly."""
    rng = np.random.default_rng(3)
    q = rng.integers(-127, 128, size=(16, 256))
    q[:, 0] = 127
    q[:, 128] = -127
    w = (q * 2.0 ** -7).astype(np.float32)
    p, s = oracle.quantize_pack(w, 8)
    assert np.all(oracle.f32_from_bf16_bits(s) == 2.0 ** -7)
    x_bits = synth.activations_bf16(14, 3, 256)
    x = oracle.f32_from_bf16_bits(x_bits).astype(np.float64)
    assert np.array_equal(oracle.linear(x_bits, p, s, 8), (x @ q.T.astype(np.float64)) * 2.0 ** -7)
