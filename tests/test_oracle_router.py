"""Pins for the oracle's router logits and shared-expert gate (CPU only).

The router is pinned by torch.nn.functional.linear in fp64 on the widened bf16
tensors and by a one-hot closed form; the gate by SciPy's logistic function and
its closed forms (0.5 at zero, the symmetry g(-z) = 1 - g(z)); the gated shared
term by its linearity in the gate (weight 1 reproduces the ungated sum, weight 0
removes the shared expert).
"""

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
import synth


def _t(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double()


@pytest.mark.parametrize("T,E,H", [(1, 256, 2048), (7, 16, 256), (33, 64, 384)])
def test_router_logits_against_torch_linear(T, E, H):
    x = synth.activations_bf16(5, T, H)
    wr = synth.router_weight_bf16(5, 0, E, H)
    got = oracle.router_logits(x, wr)
    ref = F.linear(_t(x), _t(wr)).numpy()
    assert got.shape == (T, E)
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)
    # N(0, 1/H) weights on N(0, 1) activations: logits of unit scale
    if T * E >= 256:
        assert 0.7 < got.std() < 1.3


def test_router_one_hot_closed_form():
    """x = unit vector e_h gives exactly column h of the router; 2 e_h gives twice it."""
    E, H = 32, 256
    wr = synth.router_weight_bf16(6, 0, E, H)
    W = oracle.f32_from_bf16_bits(wr).astype(np.float64)
    for h in (0, 77, 255):
        x = np.zeros((2, H), np.float32)
        x[0, h], x[1, h] = 1.0, 2.0
        got = oracle.router_logits(oracle.bf16_bits_from_f32(x), wr)
        assert np.array_equal(got[0], W[:, h]) and np.array_equal(got[1], 2 * W[:, h])


def test_shared_gate_against_scipy_and_closed_forms():
    T, H = 9, 512
    x = synth.activations_bf16(7, T, H)
    wg = synth.shared_gate_weight_bf16(7, 0, H)
    g = oracle.shared_gate(x, wg)
    z = F.linear(_t(x), _t(wg)[None]).numpy()[:, 0]
    assert np.allclose(g, scipy.special.expit(z), rtol=1e-14, atol=0)
    assert np.all((g > 0) & (g < 1))
    # zero weights: exactly one half; negated activations: 1 - g
    assert np.all(oracle.shared_gate(x, np.zeros_like(wg)) == 0.5)
    neg = oracle.bf16_bits_from_f32(-oracle.f32_from_bf16_bits(x))
    assert np.allclose(oracle.shared_gate(neg, wg), 1 - g, rtol=0, atol=1e-15)


def test_gated_shared_term_is_linear_in_the_gate():
    E, H, I, k, T = 8, 256, 128, 2, 5
    w13 = np.stack([synth.expert_w13(8, 0, e, H, I) for e in range(E)])
    w2 = np.stack([synth.expert_w2(8, 0, e, H, I) for e in range(E)])
    p13, s13 = oracle.quantize_pack(w13, 4)
    p2, s2 = oracle.quantize_pack(w2, 4)
    sp13, ss13 = oracle.quantize_pack(synth.expert_w13(8, 0, 0, H, I, shared=True), 8)
    sp2, ss2 = oracle.quantize_pack(synth.expert_w2(8, 0, 0, H, I, shared=True), 8)
    shared = dict(w13=sp13, s13=ss13, w2=sp2, s2=ss2, bits=8)
    x = synth.activations_bf16(8, T, H)
    ids, w, *_ = oracle.route(synth.router_logits(8, T, E), k)
    args = (x, ids, w, p13, s13, p2, s2, 4)
    routed = oracle.moe_ffn(*args)
    full = oracle.moe_ffn(*args, shared=shared)
    assert np.array_equal(oracle.moe_ffn(*args, shared=shared, shared_gate=np.ones(T)), full)
    assert np.array_equal(oracle.moe_ffn(*args, shared=shared, shared_gate=np.zeros(T)), routed)
    g = np.linspace(0.1, 0.9, T)
    mixed = oracle.moe_ffn(*args, shared=shared, shared_gate=g)
    assert np.allclose(mixed, routed + g[:, None] * (full - routed), rtol=1e-12, atol=1e-13)
