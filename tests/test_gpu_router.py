"""GPU parity of the bf16 router and the sigmoid shared-expert gate, through the C ABI.

The logits are fp32 sums of 2048 exact bf16 products; the oracle forms them in fp64.
Their difference is held to the standard bound of recursive fp32 summation,
``|l_gpu - l_ref| <= gamma_K * sum_h |x_h w_h|`` with ``gamma_K = K u / (1 - K u)``,
evaluated per logit (the products themselves are exact in fp32); ``u = 2^-23`` so that
the bound holds whether the matrix unit's internal additions round to nearest or
truncate.  The gate then differs by at most a quarter of its logit's bound (the sigmoid's slope is at
most 1/4) plus the fp32 evaluation of the sigmoid (1e-6).

The top-k is an integer decision on fp32 logits, so it is checked where it is unique:
the GPU's ids, weights, counts, offsets and permutation must be exactly the oracle's
routing of the GPU's own logits; and against the oracle's routing of its own logits
they may differ only on tokens whose k-th and (k+1)-th logits lie within twice the
largest observed logit difference of each other.  The FFN output is then checked with the GPU's routing
and the oracle's gate values.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_int4_rtn_amd as w4
from gpu_util import DEV, OracleExperts, bf16_to_dev, check_ffn, gpu_layer, say

pytestmark = pytest.mark.gpu

U = 2.0 ** -23


def _bound(x_bits, w_bits):
    """Per-element bound of fp32 recursive summation of the exact products."""
    x = np.abs(oracle.f32_from_bf16_bits(x_bits).astype(np.float64))
    w = np.abs(oracle.f32_from_bf16_bits(w_bits).astype(np.float64))
    K = x.shape[1]
    gamma = K * U / (1 - K * U)
    return gamma * (x @ w.T)


def _check_router(x, wr, wg, r, k, what):
    T = x.shape[0]
    lg = r["logits"].cpu().numpy()
    ref = oracle.router_logits(x, wr)
    bnd = _bound(x, wr)
    err = np.abs(lg.astype(np.float64) - ref)
    say(f"  {what}: logits max|d| {err.max():.2e}, bound max {bnd.max():.2e}, min slack {(bnd - err).min():.2e}")
    assert np.all(err <= bnd), what
    if wg is not None:
        g = r["shared_gate"].cpu().numpy().astype(np.float64)
        gref = oracle.shared_gate(x, wg)
        gb = _bound(x, wg[None])[:, 0] / 4 + 1e-6
        assert np.all(np.abs(g - gref) <= gb), (what, np.abs(g - gref).max())
    # routing decided on the GPU's logits: exactly the oracle's decision on the same values
    ids, wts, counts, offsets, pairs = oracle.route(lg, k)
    assert np.array_equal(r["ids"].cpu().numpy(), ids)
    assert np.array_equal(r["counts"].cpu().numpy(), counts)
    assert np.array_equal(r["offsets"].cpu().numpy(), offsets)
    assert np.array_equal(r["sorted_pairs"].cpu().numpy(), pairs)
    assert np.abs(r["w"].cpu().numpy() - wts).max() <= 1e-6
    # and the oracle's own (fp32-rounded) logits choose the same experts, except where two
    # of them lie within twice the largest observed difference e (an order flip between
    # two value sets that differ by at most e needs a gap of at most 2e)
    ref32 = ref.astype(np.float32)
    e = np.abs(ref32.astype(np.float64) - lg.astype(np.float64)).max()
    ids_ref = oracle.route(ref32, k)[0]
    srt = -np.sort(-ref32.astype(np.float64), axis=1)
    gap = srt[:, k - 1] - srt[:, k] if k < ref.shape[1] else np.full(T, np.inf)
    differ = np.nonzero(np.any(ids_ref != ids, axis=1))[0]
    say(f"  {len(differ)} of {T} tokens choose differently on the oracle's logits (max |d| {e:.2e})")
    assert np.all(gap[differ] <= 2 * e), (what, differ)
    return ids, wts


def _zero_bank(E, H, I=128):
    return (torch.zeros((E, 2 * I, H // 8), dtype=torch.int32, device=DEV),
            torch.zeros((E, 2 * I, H // 128), dtype=torch.bfloat16, device=DEV),
            torch.zeros((E, H, I // 8), dtype=torch.int32, device=DEV),
            torch.zeros((E, H, I // 128), dtype=torch.bfloat16, device=DEV))


@pytest.mark.parametrize("T", [1, 2, 4, 16, 17, 32, 64, 100, 256, 257, 8192])
def test_router_logits_gate_and_routing(T):
    """Full router shape (256 experts, hidden 2048), with the gate of an INT8 shared expert,
    on every launch path of the forward (single launch, streaming decode, prefill)."""
    E, H, k = 256, 2048, 8
    say(f"router T={T}")
    x = synth.activations_bf16(300 + T, T, H)
    wr = synth.router_weight_bf16(3, 0, E, H)
    wg = synth.shared_gate_weight_bf16(3, 0, H)
    bank = _zero_bank(E, H)
    sh = {n: t[0] for n, t in zip(("w13", "s13", "w2", "s2"), _zero_bank(1, H))}
    sh["bits"] = 4
    y, r = w4.moe_w4a16_forward(bf16_to_dev(x), *bank, top_k=k, router_w=bf16_to_dev(wr), shared=sh,
                                shared_gate_w=bf16_to_dev(wg), routing_out=True)
    torch.cuda.synchronize()
    _check_router(x, wr, wg, r, k, f"T={T}")
    assert not torch.any(y.float() != 0)   # zero experts


@pytest.mark.parametrize("T,bits,shared_bits", [(1, 4, 8), (2, 8, 8), (4, 4, 8), (32, 4, 8), (300, 8, 4),
                                                (1000, 4, 8)])
def test_self_routed_ffn_with_gated_shared_expert(T, bits, shared_bits):
    """The whole layer from x alone: router, top-k, experts, gated shared expert, residual."""
    E, H, I, k = 64, 1024, 256, 8
    say(f"self-routed ffn T={T} bits={bits} shared={shared_bits}")
    routed = gpu_layer(61, 0, E, H, I, bits)
    ref = OracleExperts(61, 0, H, I, bits)
    sh_gpu = gpu_layer(61, 0, 1, H, 512, shared_bits, shared=True)
    sh_ref = OracleExperts(61, 0, H, 512, shared_bits, shared=True).shared_dict()
    x = synth.activations_bf16(400 + T, T, H)
    res = synth.activations_bf16(401 + T, T, H)
    wr = synth.router_weight_bf16(61, 0, E, H)
    wg = synth.shared_gate_weight_bf16(61, 0, H)
    y, r = w4.moe_w4a16_forward(bf16_to_dev(x), *routed, top_k=k, bits=bits, router_w=bf16_to_dev(wr),
                                shared=sh_gpu, shared_gate_w=bf16_to_dev(wg), residual=bf16_to_dev(res),
                                routing_out=True)
    torch.cuda.synchronize()
    ids, wts = _check_router(x, wr, wg, r, k, f"T={T}")
    y_ref = oracle.moe_ffn(x, ids, wts, *ref.as_args(), bits, shared=sh_ref, residual_bits=res,
                           shared_gate=oracle.shared_gate(x, wg))
    check_ffn(y, y_ref, f"self-routed T={T}")
    # the prepared call gives the same bits
    call = w4.MoeCall(bf16_to_dev(x), *routed, top_k=k, bits=bits, shared=sh_gpu, router_w=bf16_to_dev(wr),
                      shared_gate_w=bf16_to_dev(wg))
    out = torch.empty_like(y)
    call(bf16_to_dev(x), out, residual=bf16_to_dev(res))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), y.view(torch.int16))


def test_router_argument_rules():
    E, H, T = 16, 256, 2
    bank = _zero_bank(E, H)
    x = bf16_to_dev(synth.activations_bf16(1, T, H))
    wr = bf16_to_dev(synth.router_weight_bf16(1, 0, E, H))
    with pytest.raises(ValueError):   # logits and router are exclusive
        w4.moe_w4a16_forward(x, *bank, top_k=2, router_w=wr, router_logits=torch.zeros((T, E), device=DEV))
    with pytest.raises(ValueError):   # a gate needs a shared expert
        w4.moe_w4a16_forward(x, *bank, top_k=2, router_w=wr, shared_gate_w=wr[0])
    with pytest.raises(ValueError):   # router of another hidden size
        w4.moe_w4a16_forward(x, *bank, top_k=2, router_w=wr[:, :128].contiguous())
