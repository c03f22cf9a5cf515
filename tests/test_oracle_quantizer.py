"""Pins for the oracle's RTN quantizer and packer (CPU only).

Each check is fixed by something other than the oracle itself: a closed-form
grid, the IEEE round-half-to-even rule, algebraic invariants, a library
conversion, or the error band printed on page "Nex-N2.5-mini Int4-Int8Mix"
(Recipe).  The last test plants plausible mistakes in copies of the quantizer
and checks that the pins catch each of them.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import rtn_moe

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def facts():
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        return json.load(f)


# --------------------------------------------------------------- bf16 helper

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(10000) * 1e-30).astype(np.float32),
        (rng.standard_normal(10000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.4e38, -3.4e38, 1e-45, 2 ** -126,
                  np.float32(1.00390625), np.float32(1.01171875)], dtype=np.float32),
    ])
    # values exactly half-way between two bf16 neighbours, odd and even
    mid = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, mid, -mid])
    ours = oracle.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = oracle.f32_from_bf16_bits(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


# ------------------------------------------------------------ closed forms

@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("m", [-12, -7, 0, 3])
def test_lossless_grid(bits, m):
    """W = q0 * 2^m with |q0| <= QMAX and +-QMAX in every group quantizes to
    exactly (q0, 2^m): QMAX*2^m / QMAX = 2^m is exact and a bf16."""
    qmax = oracle.QMAX[bits]
    rng = np.random.default_rng(bits * 100 + m)
    q0 = rng.integers(-qmax, qmax + 1, size=(6, 512))
    q0[:, ::128] = qmax * rng.choice([-1, 1], size=(6, 4))
    w = (q0 * 2.0 ** m).astype(np.float32)
    q, s_bits = oracle.rtn_quantize(w, bits)
    assert np.array_equal(q, q0)
    assert np.all(oracle.f32_from_bf16_bits(s_bits) == np.float32(2.0 ** m))


def test_round_half_to_even_worked_example():
    """Group absmax 7 * 2^-7 gives s = 2^-7 exactly; then w/s is exact and the
    five half-way inputs 0.5, 1.5, 2.5, -2.5, 3.5 must round to 0, 2, 2, -2, 4
    (round-half-away-from-zero would give 1, 2, 3, -3, 4)."""
    u = 2.0 ** -7
    w = np.zeros((1, 128), np.float32)
    w[0, :6] = np.array([7, 0.5, 1.5, 2.5, -2.5, 3.5]) * u
    q, s_bits = oracle.rtn_quantize(w, 4)
    assert oracle.f32_from_bf16_bits(s_bits)[0, 0] == np.float32(u)
    assert list(q[0, :6]) == [7, 0, 2, 2, -2, 4]


def test_scale_is_rounded_to_bf16_before_dividing():
    """absmax = 1.0: 1/7 in fp32 is 0x3E124925, bf16 RNE of it is 0x3E12
    (0.142578125).  Dividing by that stored scale, w = 0.5 gives
    0.5 / 0.142578125 = 3.5068... -> 4; with the unrounded 1/7 it would be 3.5 -> 4
    as well, so use w = 0.4993: 3.5019 -> 4 against 3.4951 -> 3."""
    w = np.zeros((1, 128), np.float32)
    w[0, 0] = 1.0
    w[0, 1] = 0.4993
    q, s_bits = oracle.rtn_quantize(w, 4)
    assert s_bits[0, 0] == 0x3E12
    assert q[0, 0] == 7 and q[0, 1] == 4


def test_zero_group_gives_zero_scale_and_codes():
    w = np.zeros((3, 256), np.float32)
    w[1, 128:] = 0.25
    q, s_bits = oracle.rtn_quantize(w, 4)
    assert np.all(q[0] == 0) and np.all(q[1, :128] == 0) and np.all(q[2] == 0)
    assert s_bits[0, 0] == 0 and s_bits[1, 0] == 0 and s_bits[1, 1] != 0
    assert np.all(q[1, 128:] == 7)


# --------------------------------------------------------------- invariants

@pytest.mark.parametrize("bits", [4, 8])
def test_invariants_gaussian(bits):
    rng = np.random.default_rng(7 + bits)
    w = (rng.standard_normal((64, 1024)) * 0.02).astype(np.float32)
    qmax = oracle.QMAX[bits]
    q, s_bits = oracle.rtn_quantize(w, bits)
    s = oracle.f32_from_bf16_bits(s_bits).astype(np.float64)
    # codes stay inside the symmetric grid
    assert q.min() >= -qmax and q.max() <= qmax
    # the absmax element of each group lands on +-qmax with its sign
    g = w.reshape(64, 8, 128)
    qg = q.reshape(64, 8, 128)
    arg = np.abs(g).argmax(axis=-1)
    top = np.take_along_axis(qg, arg[..., None], -1)[..., 0]
    sign = np.sign(np.take_along_axis(g, arg[..., None], -1)[..., 0])
    assert np.array_equal(top, (qmax * sign).astype(np.int32))
    # rounding error at most half a step (plus the fp32 rounding of w/s)
    err = np.abs(g.astype(np.float64) - qg * s[..., None])
    assert np.all(err <= s[..., None] * (0.5 + 2.0 ** -20))
    # odd symmetry and power-of-two scale equivariance
    qn, sn = oracle.rtn_quantize(-w, bits)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s_bits)
    for m in (-3, 5):
        qm, sm = oracle.rtn_quantize((w * 2.0 ** m).astype(np.float32), bits)
        assert np.array_equal(qm, q)
        assert np.array_equal(oracle.f32_from_bf16_bits(sm), (s * 2.0 ** m).astype(np.float32))


def test_bf16_input_equals_fp32_of_same_values():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    wb = oracle.f32_from_bf16_bits(oracle.bf16_bits_from_f32(w))
    q1, s1 = oracle.rtn_quantize(wb, 4)
    q2, s2 = oracle.rtn_quantize(torch.from_numpy(w).to(torch.bfloat16).float().numpy(), 4)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


# ---------------------------------------------- the pages' round-trip band

def _mean_rel_error(w, bits):
    packed, s_bits = oracle.quantize_pack(w, bits)
    wh = oracle.dequantize(packed, s_bits, bits).astype(np.float64)
    return np.abs(wh - w).sum() / np.abs(w).sum()


def test_roundtrip_error_in_page_band():
    """Int4-Int8Mix Recipe: INT4 about 11-14 % mean relative per weight, INT8
    about 0.8 %.  Read as sum|w_hat - w| / sum|w| per matrix; Gaussian N(0, 0.02)
    weights of the gate/up shape give about 12.6 % and 0.7 %."""
    f = facts()
    lo, hi = f["int4_roundtrip_mean_rel_error_pct"]["value"]
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((512, 2048)) * 0.02).astype(np.float32)
    e4 = 100 * _mean_rel_error(w, 4)
    e8 = 100 * _mean_rel_error(w, 8)
    assert lo <= e4 <= hi, e4
    assert 0.5 <= e8 <= 1.0, e8
    assert abs(e8 - f["int8_roundtrip_mean_rel_error_pct"]["value"]) < 0.3


# ------------------------------------------------------------------- packing

def test_pack_layout_and_roundtrip():
    q = np.arange(-8, 8, dtype=np.int32)[None, :]
    words = oracle.pack_codes(q, 4).view(np.uint32)
    assert list(words[0]) == [0x76543210, 0xFEDCBA98]
    q8 = np.array([[-128, -1, 0, 127]], np.int32)
    assert oracle.pack_codes(q8, 8).view(np.uint32)[0, 0] == 0xFF80_7F00
    rng = np.random.default_rng(5)
    for bits in (4, 8):
        qmax = oracle.QMAX[bits]
        q = rng.integers(-qmax - 1, qmax + 1, size=(3, 5, 256)).astype(np.int32)
        assert np.array_equal(oracle.unpack_codes(oracle.pack_codes(q, bits), bits), q)


def test_nibble_histogram_symmetric_for_gaussian():
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((256, 2048)) * 0.02).astype(np.float32)
    packed, _ = oracle.quantize_pack(w, 4)
    u = oracle.unpack_codes(packed, 4) + 8
    h = np.bincount(u.ravel(), minlength=16)
    assert h[0] == 0                                   # -8 is never produced
    for d in range(1, 8):                              # 8 +- d equally frequent
        assert abs(h[8 + d] - h[8 - d]) < 0.02 * (h[8 + d] + h[8 - d]) + 50


def test_dequant_is_exact_product():
    rng = np.random.default_rng(4)
    for bits in (4, 8):
        w = (rng.standard_normal((16, 384)) * 0.05).astype(np.float32)
        packed, s_bits = oracle.quantize_pack(w, bits)
        q = oracle.unpack_codes(packed, bits).astype(np.float64)
        s = oracle.f32_from_bf16_bits(s_bits).astype(np.float64)
        exact = (q.reshape(16, 3, 128) * s[..., None]).reshape(16, 384)
        assert np.array_equal(oracle.dequantize(packed, s_bits, bits).astype(np.float64), exact)


# ----------------------------------------------------------- page accounting

def test_page_tensor_accounting():
    """Int4-Int8Mix Stats: 30,720 INT4 expert matrices are 40 layers x 256
    experts x 3 projections, and the 93,594 tensors are three per quantized
    matrix (packed, scale, shape) plus the pass-through tensors."""
    f = facts()
    n4 = f["int4_expert_matrices"]["value"]
    assert n4 == f["layers"]["value"] * f["routed_experts"]["value"] * 3
    assert 3 * (n4 + f["int8_side_matrices"]["value"]) + f["passthrough_tensors"]["value"] == \
        f["total_tensors"]["value"]
    E, twoI, H = f["fused_gate_up_bank_shape"]["value"]
    assert f["fused_down_bank_shape"]["value"] == [E, H, twoI // 2]
    assert H == f["hidden_size"]["value"]
    params = f["layers"]["value"] * E * (twoI * H + H * twoI // 2)
    assert abs(params / 1e9 - f["routed_expert_params_billions"]["value"]) < 0.005


# --------------------------------------------------- the pins catch mistakes

def _variant(kind):
    """Quantizers with one plausible mistake each, built from the oracle's pieces."""
    def quant(w, bits, group=128):
        w = np.asarray(w, np.float32)
        qmax = oracle.QMAX[bits]
        if kind == "transposed_groups":
            g = w.reshape(-1, group, w.shape[-1] // group).swapaxes(-1, -2)
        else:
            g = w.reshape(*w.shape[:-1], w.shape[-1] // group, group)
        div = np.float32(qmax + 0.5) if kind == "half_range" else np.float32(qmax)
        s_bits = oracle.bf16_bits_from_f32(np.abs(g).max(-1) / div)
        s = oracle.f32_from_bf16_bits(s_bits)
        if kind == "unrounded_scale":
            s = (np.abs(g).max(-1) / div).astype(np.float32)
        r = g / s[..., None]
        if kind == "half_away":
            qq = np.sign(r) * np.floor(np.abs(r) + 0.5)
        else:
            qq = np.rint(r)
        qq = np.clip(qq, -qmax - 1, qmax)
        if kind == "transposed_groups":
            qq = qq.swapaxes(-1, -2)
        return qq.astype(np.int32).reshape(w.shape), s_bits
    return quant


@pytest.mark.parametrize("kind", ["half_away", "half_range", "unrounded_scale", "transposed_groups"])
def test_pins_catch_planted_mistakes(kind, monkeypatch):
    monkeypatch.setattr(rtn_moe, "rtn_quantize", _variant(kind))
    monkeypatch.setattr(oracle, "rtn_quantize", _variant(kind))
    checks = [
        test_round_half_to_even_worked_example,
        lambda: test_lossless_grid(4, -7),
        test_scale_is_rounded_to_bf16_before_dividing,
        lambda: test_invariants_gaussian(4),
    ]
    failures = 0
    for c in checks:
        try:
            c()
        except AssertionError:
            failures += 1
    assert failures >= 1
