"""Pins for the oracle's FP8 E4M3 per-channel and MXFP4 formats (CPU only).

FP8: the E4M3 rounding and decoding against torch's float8_e4m3fn conversions (a
library routine), the absmax-to-448 closed form, sign symmetry, power-of-two scaling
and the half-step error bound.  MXFP4: the E2M1 grid and its ties, the OCP
round-to-nearest exponent in closed form, lossless grids, an independent brute-force
re-evaluation of the scale search written with np.percentile and math.log2 on small
blocks, and the search's defining property (its error never exceeds that of any
candidate, the plain RTN exponent included when it is one).
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth
from oracle import formats as FM


# ---------------------------------------------------------------------------- FP8

def test_e4m3_rounding_matches_torch():
    rng = np.random.default_rng(0)
    r = np.concatenate([
        (rng.standard_normal(200000) * 60).astype(np.float32),
        (rng.standard_normal(200000) * 0.01).astype(np.float32),
        # every representable value, every midpoint between neighbours (ties), +-0, the range ends
        FM.e4m3_decode(np.arange(0, 127)).astype(np.float32),
        ((FM.e4m3_decode(np.arange(0, 126)) + FM.e4m3_decode(np.arange(1, 127))) / 2).astype(np.float32),
        np.float32([0.0, -0.0, 448.0, -448.0, 450.0, 463.0, 2.0 ** -10, -(2.0 ** -10), 3 * 2.0 ** -11]),
    ])
    r = np.concatenate([r, -r])
    mine = FM.e4m3_encode(r)
    ref = torch.from_numpy(r).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)


def test_e4m3_decode_matches_torch():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(FM.e4m3_decode(codes), ref.astype(np.float64))
    assert np.all(np.isnan(FM.e4m3_decode(np.array([0x7F, 0xFF], dtype=np.uint8))))
    assert FM.e4m3_decode(np.uint8(0x7E)) == 448.0 and FM.e4m3_decode(np.uint8(1)) == 2.0 ** -9


def test_fp8_quantize_closed_forms_and_invariants():
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((16, 512)) * 0.02).astype(np.float32)
    w[3] = 0.0                                          # an all-zero channel
    codes, s = FM.fp8_quantize(w)
    assert s.dtype == np.float32 and s.shape == (16,)
    assert s[3] == 0 and np.all(codes[3] == 0)
    amax = np.abs(w).max(axis=1)
    assert np.array_equal(s, (amax / np.float32(448)).astype(np.float32))
    # the absmax element of each channel maps to +-448 (code 0x7E with its sign)
    for r in range(16):
        if r == 3:
            continue
        j = np.argmax(np.abs(w[r]))
        assert codes[r, j] & 0x7F == 0x7E and (codes[r, j] >> 7) == (w[r, j] < 0)
    deq = FM.e4m3_decode(codes) * s.astype(np.float64)[:, None]
    # at most half a step of the E4M3 grid at each value (3 mantissa bits; 2^-9 below 2^-6)
    r_ = np.abs(w.astype(np.float64)) / np.where(s == 0, 1, s)[:, None]
    step = np.where(r_ >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(r_, 1e-300))) - 3), 2.0 ** -9)
    assert np.all(np.abs(deq - w) <= step / 2 * np.where(s == 0, 0, s)[:, None] * (1 + 1e-12))
    # sign symmetry and power-of-two scaling
    cn, sn = FM.fp8_quantize(-w)
    assert np.array_equal(sn, s) and np.array_equal(cn[s > 0], (codes ^ 0x80)[s > 0])
    c2, s2 = FM.fp8_quantize(w * np.float32(8))
    assert np.array_equal(c2, codes) and np.array_equal(s2, s * 8)


def test_fp8_pack_layout_and_dequantize():
    codes = np.arange(16, dtype=np.uint8).reshape(2, 8)
    p = FM.fp8_pack(codes)
    assert p.shape == (2, 2) and p.view(np.uint32)[0, 0] == 0x03020100
    w = (np.random.default_rng(2).standard_normal((4, 256)) * 0.02).astype(np.float32)
    packed, s = FM.fp8_quantize_pack(w)
    codes, _ = FM.fp8_quantize(w)
    assert np.array_equal(FM.fp8_dequantize(packed, s), FM.e4m3_decode(codes) * s.astype(np.float64)[:, None])


# -------------------------------------------------------------------------- MXFP4

def test_e2m1_grid_and_ties():
    assert list(FM.e2m1_decode(np.arange(8))) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(FM.e2m1_decode(np.arange(8, 16))) == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    vals = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 100.0, 0.2, 0.3])
    assert list(FM.e2m1_encode(vals)) == [0, 2, 2, 4, 4, 6, 6, 7, 7, 0, 1]
    assert list(FM.e2m1_encode(-vals)) == [8, 10, 10, 12, 12, 14, 14, 15, 15, 8, 9]
    grid = FM.E2M1_VALUES
    assert np.array_equal(FM.e2m1_decode(FM.e2m1_encode(grid)), grid)


def test_mxfp4_rtn_exponent_closed_form():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    e = FM.mxfp4_exponents(w, "rtn")
    amax = np.abs(w.reshape(8, 8, 32)).max(-1)
    assert np.array_equal(e, np.floor(np.log2(amax.astype(np.float64))).astype(np.int64) - 2)
    # a block whose largest value is 6 * 2^k is exact on the grid 2^k; 7 * 2^k clips to 6 * 2^k
    k = -9
    blk = np.zeros((1, 32), np.float32)
    blk[0, :8] = np.float32(FM.E2M1_VALUES * 2.0 ** k)
    nib, sc = FM.mxfp4_quantize(blk, "rtn")
    assert sc[0, 0] == k + 127
    assert np.array_equal(FM.mxfp4_dequantize(FM.mxfp4_pack(nib), sc), blk.astype(np.float64))
    blk[0, 0] = np.float32(7 * 2.0 ** k)
    nib, sc = FM.mxfp4_quantize(blk, "rtn")
    assert sc[0, 0] == k + 127 and FM.e2m1_decode(nib[0, 0]) == 6.0


def test_mxfp4_mse_lossless_grid_and_zero_block():
    k = -7
    rng = np.random.default_rng(4)
    blk = (FM.E2M1_VALUES[rng.integers(0, 8, 32)] * np.where(rng.random(32) < 0.5, -1, 1)).astype(np.float32)
    blk[:2] = [6.0, -6.0]                       # the top two |values| are 6: p99.5 = 6 * 2^k
    w = np.stack([blk * np.float32(2.0 ** k), np.zeros(32, np.float32)])
    e = FM.mxfp4_exponents(w, "mse")
    assert e[0, 0] == k and e[1, 0] == -127
    nib, sc = FM.mxfp4_quantize(w, "mse")
    assert np.array_equal(FM.mxfp4_dequantize(FM.mxfp4_pack(nib), sc), w.astype(np.float64))


def _brute_mse_exponent(block):
    """The page's search written independently: np.percentile, math.log2, a plain sum."""
    a = np.abs(block.astype(np.float64))
    amax = a.max()
    if amax == 0:
        return -127
    p = np.percentile(a, 99.5)
    e0 = math.floor(math.log2(p / 6))
    e_nc = math.ceil(math.log2(amax / 6))
    best = None
    for e in sorted(set(range(e0 - 4, e0 + 2)) | {e_nc}):
        scale = 2.0 ** e
        err = 0.0
        for v in block.astype(np.float64):
            r = v / scale
            q = min(FM.E2M1_VALUES, key=lambda g: (abs(abs(r) - g), g not in (0, 1, 2, 4)))
            err += (v - math.copysign(min(q, 6.0), r) * scale) ** 2
        if best is None or err < best[0] - 1e-30:
            best = (err, e)
    return best[1]


def test_mxfp4_mse_search_against_brute_force():
    rng = np.random.default_rng(5)
    w = np.concatenate([(rng.standard_normal((6, 64)) * 0.02),
                        (rng.standard_t(3, (6, 64)) * 0.01)]).astype(np.float32)
    e = FM.mxfp4_exponents(w, "mse")
    for r in range(w.shape[0]):
        for b in range(2):
            assert e[r, b] == _brute_mse_exponent(w[r, 32 * b:32 * (b + 1)]), (r, b)


def test_mxfp4_percentile_matches_numpy():
    rng = np.random.default_rng(6)
    a = np.abs(rng.standard_normal((1000, 32)))
    assert np.allclose(FM._p995(a), np.percentile(a, 99.5, axis=-1), rtol=1e-15, atol=0)


def test_mxfp4_mse_never_worse_than_rtn_when_rtn_is_a_candidate():
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((64, 2048)) * 0.02).astype(np.float32)
    v = w.reshape(64, 64, 32).astype(np.float64)
    e_mse = FM.mxfp4_exponents(w, "mse")
    e_rtn = FM.mxfp4_exponents(w, "rtn")
    sse_mse = FM._block_sse(v, e_mse)
    sse_rtn = FM._block_sse(v, e_rtn)
    p = FM._p995(np.abs(v))
    e0 = np.floor(np.log2(p / 6)).astype(np.int64)
    in_set = (e_rtn >= e0 - 4) & (e_rtn <= e0 + 1)
    assert in_set.mean() > 0.99
    assert np.all(sse_mse[in_set] <= sse_rtn[in_set])
    # and over the whole matrix the search lowers the weight error
    assert sse_mse.sum() < sse_rtn.sum()


def test_mxfp4_pack_layout():
    nib = np.arange(16).reshape(2, 8)
    p = FM.mxfp4_pack(nib)
    assert p.view(np.uint32)[0, 0] == 0x76543210 and p.view(np.uint32)[1, 0] == 0xFEDCBA98


# ------------------------------------------------------------- FFN in either format

@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_single_expert_ffn_matches_torch_functional(fmt):
    H, I = 256, 128
    w13 = synth.expert_w13(9, 0, 0, H, I)
    w2 = synth.expert_w2(9, 0, 0, H, I)
    if fmt == "fp8":
        p13, s13 = FM.fp8_quantize_pack(w13)
        p2, s2 = FM.fp8_quantize_pack(w2)
        D13, D2 = FM.fp8_dequantize(p13, s13), FM.fp8_dequantize(p2, s2)
    else:
        p13, s13 = FM.mxfp4_quantize_pack(w13)
        p2, s2 = FM.mxfp4_quantize_pack(w2)
        D13, D2 = FM.mxfp4_dequantize(p13, s13), FM.mxfp4_dequantize(p2, s2)
    x_bits = synth.activations_bf16(9, 3, H)
    y = oracle.moe_ffn(x_bits, np.zeros((3, 1), np.int32), np.ones((3, 1), np.float32), p13[None], s13[None],
                       p2[None], s2[None], 8 if fmt == "fp8" else 4, weight_format=fmt)
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).double()
    W13, W2 = torch.from_numpy(D13), torch.from_numpy(D2)
    ref = F.linear(F.silu(F.linear(x, W13[:I])) * F.linear(x, W13[I:]), W2)
    assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)
    # the formats approximate the fp32 weights closely
    rel = np.abs(D13 - w13).sum() / np.abs(w13).sum()
    assert rel < (0.03 if fmt == "fp8" else 0.12)
