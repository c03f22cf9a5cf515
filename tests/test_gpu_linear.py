"""GPU parity of the dense quantized projection ``w4a16_linear`` through the C ABI.

The shapes are the INT8 group-128 projections of the Int4-Int8Mix recipe at this model's
size (hidden 2048): attention q_proj (8192 x 2048, query and output gate), k_proj and
v_proj (512 x 2048), o_proj (2048 x 4096); Gated DeltaNet in_proj_qkv (8192 x 2048),
in_proj_z (4096 x 2048), out_proj (2048 x 4096) -- with these, ten attention layers hold
0.27 B and thirty DeltaNet layers 1.01 B parameters, the counts the NVFP4-FP8 page's
parameter census gives.  Token counts cover the small-batch kernel (1..64) and the
grouped GEMM (65 and up, several M-tiles, a ragged tail).  Bar: the FFN acceptance
tolerance against the oracle's fp64 product on its own quantization.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_int4_rtn_amd as w4
from oracle import formats as FM
from gpu_util import DEV, bf16_to_dev, check_ffn, f32_to_dev, say

pytestmark = pytest.mark.gpu

SHAPES = {"q_proj": (8192, 2048), "k_proj": (512, 2048), "o_proj": (2048, 4096), "in_proj_z": (4096, 2048)}


_ORACLE_Q = {}   # the oracle's quantization of each weight matrix, shared by parametrized cases


def _weights(N, K, seed, fmt="int", bits=8):
    w = synth.expert_weight(40 + seed, 0, 0, 6, N, K)
    dev = f32_to_dev(w)
    key = (N, K, seed, fmt, bits)
    if fmt == "int":
        g = w4.rtn_quantize_pack(dev, bits)
        if key not in _ORACLE_Q:
            _ORACLE_Q[key] = oracle.quantize_pack(w, bits)
    elif fmt == "fp8":
        g = w4.fp8_quantize_pack(dev)
        if key not in _ORACLE_Q:
            _ORACLE_Q[key] = FM.fp8_quantize_pack(w)
    else:
        g = w4.mxfp4_quantize_pack(dev, "mse")
        if key not in _ORACLE_Q:
            _ORACLE_Q[key] = FM.mxfp4_quantize_pack(w, "mse")
    torch.cuda.synchronize()
    return g, _ORACLE_Q[key]


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("T", [1, 4, 32, 64, 65, 300])
def test_linear_int8_projection_shapes(name, T):
    N, K = SHAPES[name]
    say(f"linear {name} T={T}")
    (p, s), (pr, sr) = _weights(N, K, hash(name) % 97)
    x = synth.activations_bf16(800 + T, T, K)
    y = w4.w4a16_linear(bf16_to_dev(x), p, s, bits=8)
    torch.cuda.synchronize()
    check_ffn(y, oracle.linear(x, pr, sr, 8), f"{name} T={T}")


@pytest.mark.parametrize("fmt,bits", [("int", 4), ("fp8", 8), ("mxfp4", 4)])
@pytest.mark.parametrize("T", [2, 200])
def test_linear_other_formats(fmt, bits, T):
    N, K = 1024, 2048
    say(f"linear {fmt} bits={bits} T={T}")
    (p, s), (pr, sr) = _weights(N, K, 7, fmt, bits)
    x = synth.activations_bf16(900 + T, T, K)
    y = w4.w4a16_linear(bf16_to_dev(x), p, s, bits=bits, weight_format=fmt)
    torch.cuda.synchronize()
    check_ffn(y, oracle.linear(x, pr, sr, bits, weight_format=fmt), f"{fmt} T={T}")


@pytest.mark.parametrize("T", [3, 1000])
def test_linear_residual_in_place_and_reproducible(T):
    N, K = 2048, 4096
    say(f"linear residual T={T}")
    (p, s), (pr, sr) = _weights(N, K, 9)
    x = synth.activations_bf16(950 + T, T, K)
    r = synth.activations_bf16(951 + T, T, N)
    rd = bf16_to_dev(r)
    y = w4.w4a16_linear(bf16_to_dev(x), p, s, residual=rd)
    torch.cuda.synchronize()
    ref = oracle.linear(x, pr, sr, 8, residual_bits=r)
    check_ffn(y, ref, f"residual T={T}")
    w4.w4a16_linear(bf16_to_dev(x), p, s, residual=rd, out=rd)   # y overwrites the residual
    torch.cuda.synchronize()
    assert torch.equal(rd.view(torch.int16), y.view(torch.int16))


# Small batches run one weight-streaming kernel when K / 128 splits into at most 16 equal
# ranges of 1, 2 or 4 groups (at most 2 for 8-bit codes), else the down-projection path:
# (N, K, bits, format) with K / 128 = 3 (3 waves of one group), 17 (too many ranges: the
# down path), 64 (16 waves of 4 INT4 groups; INT8: the down path) and 1.  Above 16 tokens
# the last three shapes take two 16-row blocks per workgroup (INT4 two groups per wave,
# FP8 and MXFP4 one), as q_proj and in_proj_z do in the INT8 shapes above.
@pytest.mark.parametrize("N,K,bits,fmt", [(256, 384, 8, "int"), (256, 2176, 8, "int"), (512, 8192, 4, "int"),
                                          (512, 8192, 8, "int"), (128, 128, 4, "mxfp4"), (384, 1024, 8, "fp8"),
                                          (8192, 2048, 4, "int"), (4096, 2048, 8, "fp8"), (4096, 2048, 4, "mxfp4")])
@pytest.mark.parametrize("T", [1, 17, 64])
def test_linear_small_batch_group_splits(N, K, bits, fmt, T):
    say(f"linear small N={N} K={K} bits={bits} {fmt} T={T}")
    (p, s), (pr, sr) = _weights(N, K, 11, fmt, bits)
    x = synth.activations_bf16(700 + T, T, K)
    y = w4.w4a16_linear(bf16_to_dev(x), p, s, bits=bits, weight_format=fmt)
    torch.cuda.synchronize()
    check_ffn(y, oracle.linear(x, pr, sr, bits, weight_format=fmt), f"N={N} K={K} {fmt}{bits} T={T}")
    y2 = w4.w4a16_linear(bf16_to_dev(x), p, s, bits=bits, weight_format=fmt)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))   # partials summed in a fixed order
