"""Plain NumPy oracle of the W4A16 routed-expert path.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by the tests,
the smoke check and the benchmark's CPU-baseline leg, never by the library.

Precision.  Integer decisions (the quantized codes, the top-k choice) are taken
in fp32, the precision of the stored weights and logits, with IEEE
correctly-rounded division and round-half-to-even, exactly as stated at each
function.  Everything that only produces a floating-point result (routing
weights, the expert MLPs, the weighted sum) is computed in fp64, so the oracle
is at least as accurate as the fp32 arithmetic the path is held to.

Parity pins.  Every function here is pinned by CPU tests to facts that do not
come from this file: closed-form quantizer grids and tie cases, the error band
the Int4-Int8Mix page reports, brute-force sorting, library softmax and a
``torch.nn.functional`` MLP, and algebraic invariants.  Two facts remain
readings rather than pins, because no page and no artifact fixes them: the bit
layout of the packed words (offset-binary, lowest column in the lowest bits)
and the order of the fused gate/up rows (gate first).  Both are listed as
"parity unpinned" where the design notes list the readings.
"""

from __future__ import annotations

from collections import defaultdict

import numpy as np

# One scale per 128 consecutive input columns of an [out, in] matrix
# (page "Nex-N2.5-mini Int4-Int8Mix", section Recipe, precision table).
GROUP = 128

# Largest code magnitude of the symmetric grid: the group's absmax element maps
# to +-QMAX.  The Recipe section says "symmetric" with min-max scales; the plain
# symmetric reading of that is absmax / (2^(bits-1) - 1), which keeps the grid
# sign-symmetric (Q(-W) = -Q(W)).
QMAX = {4: 7, 8: 127}


# ---------------------------------------------------------------------------
# bfloat16 helpers (scales and activations are stored as bf16 bit patterns)
# ---------------------------------------------------------------------------

def bf16_bits_from_f32(x) -> np.ndarray:
    """Round fp32 values to bfloat16, ties to even; return the uint16 bit patterns.

    bf16 keeps the top 16 bits of an fp32.  Round-to-nearest-even on the 16
    dropped bits: add 0x7FFF plus the lowest kept bit, then truncate.  A finite
    value that rounds past the largest bf16 becomes infinity, as IEEE rounding
    requires.  NaN maps to the canonical quiet NaN 0x7FC0.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    return np.where(np.isnan(x), np.uint16(0x7FC0), r).astype(np.uint16)


def f32_from_bf16_bits(b) -> np.ndarray:
    """Widen bfloat16 bit patterns to fp32 (exact: append 16 zero bits)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# RTN group quantizer and packer
# ---------------------------------------------------------------------------

def rtn_quantize(w, bits: int, group: int = GROUP):
    """Symmetric round-to-nearest group quantization of ``w[..., rows, cols]``.

    Page "Nex-N2.5-mini Int4-Int8Mix", section Recipe: data-free
    round-to-nearest per group with min-max scales, symmetric, group 128
    (INT4 for routed experts, INT8 for the other projections).

    For every row and every group of ``group`` consecutive input columns:

    1. ``a`` = largest |w| in the group (exact in fp32);
    2. ``s`` = bf16( a / QMAX ) with an IEEE fp32 division, then round to bf16
       ties-to-even (the stored scale is 16-bit);
    3. ``q`` = clamp( rint( w / s ), -QMAX-1, QMAX ), dividing by the *stored*
       bf16 scale with an IEEE fp32 division and rounding ties to even;
    4. an all-zero group has ``s = 0`` and every ``q = 0``.

    Returns ``(q, scale_bits)``: int32 codes shaped like ``w`` and uint16 bf16
    bit patterns shaped ``[..., rows, cols // group]``.
    """
    if bits not in QMAX:
        raise ValueError("bits must be 4 or 8")
    w = np.ascontiguousarray(w, dtype=np.float32)
    cols = w.shape[-1]
    if cols % group:
        raise ValueError("cols must be a multiple of the group size")
    qmax = QMAX[bits]
    qmin = -qmax - 1
    g = w.reshape(*w.shape[:-1], cols // group, group)
    absmax = np.max(np.abs(g), axis=-1)
    s32 = (absmax / np.float32(qmax)).astype(np.float32)
    s_bits = bf16_bits_from_f32(s32)
    s = f32_from_bf16_bits(s_bits)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (g / s[..., None]).astype(np.float32)
    q = np.clip(np.rint(ratio), qmin, qmax)
    q = np.where(s[..., None] == 0, 0.0, q)
    return q.astype(np.int32).reshape(w.shape), s_bits


def pack_codes(q, bits: int) -> np.ndarray:
    """Pack signed codes along the last axis into int32 words.

    Each code is stored offset-binary, ``u = q + 2^(bits-1)`` (so INT4 codes
    -8..7 become nibbles 0..15).  Column ``c`` lands in word ``c // (32/bits)``
    at bit offset ``bits * (c mod 32/bits)``: eight nibbles per word for INT4,
    four bytes for INT8, lowest column in the lowest bits.
    """
    per = 32 // bits
    q = np.asarray(q)
    if q.shape[-1] % per:
        raise ValueError("last axis must be a multiple of 32/bits")
    u = (q.astype(np.int64) + (1 << (bits - 1))).astype(np.uint32)
    if np.any(u >> np.uint32(bits)):
        raise ValueError("code out of range")
    u = u.reshape(*q.shape[:-1], q.shape[-1] // per, per)
    word = np.zeros(u.shape[:-1], dtype=np.uint32)
    for i in range(per):
        word |= u[..., i] << np.uint32(bits * i)
    return word.view(np.int32)


def unpack_codes(words, bits: int) -> np.ndarray:
    """Inverse of :func:`pack_codes`: int32 words -> signed int32 codes."""
    per = 32 // bits
    w = np.ascontiguousarray(words).view(np.uint32)
    mask = np.uint32((1 << bits) - 1)
    out = np.empty((*w.shape, per), dtype=np.int32)
    for i in range(per):
        out[..., i] = ((w >> np.uint32(bits * i)) & mask).astype(np.int32)
    out -= 1 << (bits - 1)
    return out.reshape(*w.shape[:-1], w.shape[-1] * per)


def quantize_pack(w, bits: int, group: int = GROUP):
    """RTN-quantize then pack: ``w[..., rows, cols]`` -> (packed int32, scale bf16 bits).

    The two arrays, together with the matrix shape, are the three tensors the
    Int4-Int8Mix page (Recipe and its Stats line) stores per quantized matrix.
    """
    q, s_bits = rtn_quantize(w, bits, group)
    return pack_codes(q, bits), s_bits


def dequantize(packed, scale_bits, bits: int, group: int = GROUP) -> np.ndarray:
    """``W_hat = q * s`` in fp32.  Exact: q has at most 8 significant bits and
    a bf16 scale 8, so the product fits fp32's 24-bit significand."""
    q = unpack_codes(packed, bits)
    s = f32_from_bf16_bits(scale_bits)
    cols = q.shape[-1]
    qg = q.reshape(*q.shape[:-1], cols // group, group).astype(np.float32)
    return (qg * s[..., None]).reshape(q.shape)


# ---------------------------------------------------------------------------
# Routing
# ---------------------------------------------------------------------------

def route(logits, k: int):
    """Top-k routing with renormalised softmax weights and the canonical permutation.

    Page "Nex-N2.5-mini FP8 W8A8 with Calibrated FP8 KV Scales", Artifact
    summary: 256 routed experts, 8 active per token.  The weighting is the
    softmax over all experts, renormalised over the k chosen ones.

    * selection on the fp32 logits, largest first; equal logits go to the
      lower expert index; slot j holds the j-th chosen expert;
    * ``p = softmax(logits)`` over all E in fp64, ``w_j = p[ids_j] / sum_j p[ids_j]``,
      stored as fp32;
    * ``counts[e]`` = number of (token, slot) pairs routed to e,
      ``offsets`` = exclusive prefix sum (E + 1 entries);
    * ``sorted_pairs``: pair ids ``t*k + j`` ordered by expert, then token.

    Returns ``(ids int32 [T,k], w fp32 [T,k], counts int32 [E],
    offsets int32 [E+1], sorted_pairs int32 [T*k])``.
    """
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    expert_index = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((expert_index, -logits), axis=-1)
    ids = order[:, :k].astype(np.int32)

    l64 = logits.astype(np.float64)
    p = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    p_sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    w = (p_sel / p_sel.sum(axis=1, keepdims=True)).astype(np.float32)

    flat = ids.reshape(-1)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    pair_id = np.arange(T * k)
    sorted_pairs = np.lexsort((pair_id, flat)).astype(np.int32)
    return ids, w, counts, offsets, sorted_pairs


# ---------------------------------------------------------------------------
# Router and shared-expert gate (kept in BF16)
# ---------------------------------------------------------------------------

def router_logits(x_bits, wr_bits):
    """Router logits ``l[t, e] = sum_h x[t, h] * Wr[e, h]``, fp64.

    Page "Nex-N2.5-mini Int4-Int8Mix", Recipe table: the routers (``mlp.gate``)
    are left in BF16; page "Nex-N2.5-mini FP8 W8A8 with Calibrated FP8 KV Scales",
    "Components retained at source precision": MoE routers.  So the router is a
    plain bf16 linear map ``[E, H]`` applied to the bf16 activation; both are
    widened exactly and the sum is taken in fp64.

    ``x_bits`` uint16 bf16 ``[T, H]``; ``wr_bits`` uint16 bf16 ``[E, H]``.
    Returns fp64 ``[T, E]``.
    """
    x = f32_from_bf16_bits(x_bits).astype(np.float64)
    wr = f32_from_bf16_bits(wr_bits).astype(np.float64)
    return x @ wr.T


def shared_gate(x_bits, wg_bits):
    """Shared-expert gate ``g[t] = sigmoid(sum_h x[t, h] * wg[h])``, fp64.

    The same two pages keep ``shared_expert_gate`` in BF16 next to the router.
    The pages name the gate but not its function; the reading taken is the
    plainest one for a single-output gate on a residual branch: a bf16 linear
    map ``[1, H]`` followed by the logistic sigmoid ``1 / (1 + exp(-z))``, whose
    value scales the shared expert's output for that token.

    ``x_bits`` uint16 bf16 ``[T, H]``; ``wg_bits`` uint16 bf16 ``[H]``.
    Returns fp64 ``[T]``.
    """
    x = f32_from_bf16_bits(x_bits).astype(np.float64)
    wg = f32_from_bf16_bits(wg_bits).astype(np.float64)
    z = x @ wg
    return 1.0 / (1.0 + np.exp(-z))


# ---------------------------------------------------------------------------
# Expert MLP and the routed sum
# ---------------------------------------------------------------------------

def expert_ffn(x, w13, w2):
    """One routed expert on one token, fp64.

    Page "Nex-N2.5-mini Int4-Int8Mix", Recipe table: an expert is gate_proj,
    up_proj and down_proj.  ``w13`` is ``[2I, H]`` with the gate rows first and
    the up rows second (the split of the fused ``gate_up_proj`` bank the Recipe
    section describes); ``w2`` is ``[H, I]``.

    ``a = SiLU(Wg x) * (Wu x)`` with ``SiLU(z) = z / (1 + exp(-z))``; returns
    ``W2 a``.  ``x`` may also be ``[H, n]``: n tokens as columns, each evaluated
    independently (the same products, as a matrix instead of n vectors).
    """
    I = w13.shape[0] // 2
    g = w13[:I] @ x
    u = w13[I:] @ x
    with np.errstate(over="ignore"):
        a = g / (1.0 + np.exp(-g)) * u
    return w2 @ a


def dequantize_as(packed, scales, bits: int, weight_format: str = "int") -> np.ndarray:
    """Dequantize one packed matrix in any of the expert weight formats, fp64:
    ``int`` (RTN group 128, bf16 scales: :func:`dequantize`), ``fp8`` (E4M3 codes with
    one fp32 scale per row) or ``mxfp4`` (E2M1 codes with E8M0 scales per 32 columns);
    see ``oracle.formats``."""
    if weight_format == "int":
        return dequantize(packed, scales, bits).astype(np.float64)
    from . import formats
    if weight_format == "fp8":
        return formats.fp8_dequantize(packed, scales)
    if weight_format == "mxfp4":
        return formats.mxfp4_dequantize(packed, scales)
    raise ValueError(f"unknown weight format {weight_format!r}")


def moe_ffn(x_bits, ids, w, w13, s13, w2, s2, bits: int, tokens=None,
            shared=None, residual_bits=None, shared_gate=None, weight_format: str = "int"):
    """Router-weighted sum of the selected W4A16 experts, fp64.

    ``y_t = sum_j w[t,j] * FFN_{ids[t,j]}(x_t)`` over the slots in order, then
    plus the shared expert (weight 1) when ``shared`` is given, then plus the
    residual when given.  The expert weights are the dequantized ``q * s`` of
    the packed tensors; ``x`` is the bf16 activation widened exactly.

    Arguments: ``x_bits`` uint16 bf16 ``[T, H]``; ``ids`` / ``w`` ``[T, k]``;
    ``w13`` int32 ``[E, 2I, H*bits/32]`` with scales ``s13`` ``[E, 2I, H/128]``;
    ``w2`` int32 ``[E, H, I*bits/32]`` with scales ``s2`` ``[E, H, I/128]``.
    ``tokens`` restricts the output to those token indices (default: all).
    ``shared`` is a dict with keys ``w13, s13, w2, s2, bits`` (one expert,
    leading axis absent); ``shared_gate`` (``[T]``, see :func:`shared_gate`)
    scales its output per token instead of the weight 1.  Returns fp64
    ``[len(tokens), H]``.  ``weight_format`` names the routed experts' format
    (``int``, ``fp8`` or ``mxfp4``, see :func:`dequantize_as`); the shared expert is
    always the ``int`` format.
    """
    x = f32_from_bf16_bits(x_bits).astype(np.float64)
    T, k = ids.shape
    tokens = list(range(T)) if tokens is None else [int(t) for t in tokens]
    H = x.shape[1]

    by_expert = defaultdict(list)
    for ti, t in enumerate(tokens):
        for j in range(k):
            by_expert[int(ids[t, j])].append((ti, j))
    out = np.zeros((len(tokens), k, H))
    for e in sorted(by_expert):
        W13 = dequantize_as(w13[e], s13[e], bits, weight_format)
        W2 = dequantize_as(w2[e], s2[e], bits, weight_format)
        rows = by_expert[e]
        # every (token, slot) routed to e at once: token activations as the columns
        X = x[[tokens[ti] for ti, _ in rows]].T
        O = expert_ffn(X, W13, W2).T
        for r, (ti, j) in enumerate(rows):
            out[ti, j] = O[r]

    y = np.zeros((len(tokens), H))
    wsel = np.asarray(w, dtype=np.float32).astype(np.float64)[tokens]
    for j in range(k):
        y += wsel[:, j:j + 1] * out[:, j]
    if shared is not None:
        S13 = dequantize(shared["w13"], shared["s13"], shared["bits"]).astype(np.float64)
        S2 = dequantize(shared["w2"], shared["s2"], shared["bits"]).astype(np.float64)
        ys = expert_ffn(x[tokens].T, S13, S2).T
        if shared_gate is not None:
            ys = np.asarray(shared_gate, dtype=np.float64)[tokens][:, None] * ys
        y += ys
    if residual_bits is not None:
        y += f32_from_bf16_bits(residual_bits).astype(np.float64)[tokens]
    return y


def moe_layer(x_bits, logits, k: int, w13, s13, w2, s2, bits: int, tokens=None,
              shared=None, residual_bits=None, shared_gate=None, weight_format: str = "int"):
    """Routing followed by the routed sum: ``(y fp64, route outputs)``."""
    r = route(logits, k)
    y = moe_ffn(x_bits, r[0], r[1], w13, s13, w2, s2, bits, tokens=tokens,
                shared=shared, residual_bits=residual_bits, shared_gate=shared_gate,
                weight_format=weight_format)
    return y, r


# ---------------------------------------------------------------------------
# Dense projections (the non-expert INT8 matrices of the recipe)
# ---------------------------------------------------------------------------

def linear(x_bits, packed, scales, bits: int, residual_bits=None, weight_format: str = "int"):
    """``y = x . W_hat^T (+ residual)``, fp64, for a quantized ``[N, K]`` matrix.

    Page "Nex-N2.5-mini Int4-Int8Mix", Recipe table: the attention q/k/v/o
    projections and the Gated DeltaNet in_proj_qkv, in_proj_z and out_proj are
    INT8, symmetric, group 128.  ``x_bits`` uint16 bf16 ``[T, K]``; ``packed`` /
    ``scales`` as :func:`quantize_pack` (or the other formats, see
    :func:`dequantize_as`).  Returns fp64 ``[T, N]``.
    """
    x = f32_from_bf16_bits(x_bits).astype(np.float64)
    W = dequantize_as(packed, scales, bits, weight_format)
    y = x @ W.T
    if residual_bits is not None:
        y = y + f32_from_bf16_bits(residual_bits).astype(np.float64)
    return y
