"""Plain NumPy oracle of the two other expert weight formats the pages evaluate.

TEST INFRASTRUCTURE ONLY, like the rest of this package: imported by the tests,
the smoke check and the benchmark's CPU-baseline leg, never by the library.

* FP8 E4M3 with one scale per output channel (page "Nex-N2.5-mini-mixed-NVFP4-FP8",
  What's quantized to what: the six sensitive layers' routed experts, FP8 E4M3 per
  output channel; weights-only round-to-nearest, no calibration).
* MXFP4: E2M1 codes with one power-of-two (E8M0) scale per block of 32 input
  columns (page "Nex-N2.5-mini-MXFP4-MxWave", Model summary: MXFP4 W4A16 for the
  routed experts; Quantization method: per-block scale-exponent search by weight
  MSE; its Evaluation tables also compare the plain round-to-nearest scale).

Every integer decision (a code, an exponent, the chosen MSE candidate) is taken
with exact or fully specified arithmetic, so a second implementation can match
it bit for bit: exponents come from the binary exponent of a float (frexp), not
from a rounded logarithm; the MSE of a candidate is summed in fp64 in a fixed
pairwise order over the 32 elements of a block (element i with i + 16, then
i + 8, i + 4, i + 2, i + 1).
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# FP8 E4M3 (OCP): 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinity;
# S.1111.111 is NaN; the largest finite magnitude is 1.75 * 2^8 = 448; the
# smallest subnormal 2^-9.
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code byte, fp64 (NaN for the NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 15
    M = c & 7
    mag = np.where(E == 0, M / 8.0 * 2.0 ** -6, (1.0 + M / 8.0) * np.exp2(E - 7.0))
    mag = np.where((E == 15) & (M == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(r) -> np.ndarray:
    """Round fp32 values to E4M3, to nearest with ties to even, saturating at +-448.

    For |r| >= 2^-6 (normal range) the 3-bit mantissa of r is rounded; below it the
    value is rounded to a multiple of 2^-9 (subnormals).  Rounding is exact integer
    arithmetic on the fp32 bit pattern.  The sign bit is r's sign bit.
    """
    r = np.ascontiguousarray(r, dtype=np.float32)
    u = r.view(np.uint32).astype(np.int64)
    sign = (u >> 31) & 1
    a = u & 0x7FFFFFFF                       # |r| bits
    exp = (a >> 23) - 127                    # unbiased exponent (normal r)
    # value as an integer multiple of 2^-9 (subnormal grid) or of 2^(exp-3) (normal grid):
    # keep 3 fraction bits of the mantissa, round the dropped ones to nearest even
    mant = (a & 0x7FFFFF) | 0x800000         # 24-bit significand of a normal fp32
    normal = exp >= -6
    # normal: drop 20 bits; subnormal: shift so that the unit is 2^-9
    drop = np.where(normal, 20, 20 + (-6 - exp))
    drop = np.minimum(drop, 40)
    q = mant >> drop
    rem = mant - (q << drop)
    half = np.int64(1) << (drop - 1)
    up = (rem > half) | ((rem == half) & ((q & 1) == 1))
    q = q + up
    # normal: q in [8, 16]; 16 means the next binade
    E = np.where(normal, exp + 7, 0)
    M = np.where(normal, q - 8, q)           # subnormal: q in [0, 8]; 8 is 2^-6 (E=1, M=0)
    carry = normal & (q == 16)
    E = np.where(carry, E + 1, E)
    M = np.where(carry, 0, M)
    sub_carry = (~normal) & (q == 8)
    E = np.where(sub_carry, 1, E)
    M = np.where(sub_carry, 0, M)
    zero = a == 0
    E = np.where(zero, 0, E)
    M = np.where(zero, 0, M)
    # saturate: anything above 448 (E=15, M=6), including rounding up to the NaN pattern
    over = (E > 15) | ((E == 15) & (M == 7))
    E = np.where(over, 15, E)
    M = np.where(over, 6, M)
    return ((sign << 7) | (E << 3) | M).astype(np.uint8)


def fp8_quantize(w):
    """Per-output-channel FP8 E4M3 round-to-nearest of ``w[..., rows, cols]``.

    For every row (output channel): ``a = max |w|``; ``s = a / 448`` (IEEE fp32
    division, kept as the fp32 scale); ``q = E4M3_rne(w / s)`` (IEEE fp32 division,
    saturating at 448); an all-zero row has ``s = 0`` and every code 0.
    Returns ``(codes uint8 like w, scales fp32 [..., rows])``.
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    a = np.max(np.abs(w), axis=-1)
    s = (a / np.float32(E4M3_MAX)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (w / s[..., None]).astype(np.float32)
    r = np.where(s[..., None] == 0, np.float32(0), r)
    return e4m3_encode(r), s


def fp8_pack(codes) -> np.ndarray:
    """Four codes per int32 word, column c at byte c % 4 (lowest column lowest)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    if c.shape[-1] % 4:
        raise ValueError("cols must be a multiple of 4")
    return c.view(np.int32)


def fp8_quantize_pack(w):
    """``(packed int32 [..., rows, cols/4], scales fp32 [..., rows])``."""
    codes, s = fp8_quantize(w)
    return fp8_pack(codes), s


def fp8_dequantize(packed, scales) -> np.ndarray:
    """``W_hat = q * s`` in fp64 (exact: 4 significant bits times an fp32 scale)."""
    p = np.ascontiguousarray(packed, dtype=np.int32)
    codes = p.view(np.uint8).reshape(*p.shape[:-1], p.shape[-1] * 4)
    return e4m3_decode(codes) * np.asarray(scales, dtype=np.float32).astype(np.float64)[..., None]


# ---------------------------------------------------------------------------
# MXFP4: E2M1 elements (1 sign, 2 exponent, 1 mantissa bit: 0, 0.5, 1, 1.5, 2, 3,
# 4, 6) sharing one E8M0 scale 2^(code - 127) per block of 32 columns.
# ---------------------------------------------------------------------------

MX_BLOCK = 32
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(nibbles) -> np.ndarray:
    n = np.asarray(nibbles).astype(np.int64)
    return np.where(n & 8, -1.0, 1.0) * E2M1_VALUES[n & 7]


def e2m1_encode(r) -> np.ndarray:
    """Round values (exact in fp64) to E2M1, nearest with ties to the even code,
    saturating at +-6; the sign bit is r's sign bit."""
    r = np.asarray(r, dtype=np.float64)
    sign = np.signbit(r).astype(np.int64)
    a = np.abs(r)
    # grid points and the code of each; a tie goes to the even code (mantissa bit 0)
    codes = np.zeros(a.shape, dtype=np.int64)
    for c in range(1, 8):
        lo, hi = E2M1_VALUES[c - 1], E2M1_VALUES[c]
        mid = (lo + hi) / 2
        take = (a > mid) | ((a == mid) & (c % 2 == 0))
        codes = np.where(take, c, codes)
    return (sign << 3) | codes


def _floor_log2(y):
    """floor(log2 y) of positive finite fp64 values, from the binary exponent."""
    _, e = np.frexp(y)
    return e.astype(np.int64) - 1


def _p995(absblocks):
    """The 99.5th percentile of each block's 32 values |w|, by linear interpolation between
    order statistics: position 0.995 * 31 = 30.845, so p = a + (b - a) * 0.845 with a, b the
    31st and 32nd smallest (fp64, the product rounded before the sum)."""
    srt = np.sort(absblocks.astype(np.float64), axis=-1)
    a, b = srt[..., MX_BLOCK - 2], srt[..., MX_BLOCK - 1]
    return a + (b - a) * 0.845


def _block_sse(v, e):
    """Sum over a block of (v - dequant(quant(v / 2^e)) * 2^e)^2 in fp64, pairwise in the
    fixed order i + 16, i + 8, i + 4, i + 2, i + 1."""
    scale = np.exp2(e.astype(np.float64))[..., None]
    rec = e2m1_decode(e2m1_encode(v / scale)) * scale
    d = v - rec
    s = d * d
    for half in (16, 8, 4, 2, 1):
        s = s[..., :half] + s[..., half:2 * half]
    return s[..., 0]


def mxfp4_exponents(w, method: str = "mse") -> np.ndarray:
    """Shared exponent of every block of 32 columns of ``w[..., rows, cols]``.

    ``rtn``: the round-to-nearest scale of the OCP MX format, ``floor(log2 amax) - 2``
    (2 = the largest E2M1 exponent).
    ``mse``: the page's search: the candidates ``floor(log2(p99.5 / 6)) - 4`` through
    ``floor(log2(p99.5 / 6)) + 1`` plus the smallest exponent that avoids clipping
    (``amax / 2^e <= 6``), the one with the lowest squared weight error winning (equal
    errors: the smallest exponent).  An all-zero block gets -127.  Exponents are kept in
    the E8M0 range [-127, 127].
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    cols = w.shape[-1]
    if cols % MX_BLOCK:
        raise ValueError("cols must be a multiple of 32")
    v = w.reshape(*w.shape[:-1], cols // MX_BLOCK, MX_BLOCK).astype(np.float64)
    amax = np.max(np.abs(v), axis=-1)
    zero = amax == 0
    safe = np.where(zero, 1.0, amax)
    E = _floor_log2(safe)
    if method == "rtn":
        e = E - 2
    elif method == "mse":
        m, _ = np.frexp(safe)                       # safe = m * 2^(E + 1), m in [0.5, 1)
        e_nc = np.where(2 * m <= 1.5, E - 2, E - 1)  # smallest e with amax <= 6 * 2^e
        p = _p995(np.abs(v))
        e0 = _floor_log2(np.where(zero, 6.0, p) / 6.0)
        cands = [e0 + d for d in range(-4, 2)] + [e_nc]
        cands = np.stack([np.clip(c, -127, 127) for c in cands], axis=-1)
        cands = np.sort(cands, axis=-1)             # ascending: ties go to the smallest
        best_e = cands[..., 0]
        best = _block_sse(v, best_e)
        for j in range(1, cands.shape[-1]):
            c = cands[..., j]
            err = _block_sse(v, c)
            better = err < best
            best = np.where(better, err, best)
            best_e = np.where(better, c, best_e)
        e = best_e
    else:
        raise ValueError("method must be 'rtn' or 'mse'")
    return np.where(zero, -127, np.clip(e, -127, 127)).astype(np.int64)


def mxfp4_quantize(w, method: str = "mse"):
    """``(nibbles int64 like w, scale codes uint8 [..., rows, cols/32])``: each element
    is ``E2M1_rne(w / 2^e)`` of its block's exponent e; the scale code is e + 127."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    e = mxfp4_exponents(w, method)
    v = w.reshape(*w.shape[:-1], w.shape[-1] // MX_BLOCK, MX_BLOCK).astype(np.float64)
    nib = e2m1_encode(v / np.exp2(e.astype(np.float64))[..., None]).reshape(w.shape)
    return nib, (e + 127).astype(np.uint8)


def mxfp4_pack(nibbles) -> np.ndarray:
    """Eight nibbles per int32 word, column c at bits 4 * (c % 8) (lowest column lowest)."""
    n = np.asarray(nibbles).astype(np.uint32)
    n = n.reshape(*n.shape[:-1], n.shape[-1] // 8, 8)
    word = np.zeros(n.shape[:-1], dtype=np.uint32)
    for i in range(8):
        word |= n[..., i] << np.uint32(4 * i)
    return word.view(np.int32)


def mxfp4_quantize_pack(w, method: str = "mse"):
    """``(packed int32 [..., rows, cols/8], scale codes uint8 [..., rows, cols/32])``."""
    nib, sc = mxfp4_quantize(w, method)
    return mxfp4_pack(nib), sc


def mxfp4_dequantize(packed, scale_codes) -> np.ndarray:
    """``W_hat = E2M1(nibble) * 2^(code - 127)``, fp64 (exact)."""
    p = np.ascontiguousarray(packed).view(np.uint32)
    nib = np.stack([(p >> np.uint32(4 * i)) & np.uint32(15) for i in range(8)], axis=-1)
    nib = nib.reshape(*p.shape[:-1], p.shape[-1] * 8)
    vals = e2m1_decode(nib)
    sc = np.exp2(np.asarray(scale_codes).astype(np.float64) - 127.0)
    return (vals.reshape(*vals.shape[:-1], vals.shape[-1] // MX_BLOCK, MX_BLOCK) * sc[..., None]).reshape(vals.shape)
