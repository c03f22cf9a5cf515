"""Seeded synthetic inputs for the W4A16 routed-expert path.

Shared by the tests, the smoke check and the benchmark.  This module holds no
quantization, routing or MLP arithmetic: it only draws random numbers.

Distributions (page "Nex-N2.5-mini Int4-Int8Mix", Recipe; the layer shape of
page "Nex-N2.5-mini — MQ4R quant for hipfire", architecture paragraph):

* expert weights: N(0, 0.02) fp32, one ``[out, in]`` matrix per projection;
* activations:   N(0, 1) fp32 rounded to bf16 (returned as uint16 bit patterns);
* router logits: N(0, 1) fp32, independent per (layer, token, iteration).

Seeds are tuples fed to ``numpy.random.default_rng``:

* weights ``(2026, group, layer, expert, tensor)`` with tensor 0 = gate,
  1 = up, 2 = down, 3/4/5 = shared gate/up/down, so one expert can be
  regenerated without the rest of the layer; 6 = the router ``[E, H]`` and
  7 = the shared-expert gate ``[H]`` (expert 0), both N(0, 1/H) so that the
  logits of N(0, 1) activations are about N(0, 1), rounded to bf16;
* activations ``(2026, cfg, 10)``;
* logits ``(2026, cfg, 11, layer, iteration)``.

``device_*`` helpers draw the same distributions directly on a torch device
(a different stream of numbers, used where only the distribution matters, such
as filling benchmark layers quickly).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED = 2026
WEIGHT_STD = 0.02

GATE, UP, DOWN, SHARED_GATE, SHARED_UP, SHARED_DOWN, ROUTER, SHARED_GATE_W = range(8)


@dataclass(frozen=True)
class LayerConfig:
    """Shape of one MoE layer and its token batch."""
    name: str
    E: int
    k: int
    H: int
    I: int
    T: int
    group: int          # weight seed group
    layers: int = 1
    int8_layers: tuple = field(default_factory=tuple)
    shared_I: int = 0   # 0: no shared expert


# Tiny layer, single-token decode, 32-token decode, 8192-token prefill chunk,
# and a 40-layer decode stack at batch 4 with an INT8 shared expert per layer
# and INT8 routed experts on layers 7, 13, 18, 23, 29 and 35 (page
# "primitive-ai/Nex-N2.5-mini-mixed-NVFP4-FP8", How the six layers were chosen).
CONFIGS = {
    "tiny": LayerConfig("tiny", E=8, k=2, H=256, I=128, T=4, group=0),
    "decode1": LayerConfig("decode1", E=256, k=8, H=2048, I=512, T=1, group=1),
    "decode32": LayerConfig("decode32", E=256, k=8, H=2048, I=512, T=32, group=1),
    "prefill8192": LayerConfig("prefill8192", E=256, k=8, H=2048, I=512, T=8192, group=1),
    "stack40": LayerConfig("stack40", E=256, k=8, H=2048, I=512, T=4, group=4, layers=40,
                           int8_layers=(7, 13, 18, 23, 29, 35), shared_I=512),
}
CONFIG_INDEX = {"tiny": 0, "decode1": 1, "decode32": 2, "prefill8192": 3, "stack40": 4}


def _normal(seed, shape, std=1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def expert_weight(group: int, layer: int, expert: int, tensor: int, rows: int, cols: int) -> np.ndarray:
    """One fp32 ``[rows, cols]`` projection, N(0, 0.02)."""
    return _normal((SEED, group, layer, expert, tensor), (rows, cols), WEIGHT_STD)


def expert_w13(group: int, layer: int, expert: int, H: int, I: int, shared: bool = False) -> np.ndarray:
    """Fused ``[2I, H]`` gate/up bank of one expert: gate rows, then up rows."""
    tg, tu = (SHARED_GATE, SHARED_UP) if shared else (GATE, UP)
    return np.concatenate([expert_weight(group, layer, expert, tg, I, H),
                           expert_weight(group, layer, expert, tu, I, H)], axis=0)


def expert_w2(group: int, layer: int, expert: int, H: int, I: int, shared: bool = False) -> np.ndarray:
    """Down projection ``[H, I]`` of one expert."""
    return expert_weight(group, layer, expert, SHARED_DOWN if shared else DOWN, H, I)


def layer_weights(group: int, layer: int, E: int, H: int, I: int):
    """All experts of one layer: ``(w13 [E, 2I, H], w2 [E, H, I])`` fp32."""
    w13 = np.stack([expert_w13(group, layer, e, H, I) for e in range(E)])
    w2 = np.stack([expert_w2(group, layer, e, H, I) for e in range(E)])
    return w13, w2


def _bf16_bits(a: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def router_weight_bf16(group: int, layer: int, E: int, H: int) -> np.ndarray:
    """Router ``[E, H]``, N(0, 1/H) fp32 rounded to bf16 (uint16 bit patterns)."""
    return _bf16_bits(_normal((SEED, group, layer, 0, ROUTER), (E, H), float(H) ** -0.5))


def shared_gate_weight_bf16(group: int, layer: int, H: int) -> np.ndarray:
    """Shared-expert gate ``[H]``, N(0, 1/H) fp32 rounded to bf16 (uint16 bit patterns)."""
    return _bf16_bits(_normal((SEED, group, layer, 0, SHARED_GATE_W), (H,), float(H) ** -0.5))


def activations_f32(cfg: int, T: int, H: int, stream: int = 10) -> np.ndarray:
    """N(0, 1) fp32 ``[T, H]`` before rounding to bf16."""
    return _normal((SEED, cfg, stream), (T, H))


def activations_bf16(cfg: int, T: int, H: int, stream: int = 10) -> np.ndarray:
    """N(0, 1) activations rounded to bf16 by torch; uint16 bit patterns ``[T, H]``."""
    import torch
    x = torch.from_numpy(activations_f32(cfg, T, H, stream))
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def router_logits(cfg: int, T: int, E: int, layer: int = 0, iteration: int = 0) -> np.ndarray:
    """N(0, 1) fp32 router logits ``[T, E]``."""
    return _normal((SEED, cfg, 11, layer, iteration), (T, E))


def device_normal(shape, std: float, seed: int, device, dtype=None):
    """N(0, std) fp32 tensor drawn on ``device`` with a seeded torch generator."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t if dtype is None else t.to(dtype)
