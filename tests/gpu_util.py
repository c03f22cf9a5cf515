"""Shared helpers of the GPU parity tests: device transfer, seeded layers, and the
acceptance check on FFN outputs.

Tolerance (the acceptance rule of this path): over a whole output tensor,
``max|y - y_ref| <= 2e-2 * max|y_ref|`` and ``sum|y - y_ref| / sum|y_ref| <= 5e-3``,
with ``y_ref`` the fp64 oracle before any rounding.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth

DEV = torch.device("cuda:0")
MAX_REL = 2e-2
MEAN_REL = 5e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def bf16_from_dev(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32_to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def check_ffn(y_gpu: torch.Tensor, y_ref: np.ndarray, what: str = ""):
    y = oracle.f32_from_bf16_bits(bf16_from_dev(y_gpu)).astype(np.float64)
    assert y.shape == y_ref.shape, (y.shape, y_ref.shape)
    assert np.all(np.isfinite(y)), what
    err = np.abs(y - y_ref)
    scale = np.abs(y_ref).max()
    max_rel = err.max() / scale
    mean_rel = err.sum() / np.abs(y_ref).sum()
    say(f"  {what}: max|d|/max|ref| = {max_rel:.3e}, sum|d|/sum|ref| = {mean_rel:.3e}")
    assert max_rel <= MAX_REL, (what, max_rel)
    assert mean_rel <= MEAN_REL, (what, mean_rel)
    return max_rel, mean_rel


class OracleExperts:
    """The oracle's own packed experts, regenerated from the seeds on demand."""

    def __init__(self, group, layer, H, I, bits, shared=False):
        self.args = (group, layer, H, I, bits, shared)
        self.cache = {}

    def get(self, e):
        if e not in self.cache:
            group, layer, H, I, bits, shared = self.args
            p13, s13 = oracle.quantize_pack(synth.expert_w13(group, layer, e, H, I, shared=shared), bits)
            p2, s2 = oracle.quantize_pack(synth.expert_w2(group, layer, e, H, I, shared=shared), bits)
            self.cache[e] = (p13, s13, p2, s2)
        return self.cache[e]

    def prefetch(self, experts, threads=8):
        """Quantize these experts ahead, on a thread pool (NumPy releases the GIL)."""
        from concurrent.futures import ThreadPoolExecutor
        todo = [int(e) for e in experts if int(e) not in self.cache]
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(self.get, todo))

    def view(self, i):
        parent = self

        class _V:
            def __getitem__(self, e):
                return parent.get(int(e))[i]
        return _V()

    def as_args(self):
        return self.view(0), self.view(1), self.view(2), self.view(3)

    def shared_dict(self):
        p13, s13, p2, s2 = self.get(0)
        return dict(w13=p13, s13=s13, w2=p2, s2=s2, bits=self.args[4])


def gpu_layer(group, layer, E, H, I, bits, shared=False):
    """All experts of a layer generated from the seeds and quantized on the GPU by the
    library (fp32 weights are uploaded one expert at a time)."""
    import weight_only_int4_rtn_amd as w4
    n = 1 if shared else E
    w13 = torch.empty((n, 2 * I, H * bits // 32), dtype=torch.int32, device=DEV)
    s13 = torch.empty((n, 2 * I, H // 128), dtype=torch.bfloat16, device=DEV)
    w2 = torch.empty((n, H, I * bits // 32), dtype=torch.int32, device=DEV)
    s2 = torch.empty((n, H, I // 128), dtype=torch.bfloat16, device=DEV)
    chunk = 16
    for e0 in range(0, n, chunk):
        es = range(e0, min(n, e0 + chunk))
        f13 = f32_to_dev(np.stack([synth.expert_w13(group, layer, e, H, I, shared=shared) for e in es]))
        f2 = f32_to_dev(np.stack([synth.expert_w2(group, layer, e, H, I, shared=shared) for e in es]))
        w4.rtn_quantize_pack(f13, bits, packed=w13[e0:e0 + len(es)], scales=s13[e0:e0 + len(es)])
        w4.rtn_quantize_pack(f2, bits, packed=w2[e0:e0 + len(es)], scales=s2[e0:e0 + len(es)])
    torch.cuda.synchronize()
    if shared:
        return dict(w13=w13[0], s13=s13[0], w2=w2[0], s2=s2[0], bits=bits)
    return w13, s13, w2, s2
