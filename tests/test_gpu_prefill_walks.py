"""GPU parity of the large-batch (prefill) grouped GEMMs where workgroups walk several
items, compared with the oracle on EVERY output row.

The prefill kernels are persistent: each workgroup walks a list of items (128 sorted rows
of one expert by one N block) as one pipelined stream of K steps.  Everything that
happens at an item switch (the next item's tokens copied one item ahead, the epilogue
deferred past the next step's barrier, the per-item load set-up) only runs when a
workgroup owns two or more items.  The shapes below are chosen so that it does, for
4-bit and 8-bit routed codes, with and without a shared expert of either width, and with
ragged last tiles (random routing) as well as exact-multiple, single-row and empty
experts (caller-given ids).  ``walks()`` models the launch's item assignment on the host
(one workgroup per CU, at least 256, items dealt in XCD-contiguous ranges) and each test
asserts the walk lengths it relies on.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_int4_rtn_amd as w4
from gpu_util import DEV, OracleExperts, bf16_to_dev, check_ffn, f32_to_dev, gpu_layer, say

pytestmark = pytest.mark.gpu

MT, NT, MAX_ITEMS = 128, 256, 32


def _grid(max_items):
    g = max(256, (max_items + 8 + MAX_ITEMS - 1) // MAX_ITEMS)
    g = min(g, max(max_items, 8))
    return (g + 7) // 8 * 8


def _walk_lengths(total, grid):
    """Items each workgroup of `grid` takes out of `total` (XCD-contiguous dealing)."""
    C = (total + 7) // 8
    n = np.zeros(grid, dtype=np.int64)
    for b in range(grid):
        for tid in range(MAX_ITEMS):
            w = b + tid * grid
            if w < 8 * C and (w & 7) * C + (w >> 3) < total:
                n[b] += 1
    return n


def walks(counts, T, k, E, H, I, shared_I=0):
    """(gate/up walk lengths, down walk lengths) of the routed and shared streams."""
    P = T * k
    max_tiles = (P + MT - 1) // MT + min(E, P)
    tiles = int(sum((c + MT - 1) // MT for c in counts))
    s_tiles = (T + MT - 1) // MT if shared_I else 0
    nb_gk, nb_dk = I // 128, (H + NT - 1) // NT
    nbs = shared_I // 128
    g_gk = _grid(max(max_tiles * nb_gk, s_tiles * nbs))
    g_dk = _grid(max(max_tiles, s_tiles) * nb_dk)
    out = dict(gk=_walk_lengths(tiles * nb_gk, g_gk), dk=_walk_lengths(tiles * nb_dk, g_dk))
    if shared_I:
        out["gk_shared"] = _walk_lengths(s_tiles * nbs, g_gk)
        out["dk_shared"] = _walk_lengths(s_tiles * nb_dk, g_dk)
    return out


def _layer(E, H, I, bits, seed_group):
    return gpu_layer(seed_group, 0, E, H, I, bits), OracleExperts(seed_group, 0, H, I, bits)


def _run_and_check(T, E, H, I, k, bits, shared_bits, shared_I, seed_group, ids=None, wts=None, need=None):
    (w13, s13, w2, s2), ref = _layer(E, H, I, bits, seed_group)
    sh_gpu = sh_ref = None
    if shared_bits:
        sh_gpu = gpu_layer(seed_group, 0, 1, H, shared_I, shared_bits, shared=True)
        sh_ref = OracleExperts(seed_group, 0, H, shared_I, shared_bits, shared=True).shared_dict()
    x = synth.activations_bf16(700 + seed_group, T, H)
    res = synth.activations_bf16(701 + seed_group, T, H)
    if ids is None:
        logits = synth.router_logits(700 + seed_group, T, E)
        ids_ref, w_ref, counts, *_ = oracle.route(logits, k)
        kw = dict(router_logits=f32_to_dev(logits))
    else:
        ids_ref, w_ref = ids, wts
        counts = np.bincount(ids.ravel(), minlength=E)
        kw = dict(topk_ids=torch.from_numpy(ids).to(DEV), topk_w=f32_to_dev(wts))
    wl = walks(counts, T, k, E, H, I, shared_I if shared_bits else 0)
    say(f"  walks: " + ", ".join(f"{n} max {v.max()} mean {v.mean():.2f}" for n, v in wl.items()))
    for name, at_least in (need or {}).items():
        assert wl[name].max() >= at_least, (name, wl[name].max())
    y, r = w4.moe_w4a16_forward(bf16_to_dev(x), w13, s13, w2, s2, top_k=k, bits=bits, shared=sh_gpu,
                                residual=bf16_to_dev(res), routing_out=True, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(r["counts"].cpu().numpy(), counts)
    y_ref = oracle.moe_ffn(x, ids_ref, w_ref, *ref.as_args(), bits, shared=sh_ref, residual_bits=res)
    check_ffn(y, y_ref, f"T={T} E={E} H={H} I={I} k={k} bits={bits} shared={shared_bits}")
    # and without the residual, so the expert terms are not hidden under it
    y0 = w4.moe_w4a16_forward(bf16_to_dev(x), w13, s13, w2, s2, top_k=k, bits=bits, shared=sh_gpu, **kw)
    torch.cuda.synchronize()
    y0_ref = oracle.moe_ffn(x, ids_ref, w_ref, *ref.as_args(), bits, shared=sh_ref)
    check_ffn(y0, y0_ref, "  (no residual)")


# (T, E, H, I, k, bits, shared_bits, shared_I, walk lengths asserted)
CASES = [
    # 8 N blocks along I and 4 along H: long walks in both GEMMs, K = 1024 for down
    (4096, 32, 1024, 1024, 8, 4, 0, 0, {"gk": 6, "dk": 3}),
    (4096, 32, 1024, 1024, 8, 8, 8, 1024, {"gk": 6, "dk": 3}),
    # 4 N blocks per tile for both GEMMs: 2-3 items per workgroup
    (2048, 32, 1024, 512, 8, 8, 0, 0, {"gk": 2, "dk": 2}),
    # 24 experts at k = 6, H = 512: ragged walks next to 4-bit and 8-bit shared streams
    (1536, 24, 512, 1024, 6, 4, 4, 1024, {"gk": 3}),
    (1536, 24, 512, 1024, 6, 8, 4, 1024, {"gk": 3}),
    # 8192 tokens over 8 experts with a shared expert: the shared stream itself walks
    # several items in both GEMMs
    (8192, 8, 2048, 256, 2, 4, 8, 1024, {"dk": 3, "gk_shared": 2, "dk_shared": 2}),
]


@pytest.mark.parametrize("T,E,H,I,k,bits,shared_bits,shared_I,need", CASES)
def test_prefill_multi_item_walks_all_rows(T, E, H, I, k, bits, shared_bits, shared_I, need):
    say(f"prefill walks T={T} E={E} H={H} I={I} k={k} bits={bits} shared={shared_bits}/{shared_I}")
    _run_and_check(T, E, H, I, k, bits, shared_bits, shared_I, seed_group=20 + T % 97 + bits + shared_bits,
                   need=need)


def _ids_with_counts(counts, T, k, seed):
    """Caller-given ids with exactly `counts` pairs per expert: the pairs sorted by expert
    are dealt to tokens round-robin, so an expert never repeats within a token."""
    counts = np.asarray(counts)
    assert counts.sum() == T * k and counts.max() <= T
    labels = np.repeat(np.arange(len(counts)), counts)
    ids = np.empty((T, k), dtype=np.int32)
    for i, e in enumerate(labels):
        ids[i % T, i // T] = e
    rng = np.random.default_rng(seed)
    for t in range(T):   # slot order inside a token does not matter to the counts
        ids[t] = ids[t, rng.permutation(k)]
    wts = rng.random((T, k)).astype(np.float32)
    return ids, wts


@pytest.mark.parametrize("bits,shared_bits", [(4, 8), (8, 8), (4, 0)])
def test_prefill_exact_single_and_empty_experts(bits, shared_bits):
    """Experts with 512 (four full tiles), 1, 0, 129, 127, 128, 256 and 383 rows next to
    ordinary ones: full, single-row and ragged last tiles in one walk."""
    T, E, H, I, k = 1024, 16, 512, 1024, 4
    counts = [512, 1, 0, 129, 127, 128, 256, 383] + [320] * 8
    ids, wts = _ids_with_counts(counts, T, k, seed=bits * 10 + shared_bits)
    say(f"prefill structured counts bits={bits} shared={shared_bits}")
    _run_and_check(T, E, H, I, k, bits, shared_bits, 512, seed_group=90 + bits + shared_bits, ids=ids, wts=wts,
                   need={"gk": 1})


def test_walk_model_matches_the_launch_rule():
    """The host model above, on the full 8192-token layer: every gate/up and down workgroup
    of the 256-wide grid takes 8 to 10 items."""
    counts = oracle.route(synth.router_logits(3, 8192, 256), 8)[2]
    wl = walks(counts, 8192, 8, 256, 2048, 512)
    assert wl["gk"].min() >= 8 and wl["dk"].min() >= 8
