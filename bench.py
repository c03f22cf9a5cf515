#!/usr/bin/env python3
"""Benchmark of the W4A16 routed-expert MoE path on one MI355X.

One step is one full forward of the hot path over one batch: routing (top-k,
renormalised softmax, expert histogram, permutation), the fused dequant gate/up
projection with SiLU(gate)*up, and the fused dequant down projection with the
router-weighted un-permute.  Inputs (packed weights, activations, logits) are
resident in HBM before the timed region starts.

The headline workload is single-token decode of one full layer (256 experts, top-8,
hidden 2048, intermediate 512, INT4 group-128 weights).  The 32-token decode batch
and the 8192-token prefill chunk are measured the same way and reported in the same
JSON line.  Decode runs rotate through several independently drawn copies of the
layer and through a bank of router logits, so that the experts a step touches are
not left in the 256 MB Infinity Cache by earlier steps.

Per-kernel durations come from HIP events recorded on the library's stream around
every kernel (``moe_w4a16_forward_timed``) over a second pass of the same steps.

Prints exactly one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "decode tok/s + expert-weight HBM GB/s (bs1/32); prefill TFLOP/s at 8192 tok"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
E, K, H, I = 256, 8, 2048, 512


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def expert_bytes(bits=4):
    """Algorithmic bytes of one expert: packed codes plus bf16 group scales."""
    gate_up = 2 * I * H * bits // 8 + 2 * I * (H // 128) * 2
    down = H * I * bits // 8 + H * (I // 128) * 2
    return gate_up, down


def make_layers(n_copies, seed, bits=4):
    """n_copies independently drawn layers, quantized on the GPU by the library."""
    import torch
    import synth
    import weight_only_int4_rtn_amd as w4
    dev = torch.device("cuda:0")
    layers = []
    chunk = 32
    for c in range(n_copies):
        w13 = torch.empty((E, 2 * I, H * bits // 32), dtype=torch.int32, device=dev)
        s13 = torch.empty((E, 2 * I, H // 128), dtype=torch.bfloat16, device=dev)
        w2 = torch.empty((E, H, I * bits // 32), dtype=torch.int32, device=dev)
        s2 = torch.empty((E, H, I // 128), dtype=torch.bfloat16, device=dev)
        for e0 in range(0, E, chunk):
            f13 = synth.device_normal((chunk, 2 * I, H), synth.WEIGHT_STD, seed * 1000 + c * 64 + e0 // chunk, dev)
            w4.rtn_quantize_pack(f13, bits, packed=w13[e0:e0 + chunk], scales=s13[e0:e0 + chunk])
            f2 = synth.device_normal((chunk, H, I), synth.WEIGHT_STD, seed * 1000 + c * 64 + 32 + e0 // chunk, dev)
            w4.rtn_quantize_pack(f2, bits, packed=w2[e0:e0 + chunk], scales=s2[e0:e0 + chunk])
            del f13, f2
        layers.append((w13, s13, w2, s2))
    torch.cuda.synchronize()
    return layers


def time_quantizer(bits=4):
    """Throughput of rtn_quantize_pack on one full gate/up bank (fp32 in)."""
    import torch
    import synth
    import weight_only_int4_rtn_amd as w4
    dev = torch.device("cuda:0")
    w = synth.device_normal((E, 2 * I, H), synth.WEIGHT_STD, 7, dev)
    packed = torch.empty((E, 2 * I, H * bits // 32), dtype=torch.int32, device=dev)
    scales = torch.empty((E, 2 * I, H // 128), dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        w4.rtn_quantize_pack(w, bits, packed=packed, scales=scales)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 10
    s.record()
    for _ in range(n):
        w4.rtn_quantize_pack(w, bits, packed=packed, scales=scales)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / n
    nbytes = w.numel() * 4 + packed.numel() * 4 + scales.numel() * 2
    del w
    return {"kernel": "quantize_pack_kernel", "weights": E * 2 * I * H, "ms": round(ms, 4),
            "GBps": round(nbytes / ms / 1e6, 1), "frac_hbm": round(nbytes / ms / 1e6 / HBM_PEAK_GBPS, 4)}


def measure(name, T, layers, steps, warmup, timed_steps, seed):
    """Times `steps` forwards of a T-token batch; returns a dict of results."""
    import torch
    import synth
    import weight_only_int4_rtn_amd as w4
    dev = torch.device("cuda:0")
    n_logits = 64
    logits = [synth.device_normal((T, E), 1.0, seed * 7919 + i, dev) for i in range(n_logits)]
    xs = [synth.device_normal((T, H), 1.0, seed * 104729 + i, dev, torch.bfloat16) for i in range(8)]
    ws = w4.new_workspace(w4.moe_w4a16_workspace_size(T, H, I, E, K), dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    distinct = [int(torch.topk(l, K, dim=1).indices.unique().numel()) for l in logits]
    n_copies = len(layers)
    calls = [w4.MoeCall(xs[0], *lay, top_k=K, workspace=ws) for lay in layers]

    def step(i):
        calls[i % n_copies](xs[i % 8], out, router_logits=logits[i % n_logits])

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        step(warmup + i)
    end.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    eager_ms = start.elapsed_time(end) / steps

    # the same steps replayed from a HIP graph (one graph holds a full rotation of n_logits
    # steps), which removes host launch cost as a decode loop does in serving
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(n_logits):
            step(i)
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, -(-steps // n_logits))
    start.record()
    for _ in range(reps):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    graph_ms = start.elapsed_time(end) / (reps * n_logits)
    del graph
    ms_per_step = graph_ms

    # per-kernel durations with HIP events around each kernel, same rotation
    per = {}
    for i in range(timed_steps):
        w13, s13, w2, s2 = layers[i % n_copies]
        _, tk = w4.moe_w4a16_forward_timed(xs[i % 8], w13, s13, w2, s2, top_k=K,
                                           router_logits=logits[i % n_logits], out=out, workspace=ws)
        for nm, ms in tk:
            per.setdefault(nm, []).append(ms)
    kernels = {nm: sum(v) / len(v) * 1e3 for nm, v in per.items()}   # average us per launch

    d_mean = sum(distinct[(warmup + i) % n_logits] for i in range(steps)) / steps
    gu, dn = expert_bytes()
    weight_bytes = d_mean * (gu + dn)
    flops = 2.0 * T * K * 3 * H * I
    res = {
        "T": T, "ms_per_step": ms_per_step, "eager_ms_per_step": eager_ms, "eager_wall_ms_per_step": wall_ms / steps,
        "tok_per_s": T / (ms_per_step / 1e3),
        "distinct_experts_mean": d_mean,
        "expert_weight_bytes_per_step": weight_bytes,
        "expert_weight_GBps": weight_bytes / (ms_per_step / 1e3) / 1e9,
        "TFLOPs": flops / (ms_per_step / 1e3) / 1e12,
        "kernels_us": {k: round(v, 2) for k, v in kernels.items()},
        "copies": n_copies,
    }
    # algorithmic bytes and flops of the two expert kernels, per launch
    act_in = T * H * 2
    a_bytes = T * K * I * 2
    res["kernel_bytes"] = {"gate_up": d_mean * gu + act_in + a_bytes, "down": d_mean * dn + a_bytes + T * H * 2}
    res["kernel_bytes"]["all"] = d_mean * (gu + dn) + act_in + T * E * 4 + T * H * 2
    res["kernel_flops"] = {"gate_up": 2.0 * T * K * 2 * I * H, "down": 2.0 * T * K * H * I}
    res["kernel_flops"]["all"] = res["kernel_flops"]["gate_up"] + res["kernel_flops"]["down"]
    log(f"[bench] {name}: {ms_per_step * 1e3:.1f} us/step (graph; eager {eager_ms * 1e3:.1f}, host wall "
        f"{wall_ms / steps * 1e3:.1f}), {res['tok_per_s']:.1f} tok/s, "
        f"{res['expert_weight_GBps']:.0f} GB/s expert weights, {res['TFLOPs']:.1f} TFLOP/s, kernels {res['kernels_us']}")
    del ws, out, logits, xs
    return res


KERNEL_SOURCES = {"tiny_decode": "moe_decode.hip", "gk_decode": "moe_decode.hip", "dk_decode": "moe_decode.hip",
                  "gk_pair_stream": "decode_stream.hip",
                  "gk_stream": "decode_stream.hip", "dk_stream": "decode_stream.hip",
                  "gk_prefill": "moe_prefill.hip", "dk_prefill": "moe_prefill.hip"}
KERNEL_HEADERS = ("common.h", "route_dev.h", "route_small.h", "dma.h", "decode_dev.h")
TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "hbm_traffic.txt")


def kernel_source_digest(kernel):
    """Digest of the code a kernel is built from (its .hip file and the shared headers), with
    comments and blank space removed so that a change to the text alone keeps the digest."""
    import hashlib
    import re
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "weight_only_int4_rtn_amd", "csrc")
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[kernel],) + KERNEL_HEADERS:
        with open(os.path.join(csrc, f)) as fh:
            code = re.sub(r"/\*.*?\*/", " ", fh.read(), flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE counter runs, each
    divided by what the same counter read per byte of a plain copy kernel.  None when no
    record exists or the kernel's sources changed since the counters were taken."""
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    for ln in lines:
        if not ln.startswith("kernel="):
            continue
        f = dict(kv.split("=", 1) for kv in ln.split())
        if f.get("kernel") != kernel or f.get("workload") != workload:
            continue
        if f.get("sha") != kernel_source_digest(kernel):
            return None
        return int(float(f["fetch_kib"]) * 1024 / float(f["fetch_factor"]) +
                   float(f["write_kib"]) * 1024 / float(f["write_factor"]))
    return None


def copy_calibration():
    """A plain copy kernel of known size (fp32 out = in * 1, 512 MiB each way) for scaling the
    FETCH_SIZE / WRITE_SIZE counters: run under the same counter collection as the bench."""
    import torch
    n = 128 << 20
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: MulFunctor kernel, {n * 4} bytes read and {n * 4} bytes written per launch")
    del src, dst


def roofline_for(res, bound, workload):
    """Roofline object of the dominant (longest) expert kernel of a measurement."""
    ks = res["kernels_us"]
    if "tiny_decode" in ks:   # one launch does the whole layer: its bytes are every expert kernel's
        name, key = "tiny_decode", "all"
    else:
        gk = next(k for k in ks if k.startswith("gk_"))
        dk = next(k for k in ks if k.startswith("dk_") and k != "dk_combine")
        name, key = (gk, "gate_up") if ks[gk] >= ks[dk] else (dk, "down")
    sec = ks[name] / 1e6
    traffic = measured_traffic(name, workload)
    if bound == "hbm":
        achieved = res["kernel_bytes"][key] / sec / 1e9
        return {"bound": "hbm", "kernel": name, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "bytes_per_launch": int(res["kernel_bytes"][key]), "us_per_launch": ks[name]}
    achieved = res["kernel_flops"][key] / sec / 1e12
    return {"bound": "mfma", "kernel": name, "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": traffic,
            "flops_per_launch": res["kernel_flops"][key], "bytes_per_launch": int(res["kernel_bytes"][key]),
            "us_per_launch": ks[name]}


def make_stack_layers(n_layers, int8_layers, seed):
    """Layers of the decode stack: routed experts (INT4, or INT8 on int8_layers) and one
    INT8 shared expert (2048 -> 512 -> 2048) per layer, quantized on the GPU."""
    import torch
    import synth
    import weight_only_int4_rtn_amd as w4
    dev = torch.device("cuda:0")
    out = []
    chunk = 32
    for l in range(n_layers):
        bits = 8 if l in int8_layers else 4
        w13 = torch.empty((E, 2 * I, H * bits // 32), dtype=torch.int32, device=dev)
        s13 = torch.empty((E, 2 * I, H // 128), dtype=torch.bfloat16, device=dev)
        w2 = torch.empty((E, H, I * bits // 32), dtype=torch.int32, device=dev)
        s2 = torch.empty((E, H, I // 128), dtype=torch.bfloat16, device=dev)
        base = seed * 100000 + l * 100
        for e0 in range(0, E, chunk):
            f13 = synth.device_normal((chunk, 2 * I, H), synth.WEIGHT_STD, base + e0 // chunk, dev)
            w4.rtn_quantize_pack(f13, bits, packed=w13[e0:e0 + chunk], scales=s13[e0:e0 + chunk])
            f2 = synth.device_normal((chunk, H, I), synth.WEIGHT_STD, base + 50 + e0 // chunk, dev)
            w4.rtn_quantize_pack(f2, bits, packed=w2[e0:e0 + chunk], scales=s2[e0:e0 + chunk])
            del f13, f2
        sp13, ss13 = w4.rtn_quantize_pack(synth.device_normal((2 * I, H), synth.WEIGHT_STD, base + 98, dev), 8)
        sp2, ss2 = w4.rtn_quantize_pack(synth.device_normal((H, I), synth.WEIGHT_STD, base + 99, dev), 8)
        out.append(dict(bits=bits, w=(w13, s13, w2, s2), shared=dict(w13=sp13, s13=ss13, w2=sp2, s2=ss2, bits=8)))
    torch.cuda.synchronize()
    return out


def measure_stack(T, layers, steps, warmup, seed):
    """A decode step through every layer of the stack: h <- h + routed(h) + shared(h)."""
    import torch
    import synth
    import weight_only_int4_rtn_amd as w4
    dev = torch.device("cuda:0")
    n_logits = 8
    L = len(layers)
    logits = [[synth.device_normal((T, E), 1.0, seed * 7919 + 1000 * l + i, dev) for i in range(n_logits)]
              for l in range(L)]
    ws = w4.new_workspace(w4.moe_w4a16_workspace_size(T, H, I, E, K, 8, I), dev)
    h0 = synth.device_normal((T, H), 1.0, seed, dev, torch.bfloat16)
    hb = [torch.empty_like(h0), torch.empty_like(h0)]
    distinct = [[int(torch.topk(g, K, dim=1).indices.unique().numel()) for g in row] for row in logits]
    calls = [w4.MoeCall(h0, *lay["w"], top_k=K, bits=lay["bits"], shared=lay["shared"], workspace=ws)
             for lay in layers]

    def step(i):
        cur = h0
        for l in range(L):
            nxt = hb[l & 1]
            calls[l](cur, nxt, router_logits=logits[l][i % n_logits], residual=cur)
            cur = nxt

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        step(warmup + i)
    end.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    eager_ms = start.elapsed_time(end) / steps
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(n_logits):
            step(i)
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, -(-steps // n_logits))
    start.record()
    for _ in range(reps):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / (reps * n_logits)
    del graph
    nbytes = 0.0
    for i in range(steps):
        for l, lay in enumerate(layers):
            gu, dn = expert_bytes(lay["bits"])
            nbytes += distinct[l][(warmup + i) % n_logits] * (gu + dn) + sum(expert_bytes(8))
    nbytes /= steps
    res = {"T": T, "layers": L, "ms_per_step": ms, "eager_ms_per_step": eager_ms,
           "eager_wall_ms_per_step": wall_ms / steps,
           "tok_per_s": T / (ms / 1e3), "weight_bytes_per_step": nbytes,
           "expert_weight_GBps": nbytes / (ms / 1e3) / 1e9}
    log(f"[bench] stack{L}: {ms * 1e3:.1f} us/step (graph; eager {eager_ms * 1e3:.1f}), {res['tok_per_s']:.1f} tok/s, "
        f"{res['expert_weight_GBps']:.0f} GB/s expert weights ({nbytes / 1e9:.2f} GB per step)")
    del ws
    return res


def cpu_baseline(seconds):
    """The oracle, as it stands, on single-token decode of the same layer shape."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        threads = 1
    n_tok = 8
    logits = synth.router_logits(1, n_tok, E)
    x = synth.activations_bf16(1, n_tok, H)
    ids, *_ = oracle.route(logits, K)
    packed = {}
    for e in sorted(set(ids.ravel().tolist())):
        p13, s13 = oracle.quantize_pack(synth.expert_w13(1, 0, e, H, I), 4)
        p2, s2 = oracle.quantize_pack(synth.expert_w2(1, 0, e, H, I), 4)
        packed[e] = (p13, s13, p2, s2)

    class View:
        def __init__(self, i):
            self.i = i

        def __getitem__(self, e):
            return packed[int(e)][self.i]

    views = [View(i) for i in range(4)]
    done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        t = done % n_tok
        oracle.moe_layer(x[t:t + 1], logits[t:t + 1], K, *views, 4)
        done += 1
    el = time.perf_counter() - t0
    return {"value": round(done / el, 3), "unit": "tok/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} single-token forwards of the 256-expert top-8 H=2048 I=512 INT4 layer "
                      f"(route + dequant + fp64 SwiGLU + weighted sum), {el:.1f} s, numpy on the host"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=16, help="layer copies rotated through in decode runs")
    ap.add_argument("--only", default="", help="comma list of decode1,decode32,prefill8192,stack40 (default all)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-quant", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain copy kernel of known size (for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import torch
    import weight_only_int4_rtn_amd as w4
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    w4._lib.lib()
    only = set(args.only.split(",")) if args.only else {"decode1", "decode32", "prefill8192", "stack40"}

    if args.copy_calibration:
        copy_calibration()
    log("[bench] building layers")
    layers = make_layers(args.copies, seed=1)
    results = {}
    if "decode1" in only:
        results["decode1"] = measure("decode1", 1, layers, args.steps, args.warmup, min(args.steps, 100), 11)
    if "decode32" in only:
        results["decode32"] = measure("decode32", 32, layers, args.steps, args.warmup, min(args.steps, 100), 12)
    if "prefill8192" in only:
        pst = max(5, args.steps // 10)
        results["prefill8192"] = measure("prefill8192", 8192, layers[:4], pst, max(2, args.warmup // 4),
                                         min(pst, 10), 13)
    quant = None if args.no_quant else time_quantizer()
    del layers
    torch.cuda.empty_cache()
    stack = None
    if "stack40" in only:
        log("[bench] building the 40-layer stack")
        stack_layers = make_stack_layers(40, (7, 13, 18, 23, 29, 35), seed=4)
        stack = measure_stack(4, stack_layers, max(5, args.steps // 20), max(2, args.warmup // 5), 14)
        del stack_layers
        torch.cuda.empty_cache()

    if not results:   # only the stack was asked for: it is the headline
        line = {"metric": METRIC, "value": round(stack["tok_per_s"], 2), "unit": "tok/s", "n_gpus": 1,
                "steps": max(5, args.steps // 20), "warmup": max(2, args.warmup // 5),
                "ms_per_step": round(stack["ms_per_step"], 5), "higher_is_better": True, "scaling": "weak",
                "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
                "config": {"workload": "stack40: 40-layer decode stack, T=4", "global_batch": 4, "seq_len": 1,
                           "parallelism": "none (1 GPU)"},
                "expert_weight_GBps": round(stack["expert_weight_GBps"], 1),
                "roofline": {"bound": "hbm", "kernel": "whole stack step", "achieved": round(stack["expert_weight_GBps"], 1),
                             "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                             "frac": round(stack["expert_weight_GBps"] / HBM_PEAK_GBPS, 4), "traffic": None}}
        print(json.dumps(line), flush=True)
        return
    head_name = "decode1" if "decode1" in results else next(iter(results))
    head = results[head_name]
    line = {
        "metric": METRIC,
        "value": round(head["tok_per_s"], 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps if head_name != "prefill8192" else max(5, args.steps // 10),
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{head_name}: one MoE layer, 256 experts top-8, hidden 2048, intermediate 512, "
                               f"INT4 sym group-128 weights, bf16 activations, T={head['T']} tokens",
                   "global_batch": head["T"], "seq_len": 1, "parallelism": "none (1 GPU)"},
        "expert_weight_GBps": round(head["expert_weight_GBps"], 1),
        "launch": "HIP graph replay of the timed steps (eager stream launches reported as eager_*)",
        "eager_tok_per_s": round(head["T"] / head["eager_ms_per_step"] * 1e3, 2),
        "eager_ms_per_step": round(head["eager_ms_per_step"], 5),
        "roofline": roofline_for(head, "mfma" if head_name == "prefill8192" else "hbm", head_name),
    }
    if stack is not None:
        line["stack40"] = {"tok_per_s": round(stack["tok_per_s"], 1), "ms_per_step": round(stack["ms_per_step"], 4),
                           "eager_ms_per_step": round(stack["eager_ms_per_step"], 4),
                           "expert_weight_GBps": round(stack["expert_weight_GBps"], 1),
                           "weight_GB_per_step": round(stack["weight_bytes_per_step"] / 1e9, 3),
                           "frac_hbm": round(stack["expert_weight_GBps"] / HBM_PEAK_GBPS, 4),
                           "workload": "40 layers x (256 experts top-8, INT4; INT8 on layers 7,13,18,23,29,35) "
                                       "+ INT8 shared expert per layer, bf16 residual, T=4"}
    for nm, r in results.items():
        if r is None:
            continue
        if nm == head_name:
            line["kernels_us"] = r["kernels_us"]
            continue
        line[nm] = {"tok_per_s": round(r["tok_per_s"], 1), "ms_per_step": round(r["ms_per_step"], 5),
                    "eager_ms_per_step": round(r["eager_ms_per_step"], 5),
                    "expert_weight_GBps": round(r["expert_weight_GBps"], 1), "TFLOPs": round(r["TFLOPs"], 2),
                    "distinct_experts_mean": r["distinct_experts_mean"], "kernels_us": r["kernels_us"],
                    "roofline": roofline_for(r, "mfma" if nm == "prefill8192" else "hbm", nm)}
    if quant:
        line["quantize"] = quant
    if not args.no_cpu:
        log("[bench] timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
