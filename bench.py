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
NO_GRAPH = False   # set by --no-graph


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
    # steps), which removes host launch cost as a decode loop does in serving; an event pair
    # around every replay gives the distribution of the per-step time over replays
    if NO_GRAPH:   # counter-collection runs: eager launches only (reported in both fields)
        graph_ms = eager_ms
        pct = {"p10": eager_ms, "p50": eager_ms, "p90": eager_ms, "samples": 1, "steps_per_sample": steps}
    else:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(n_logits):
                step(i)
        graph.replay()
        torch.cuda.synchronize()
        reps = max(25, -(-steps // n_logits))
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        start.record()
        for r in range(reps):
            evs[r][0].record()
            graph.replay()
            evs[r][1].record()
        end.record()
        torch.cuda.synchronize()
        graph_ms = start.elapsed_time(end) / (reps * n_logits)
        samples = sorted(a.elapsed_time(b) / n_logits for a, b in evs)
        pct = {"p10": samples[len(samples) // 10], "p50": samples[len(samples) // 2],
               "p90": samples[(9 * len(samples)) // 10], "samples": len(samples), "steps_per_sample": n_logits}
        del graph
    # the faster of the two launch modes is the step time (both are reported)
    launch_mode = "eager" if NO_GRAPH or graph_ms > eager_ms else "graph"
    ms_per_step = min(graph_ms, eager_ms)

    # per-kernel durations with HIP events around each kernel, same rotation
    per = {}
    for i in range(timed_steps):
        w13, s13, w2, s2 = layers[i % n_copies]
        _, tk = w4.moe_w4a16_forward_timed(xs[i % 8], w13, s13, w2, s2, top_k=K,
                                           router_logits=logits[i % n_logits], out=out, workspace=ws)
        for nm, ms in tk:
            per.setdefault(nm, []).append(ms)
    kernels = {nm: sum(v) / len(v) * 1e3 for nm, v in per.items()}   # average us per launch
    kernel_pct = {nm: {"p10": round(sorted(v)[len(v) // 10] * 1e3, 2), "p90": round(sorted(v)[(9 * len(v)) // 10] * 1e3, 2)}
                  for nm, v in per.items()}

    d_mean = sum(distinct[(warmup + i) % n_logits] for i in range(steps)) / steps
    gu, dn = expert_bytes()
    weight_bytes = d_mean * (gu + dn)
    flops = 2.0 * T * K * 3 * H * I
    res = {
        "T": T, "ms_per_step": ms_per_step, "eager_ms_per_step": eager_ms, "eager_wall_ms_per_step": wall_ms / steps,
        "graph_ms_per_step": graph_ms, "launch_mode": launch_mode,
        "tok_per_s": T / (ms_per_step / 1e3),
        "distinct_experts_mean": d_mean,
        "expert_weight_bytes_per_step": weight_bytes,
        "expert_weight_GBps": weight_bytes / (ms_per_step / 1e3) / 1e9,
        "TFLOPs": flops / (ms_per_step / 1e3) / 1e12,
        "kernels_us": {k: round(v, 2) for k, v in kernels.items()},
        "kernels_us_p10_p90": kernel_pct,
        "step_ms_pct": {k: (round(v, 5) if isinstance(v, float) else v) for k, v in pct.items()},
        "copies": n_copies,
    }
    # algorithmic bytes and flops of the two expert kernels, per launch
    act_in = T * H * 2
    a_bytes = T * K * I * 2
    res["kernel_bytes"] = {"gate_up": d_mean * gu + act_in + a_bytes, "down": d_mean * dn + a_bytes + T * H * 2}
    res["kernel_bytes"]["all"] = d_mean * (gu + dn) + act_in + T * E * 4 + T * H * 2
    res["kernel_flops"] = {"gate_up": 2.0 * T * K * 2 * I * H, "down": 2.0 * T * K * H * I}
    res["kernel_flops"]["all"] = res["kernel_flops"]["gate_up"] + res["kernel_flops"]["down"]
    log(f"[bench] {name}: {ms_per_step * 1e3:.1f} us/step (graph {graph_ms * 1e3:.1f}; eager {eager_ms * 1e3:.1f}, host wall "
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
    graph_ms = start.elapsed_time(end) / (reps * n_logits)
    del graph
    ms = min(graph_ms, eager_ms)
    nbytes = 0.0
    for i in range(steps):
        for l, lay in enumerate(layers):
            gu, dn = expert_bytes(lay["bits"])
            nbytes += distinct[l][(warmup + i) % n_logits] * (gu + dn) + sum(expert_bytes(8))
    nbytes /= steps
    res = {"T": T, "layers": L, "ms_per_step": ms, "eager_ms_per_step": eager_ms, "graph_ms_per_step": graph_ms,
           "launch_mode": "graph" if graph_ms <= eager_ms else "eager",
           "eager_wall_ms_per_step": wall_ms / steps,
           "tok_per_s": T / (ms / 1e3), "weight_bytes_per_step": nbytes,
           "expert_weight_GBps": nbytes / (ms / 1e3) / 1e9}
    log(f"[bench] stack{L}: {ms * 1e3:.1f} us/step (graph {graph_ms * 1e3:.1f}; eager {eager_ms * 1e3:.1f}), "
        f"{res['tok_per_s']:.1f} tok/s, "
        f"{res['expert_weight_GBps']:.0f} GB/s expert weights ({nbytes / 1e9:.2f} GB per step)")
    del ws
    return res


class SclkSampler:
    """Polls rocm-smi for the current shader clock while the GPU is busy (a thread)."""

    def __init__(self):
        import threading
        self.mhz = []
        self.stop = threading.Event()
        self.thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        import re
        import subprocess
        while not self.stop.is_set():
            try:
                out = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                                     timeout=10).stdout
                for key, val in re.findall(r'"(sclk[^"]*)":\s*"([^"]*)"', out):
                    m = re.search(r"(\d+)\s*Mhz", val, flags=re.I)
                    if m:
                        self.mhz.append(int(m.group(1)))
            except Exception:
                return
            self.stop.wait(0.2)

    def __enter__(self):
        self.thread.start()
        return self

    def __exit__(self, *exc):
        self.stop.set()
        self.thread.join(timeout=15)

    def enough(self):
        return len(self.mhz) >= 5

    def summary(self):
        if not self.mhz:
            return None
        v = sorted(self.mhz)
        return {"median_mhz": v[len(v) // 2], "max_mhz": v[-1], "min_mhz": v[0], "samples": len(v),
                "source": "rocm-smi --showclocks while the 8192-token prefill step runs"}


def make_fmt_layers(fmt, n_copies, seed):
    """n_copies layers with routed experts in FP8 E4M3 per channel or MXFP4 (MSE scales)."""
    import torch
    import synth
    import weight_only_int4_rtn_amd as w4
    dev = torch.device("cuda:0")
    bits = 8 if fmt == "fp8" else 4
    layers = []
    chunk = 32
    for c in range(n_copies):
        w13 = torch.empty((E, 2 * I, H * bits // 32), dtype=torch.int32, device=dev)
        w2 = torch.empty((E, H, I * bits // 32), dtype=torch.int32, device=dev)
        if fmt == "fp8":
            s13 = torch.empty((E, 2 * I), dtype=torch.float32, device=dev)
            s2 = torch.empty((E, H), dtype=torch.float32, device=dev)
        else:
            s13 = torch.empty((E, 2 * I, H // 32), dtype=torch.uint8, device=dev)
            s2 = torch.empty((E, H, I // 32), dtype=torch.uint8, device=dev)
        for e0 in range(0, E, chunk):
            sl = slice(e0, e0 + chunk)
            f13 = synth.device_normal((chunk, 2 * I, H), synth.WEIGHT_STD, seed * 1000 + c * 64 + e0 // chunk, dev)
            f2 = synth.device_normal((chunk, H, I), synth.WEIGHT_STD, seed * 1000 + c * 64 + 32 + e0 // chunk, dev)
            if fmt == "fp8":
                w4.fp8_quantize_pack(f13, packed=w13[sl], scales=s13[sl])
                w4.fp8_quantize_pack(f2, packed=w2[sl], scales=s2[sl])
            else:
                w4.mxfp4_quantize_pack(f13, "mse", packed=w13[sl], scales=s13[sl])
                w4.mxfp4_quantize_pack(f2, "mse", packed=w2[sl], scales=s2[sl])
            del f13, f2
        layers.append((w13, s13, w2, s2))
    torch.cuda.synchronize()
    return layers


def fmt_expert_bytes(fmt):
    """Algorithmic bytes of one expert in FP8 (codes + fp32 row scales) or MXFP4 (codes +
    one E8M0 byte per 32 columns)."""
    if fmt == "fp8":
        return 2 * I * H + 2 * I * 4, H * I + H * 4
    return 2 * I * H // 2 + 2 * I * H // 32, H * I // 2 + H * I // 32


def measure_fmt(fmt, T, layers, steps, warmup, seed):
    """Step time of a T-token batch with FP8 / MXFP4 routed experts (eager launches, one call
    per step), the per-kernel event times, and the expert bytes and flops per step."""
    import torch
    import synth
    import weight_only_int4_rtn_amd as w4
    dev = torch.device("cuda:0")
    bits = 8 if fmt == "fp8" else 4
    n_logits = 16
    logits = [synth.device_normal((T, E), 1.0, seed * 7919 + i, dev) for i in range(n_logits)]
    x = synth.device_normal((T, H), 1.0, seed, dev, torch.bfloat16)
    ws = w4.new_workspace(w4.moe_w4a16_workspace_size(T, H, I, E, K), dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    calls = [w4.MoeCall(x, *lay, top_k=K, bits=bits, weight_format=fmt, workspace=ws) for lay in layers]
    distinct = [int(torch.topk(l, K, dim=1).indices.unique().numel()) for l in logits]

    def step(i):
        calls[i % len(calls)](x, out, router_logits=logits[i % n_logits])

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        step(warmup + i)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    per = {}
    for i in range(min(steps, 20)):
        _, tk = w4.moe_w4a16_forward_timed(x, *layers[i % len(layers)], top_k=K, bits=bits, weight_format=fmt,
                                           router_logits=logits[i % n_logits], out=out, workspace=ws)
        for nm, t in tk:
            per.setdefault(nm, []).append(t)
    kernels = {nm: round(sum(v) / len(v) * 1e3, 2) for nm, v in per.items()}
    gu, dn = fmt_expert_bytes(fmt)
    d_mean = sum(distinct[(warmup + i) % n_logits] for i in range(steps)) / steps
    wbytes = d_mean * (gu + dn)
    flops = 2.0 * T * K * 3 * H * I
    res = {"T": T, "ms_per_step": round(ms, 5), "tok_per_s": round(T / ms * 1e3, 1),
           "expert_weight_GBps": round(wbytes / ms / 1e6, 1), "TFLOPs": round(flops / ms / 1e9, 2),
           "kernels_us": kernels}
    gk = next((k for k in kernels if k.startswith("gk_")), None)
    if gk is not None:
        if T > 64:
            res["roofline"] = {"bound": "mfma", "kernel": gk,
                               "achieved": round(2.0 * T * K * 2 * I * H / kernels[gk] / 1e6, 1),
                               "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
        else:
            res["roofline"] = {"bound": "hbm", "kernel": gk,
                               "achieved": round((d_mean * gu + T * H * 2) / kernels[gk] / 1e3, 1),
                               "peak": HBM_PEAK_GBPS, "unit": "GB/s"}
        res["roofline"]["frac"] = round(res["roofline"]["achieved"] / res["roofline"]["peak"], 4)
    log(f"[bench] {fmt} T={T}: {ms * 1e3:.1f} us/step, {res['tok_per_s']} tok/s, {res['expert_weight_GBps']} GB/s, "
        f"{res['TFLOPs']} TFLOP/s, kernels {kernels}")
    del ws, out, logits
    return res


# The INT8 group-128 projections of one attention and one Gated DeltaNet layer at hidden
# 2048, (N, K): q_proj with its output gate, k_proj, v_proj, o_proj; in_proj_qkv,
# in_proj_z, out_proj.
DENSE_SHAPES = [("attn.q_proj", 8192, 2048), ("attn.k_proj", 512, 2048), ("attn.v_proj", 512, 2048),
                ("attn.o_proj", 2048, 4096), ("deltanet.in_proj_qkv", 8192, 2048),
                ("deltanet.in_proj_z", 4096, 2048), ("deltanet.out_proj", 2048, 4096)]


def measure_linear(T, copies, steps, seed):
    """The seven projections back to back at T tokens, rotating through `copies` weight
    sets (8 sets of 62 MB: more than the 256 MB Infinity Cache) so that decode reads them
    from HBM.  Timed as HIP-graph replays (one graph per weight set holding the seven
    calls) and as eager calls through the Python binding; the graph time is the GPU's,
    the eager one adds the binding's host work per call."""
    import torch
    import synth
    import weight_only_int4_rtn_amd as w4
    dev = torch.device("cuda:0")
    sets = []
    for c in range(copies):
        ws = []
        for i, (nm, N, Kd) in enumerate(DENSE_SHAPES):
            w = synth.device_normal((N, Kd), synth.WEIGHT_STD, seed * 100 + c * 10 + i, dev)
            ws.append(w4.rtn_quantize_pack(w, 8))
            del w
        sets.append(ws)
    xs = {Kd: synth.device_normal((T, Kd), 1.0, seed + Kd, dev, torch.bfloat16) for Kd in (2048, 4096)}
    outs = {N: torch.empty((T, N), dtype=torch.bfloat16, device=dev) for _, N, _ in DENSE_SHAPES}
    wsp = torch.empty((max(w4._lib.lib().w4a16_linear_workspace_size(T, Kd, N) for _, N, Kd in DENSE_SHAPES),),
                      dtype=torch.uint8, device=dev)

    def step(i):
        for (nm, N, Kd), (p, sc) in zip(DENSE_SHAPES, sets[i % copies]):
            w4.w4a16_linear(xs[Kd], p, sc, out=outs[N], workspace=wsp)

    for i in range(copies):
        step(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        step(i)
    b.record()
    torch.cuda.synchronize()
    eager_ms = a.elapsed_time(b) / steps
    graph_ms = eager_ms
    if not NO_GRAPH:
        graphs = []
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(c)
            graphs.append(g)
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        a.record()
        for i in range(steps):
            graphs[i % copies].replay()
        b.record()
        torch.cuda.synchronize()
        graph_ms = a.elapsed_time(b) / steps
        del graphs
    ms = min(graph_ms, eager_ms)
    nbytes = sum(N * Kd + N * (Kd // 128) * 2 for _, N, Kd in DENSE_SHAPES)
    flops = sum(2.0 * T * N * Kd for _, N, Kd in DENSE_SHAPES)
    res = {"T": T, "ms_per_step": round(ms, 5), "graph_ms_per_step": round(graph_ms, 5),
           "eager_ms_per_step": round(eager_ms, 5), "launch_mode": "graph" if graph_ms <= eager_ms else "eager",
           "weight_GBps": round(nbytes / ms / 1e6, 1), "TFLOPs": round(flops / ms / 1e9, 2), "weight_bytes": nbytes}
    res["frac"] = round((res["weight_GBps"] / HBM_PEAK_GBPS) if T <= 64 else (res["TFLOPs"] / BF16_PEAK_TFLOPS), 4)
    log(f"[bench] dense INT8 projections T={T}: {ms * 1e3:.1f} us for all seven (graph {graph_ms * 1e3:.1f}, eager "
        f"{eager_ms * 1e3:.1f}), {res['weight_GBps']} GB/s, {res['TFLOPs']} TFLOP/s")
    del sets, wsp
    return res


def read_floor(nbytes, n_buffers, reps):
    """The achievable time to read `nbytes` from HBM in one launch: the library's plain
    streaming read (w4a16_stream_read: 16-byte vector loads, grid-stride, XOR-folded into
    one word) over one of `n_buffers` buffers, rotated so that every read misses the 256 MB
    Infinity Cache; returns us per read (event-timed, back to back)."""
    import torch
    import weight_only_int4_rtn_amd as w4
    dev = torch.device("cuda:0")
    n = (nbytes + 15) // 16 * 4
    bufs = [torch.ones(n, dtype=torch.int32, device=dev) for _ in range(n_buffers)]
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for i in range(n_buffers):
        w4.stream_read(bufs[i], sink)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(reps):
        w4.stream_read(bufs[i % n_buffers], sink)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / reps * 1e3
    del bufs
    return us


def keep_busy(T, layers, seconds, sampler):
    """Back-to-back forwards of a T-token batch until `seconds` pass or the sampler has enough."""
    import torch
    import synth
    import weight_only_int4_rtn_amd as w4
    dev = torch.device("cuda:0")
    x = synth.device_normal((T, H), 1.0, 5, dev, torch.bfloat16)
    logits = synth.device_normal((T, E), 1.0, 6, dev)
    ws = w4.new_workspace(w4.moe_w4a16_workspace_size(T, H, I, E, K), dev)
    call = w4.MoeCall(x, *layers[0], top_k=K, workspace=ws)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end and not sampler.enough():
        for _ in range(20):
            call(x, out, router_logits=logits)
        torch.cuda.synchronize()
    del ws


def time_router(layers, seed):
    """The router GEMM (bf16 [256, 2048]) plus the shared-expert gate ahead of the routing:
    its kernel time at 1, 32 and 8192 tokens, from self-routed forwards."""
    import torch
    import synth
    import weight_only_int4_rtn_amd as w4
    dev = torch.device("cuda:0")
    out = {}
    sh = dict(w13=torch.zeros((2 * I, H // 8), dtype=torch.int32, device=dev),
              s13=torch.zeros((2 * I, H // 128), dtype=torch.bfloat16, device=dev),
              w2=torch.zeros((H, I // 8), dtype=torch.int32, device=dev),
              s2=torch.zeros((H, I // 128), dtype=torch.bfloat16, device=dev), bits=4)
    wr = synth.device_normal((E, H), H ** -0.5, seed, dev, torch.bfloat16)
    wg = synth.device_normal((H,), H ** -0.5, seed + 1, dev, torch.bfloat16)
    for T in (1, 32, 8192):
        x = synth.device_normal((T, H), 1.0, seed + T, dev, torch.bfloat16)
        ws = w4.new_workspace(w4.moe_w4a16_workspace_size(T, H, I, E, K, 4, I), dev)
        ts = []
        for i in range(12):
            _, tk = w4.moe_w4a16_forward_timed(x, *layers[i % len(layers)], top_k=K, router_w=wr, shared=sh,
                                               shared_gate_w=wg, workspace=ws)
            if i >= 2:
                ts += [ms for nm, ms in tk if nm == "router"]
        us = sum(ts) / len(ts) * 1e3
        nbytes = (E + 1) * H * 2 + T * H * 2 + T * (E + 1) * 4
        out[f"T{T}"] = {"us": round(us, 2), "GBps": round(nbytes / us / 1e3, 1),
                        "TFLOPs": round(2.0 * T * (E + 1) * H / us / 1e6, 2)}
        del ws, x
    log(f"[bench] router + shared gate: {out}")
    return out


def _cpu_child(spec):
    """One CPU-oracle timing run in its own process (BLAS threads fixed by its environment).
    Phase (i): dequantize + expert MLPs + weighted sum per forward, on bounded samples of
    decode1, decode32, the prefill chunk and one stack layer; phase (ii): the quantizer
    on a sample of experts, extrapolated to one full layer (805 M weights)."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        threads = 1
    budget = float(spec["seconds"])
    rng = np.random.default_rng(5)

    # packed experts with random valid codes and bf16 scales: the oracle's arithmetic and
    # its time do not depend on the values (the FFN is a dense product either way)
    def rand_packed(shape_words):
        return rng.integers(-2 ** 31, 2 ** 31, size=shape_words, dtype=np.int64).astype(np.int32)

    n_pool = 64
    pool = [(rand_packed((2 * I, H // 8)), np.full((2 * I, H // 128), 0x3B80, np.uint16),
             rand_packed((H, I // 8)), np.full((H, I // 128), 0x3B80, np.uint16)) for _ in range(n_pool)]

    class View:
        def __init__(self, i):
            self.i = i

        def __getitem__(self, e):
            return pool[int(e) % n_pool][self.i]

    views = [View(i) for i in range(4)]
    sh8 = dict(w13=rand_packed((2 * I, H // 4)), s13=np.full((2 * I, H // 128), 0x3B80, np.uint16),
               w2=rand_packed((H, I // 4)), s2=np.full((H, I // 128), 0x3B80, np.uint16), bits=8)

    def timed(fn, per_call_tokens, max_s):
        done, t0 = 0, time.perf_counter()
        while True:
            fn(done)
            done += 1
            el = time.perf_counter() - t0
            if el >= max_s:
                break
        return {"tok_per_s": round(done * per_call_tokens / el, 4), "calls": done, "seconds": round(el, 2)}

    phases = {}
    l1 = synth.router_logits(1, 8, E)
    x1 = synth.activations_bf16(1, 8, H)
    phases["decode1"] = timed(lambda i: oracle.moe_layer(x1[i % 8:i % 8 + 1], l1[i % 8:i % 8 + 1], K, *views, 4),
                              1, budget * 0.2)
    l32 = synth.router_logits(2, 32, E)
    x32 = synth.activations_bf16(2, 32, H)
    phases["decode32"] = timed(lambda i: oracle.moe_layer(x32, l32, K, *views, 4), 32, budget * 0.25)
    lp = synth.router_logits(3, 8192, E)[:64]
    xp = synth.activations_bf16(3, 64, H)
    phases["prefill8192_sample64"] = timed(lambda i: oracle.moe_layer(xp, lp, K, *views, 4), 64, budget * 0.25)
    l4 = synth.router_logits(4, 4, E)
    x4 = synth.activations_bf16(4, 4, H)
    st = timed(lambda i: oracle.moe_layer(x4, l4, K, *views, 4, shared=sh8, residual_bits=x4), 4, budget * 0.15)
    st["stack40_tok_per_s"] = round(st["tok_per_s"] / 40, 4)   # 40 such layers per stack step
    phases["stack40_one_layer"] = st
    # phase (ii): quantize + pack experts' fp32 weights, extrapolated to one full layer
    w13 = synth.expert_w13(1, 0, 0, H, I)
    w2 = synth.expert_w2(1, 0, 0, H, I)
    q = timed(lambda i: (oracle.quantize_pack(w13, 4), oracle.quantize_pack(w2, 4)), 1, budget * 0.15)
    per_expert_s = 1.0 / q["tok_per_s"]
    phases["quantize_full_layer"] = {"weights_per_s": round(3 * H * I / per_expert_s), "experts_timed": q["calls"],
                                     "seconds_per_layer_extrapolated": round(per_expert_s * E, 2)}
    return {"threads": threads, "phases": phases}


def cpu_baseline(seconds):
    """The oracle as it stands, timed on the host in child processes with the BLAS thread
    count fixed before import: all host threads, then one."""
    import subprocess
    try:
        model = next((ln.split(":", 1)[1].strip() for ln in open("/proc/cpuinfo") if ln.startswith("model name")),
                     "unknown")
    except OSError:
        model = "unknown"
    nproc = len(os.sched_getaffinity(0))
    runs = {}
    for n in (nproc, 1):
        env = dict(os.environ)
        for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS"):
            env[var] = str(n)
        env["CUDA_VISIBLE_DEVICES"] = ""
        env["HIP_VISIBLE_DEVICES"] = ""
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-child",
                            json.dumps({"seconds": seconds})], capture_output=True, text=True, env=env, timeout=600)
        if r.returncode != 0:
            log(f"[bench] cpu child ({n} threads) failed: {r.stderr[-500:]}")
            continue
        runs[n] = json.loads(r.stdout.strip().splitlines()[-1])
        log(f"[bench] cpu oracle, {n} threads: {runs[n]}")
    if not runs:
        return None
    main_run = runs.get(nproc) or next(iter(runs.values()))
    d1 = main_run["phases"]["decode1"]
    return {"value": d1["tok_per_s"], "unit": "tok/s", "cores": main_run["threads"], "kind": "oracle",
            "sample": f"{d1['calls']} single-token forwards of the 256-expert top-8 H=2048 I=512 INT4 layer "
                      f"(route + dequant + fp64 SwiGLU + weighted sum) in {d1['seconds']} s, numpy",
            "cpu_model": model, "nproc": nproc,
            "phases_all_threads": main_run["phases"],
            "phases_one_thread": runs[1]["phases"] if 1 in runs else None,
            "one_thread_cores": runs[1]["threads"] if 1 in runs else None}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=16, help="layer copies rotated through in decode runs")
    ap.add_argument("--only", default="", help="comma list of decode1,decode32,prefill8192,stack40 (default all)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="CPU oracle budget per thread setting")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-quant", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain copy kernel of known size (for scaling HBM byte counters)")
    ap.add_argument("--no-router", action="store_true")
    ap.add_argument("--no-formats", action="store_true", help="skip the FP8 / MXFP4 expert runs")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense INT8 projection runs")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (no HIP graph capture; for counter-collection runs)")
    ap.add_argument("--no-sclk", action="store_true",
                    help="do not sample the shader clock (it starts rocm-smi; use under a profiler)")
    ap.add_argument("--cpu-child", default=None, help=argparse.SUPPRESS)
    args = ap.parse_args()
    global NO_GRAPH
    NO_GRAPH = args.no_graph
    if args.cpu_child is not None:
        sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
        print(json.dumps(_cpu_child(json.loads(args.cpu_child))), flush=True)
        return
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
    sclk = None
    if "prefill8192" in only:
        pst = max(5, args.steps // 10)
        results["prefill8192"] = measure("prefill8192", 8192, layers[:4], pst, max(2, args.warmup // 4),
                                         min(pst, 10), 13)
        if not args.no_sclk:
            with SclkSampler() as sampler:
                keep_busy(8192, layers[:4], 4.0, sampler)   # the MFMA-bound step while the clock is sampled
            sclk = sampler.summary()
    floor = None
    if "decode1" in results:
        # the single-token layer's expert bytes (8 experts) read once by a plain kernel, and
        # the same for the 32-token batch's distinct experts
        nb1 = int(results["decode1"]["kernel_bytes"]["all"])
        floor = {"decode1_bytes": nb1, "decode1_read_us": round(read_floor(nb1, 40, 400), 2)}
        floor["decode1_frac_of_hbm"] = round(nb1 / floor["decode1_read_us"] / 1e3 / HBM_PEAK_GBPS, 4)
        floor["tiny_decode_over_floor"] = round(results["decode1"]["kernels_us"].get("tiny_decode", 0) /
                                                floor["decode1_read_us"], 2)
        if "decode32" in results:
            nb32 = int(results["decode32"]["expert_weight_bytes_per_step"])
            floor["decode32_bytes"] = nb32
            floor["decode32_read_us"] = round(read_floor(nb32, 3, 60), 2)
        log(f"[bench] read floor: {floor}")
    router = None if args.no_router else time_router(layers[:4], 17)
    del layers
    torch.cuda.empty_cache()
    formats = {}
    if not args.no_formats:
        for fmt in ("fp8", "mxfp4"):
            log(f"[bench] building {fmt} layers")
            fl = make_fmt_layers(fmt, 4, seed=21)
            formats[fmt] = {f"T{T}": measure_fmt(fmt, T, fl, st, 5, 31 + T)
                            for T, st in ((1, 100), (32, 100), (8192, 10))}
            del fl
            torch.cuda.empty_cache()
    dense = None
    if not args.no_dense:
        dense = {f"T{T}": measure_linear(T, 8, st, 41) for T, st in ((1, 64), (32, 64), (8192, 8))}
    quant = None if args.no_quant else time_quantizer()
    stack = None
    if "stack40" in only:
        log("[bench] building the 40-layer stack")
        stack_layers = make_stack_layers(40, (7, 13, 18, 23, 29, 35), seed=4)
        stack = measure_stack(4, stack_layers, max(5, args.steps // 20), max(2, args.warmup // 5), 14)
        del stack_layers
        torch.cuda.empty_cache()

    if not results and stack is None:   # side measurements only (a profiling run): no headline
        side = {"router": router, "formats": formats or None, "dense_int8": dense, "quantize": quant}
        print(json.dumps({"metric": METRIC, "value": None, "unit": "tok/s", "n_gpus": 1,
                          **{k: v for k, v in side.items() if v}}), flush=True)
        return
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
        "launch": f"{head['launch_mode']}: the faster of HIP graph replay of the timed steps and eager stream "
                  f"launches of one library call per step (both below)",
        "eager_tok_per_s": round(head["T"] / head["eager_ms_per_step"] * 1e3, 2),
        "eager_ms_per_step": round(head["eager_ms_per_step"], 5),
        "graph_tok_per_s": round(head["T"] / head["graph_ms_per_step"] * 1e3, 2),
        "graph_ms_per_step": round(head["graph_ms_per_step"], 5),
        "roofline": roofline_for(head, "mfma" if head_name == "prefill8192" else "hbm", head_name),
    }
    if stack is not None:
        line["stack40"] = {"tok_per_s": round(stack["tok_per_s"], 1), "ms_per_step": round(stack["ms_per_step"], 4),
                           "eager_ms_per_step": round(stack["eager_ms_per_step"], 4),
                           "graph_ms_per_step": round(stack["graph_ms_per_step"], 4),
                           "launch_mode": stack["launch_mode"],
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
                    "graph_ms_per_step": round(r["graph_ms_per_step"], 5), "launch_mode": r["launch_mode"],
                    "expert_weight_GBps": round(r["expert_weight_GBps"], 1), "TFLOPs": round(r["TFLOPs"], 2),
                    "distinct_experts_mean": r["distinct_experts_mean"], "kernels_us": r["kernels_us"],
                    "kernels_us_p10_p90": r["kernels_us_p10_p90"], "step_ms_pct": r["step_ms_pct"],
                    "roofline": roofline_for(r, "mfma" if nm == "prefill8192" else "hbm", nm)}
    line["step_ms_pct"] = head["step_ms_pct"]
    line["kernels_us_p10_p90"] = head["kernels_us_p10_p90"]
    if quant:
        line["quantize"] = quant
    if router:
        line["router"] = router
    if floor:
        line["read_floor"] = floor
    if formats:
        line["formats"] = formats
    if dense:
        line["dense_int8"] = dense
    line["sclk"] = sclk
    if not args.no_cpu:
        log("[bench] timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
