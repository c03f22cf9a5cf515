"""Build ``libw4a16.so`` in-tree with hipcc for gfx950.

Usage: ``python -m weight_only_int4_rtn_amd.build`` (or ``build()`` from Python).
Every source is compiled on each call; objects go to ``_build/`` at the repository
root and the shared library next to this file.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libw4a16.so")
SOURCES = ["api.hip", "quant.hip", "quant_fmt.hip", "route.hip", "router.hip", "linear.hip", "moe_decode.hip",
           "decode_stream.hip", "moe_prefill.hip", "stream_read.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no packed fp32 VALU instructions in any kernel.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         f"-I{INCLUDE}", f"-I{CSRC}"] + DEVICE_FLAGS


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [[HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
        for cmd, err in zip(cmds, ex.map(_run, cmds)):
            if verbose and err.strip():
                print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


def resource_usage(sources=None) -> str:
    """Per-kernel register, LDS and scratch use of every gfx950 kernel, from the compiler's
    kernel-resource-usage remarks (the device pass of each source, nothing linked)."""
    import re
    import subprocess as sp
    rows = []
    for src in sources or SOURCES:
        cmd = [HIPCC, *FLAGS, "--cuda-device-only", "-c", os.path.join(CSRC, src), "-o", os.devnull,
               "-Rpass-analysis=kernel-resource-usage"]
        r = sp.run(cmd, capture_output=True, text=True)
        cur = None
        for line in r.stderr.splitlines():
            m = re.search(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]"
                          r"|LDS Size \[bytes/block\]|SGPRs): (\S+)", line)
            if not m:
                continue
            key, val = m.group(1), m.group(2)
            if key == "Function Name":
                cur = {"kernel": val, "file": src}
                rows.append(cur)
            elif cur is not None:
                cur[key.split()[0]] = val
    names = {}
    try:
        out = sp.run(["c++filt"], input="\n".join(r["kernel"] for r in rows), capture_output=True, text=True).stdout
        names = dict(zip([r["kernel"] for r in rows], out.splitlines()))
    except OSError:
        pass
    lines = [f"{'file':<18} {'VGPRs':>5} {'AGPRs':>5} {'SGPRs':>5} {'scratch':>7} {'LDS':>6} {'occ':>3}  kernel"]
    for r in rows:
        nm = names.get(r["kernel"], r["kernel"]).replace("w4a16::", "").replace("(anonymous namespace)::", "")
        lines.append(f"{r['file']:<18} {r.get('VGPRs', '?'):>5} {r.get('AGPRs', '?'):>5} {r.get('SGPRs', '?'):>5} "
                     f"{r.get('ScratchSize', '?'):>7} {r.get('LDS', '?'):>6} {r.get('Occupancy', '?'):>3}  {nm}")
    return "\n".join(lines)


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--resource-usage":
        print(resource_usage(sys.argv[2:] or None))
    else:
        print(build(verbose=True))
