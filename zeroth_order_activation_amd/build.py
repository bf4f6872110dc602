"""Build libdust.so (HIP for gfx950) in-tree with hipcc.

    python -m zeroth_order_activation_amd.build

Each .hip file is compiled to an object in _build/ (in parallel), then linked
into zeroth_order_activation_amd/libdust.so.  Always rebuilds.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdust.so")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    # packed fp32 VALU ops stay off (plain fp32 code only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(extra=(), jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra)), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources", file=sys.stderr)
    return LIB


PROBE_SRC = os.path.join(PKG, "probe", "valu_mix.hip")
PROBE_LIB = os.path.join(PKG, "libdust_probe.so")
PROBE_COUNTS = os.path.join(PKG, "libdust_probe.json")
PROBE_KERNELS = {"mix_fma_kernel": 0, "mix_mad64_kernel": 1, "mix_trans_kernel": 2, "mix_head_kernel": 3}


def loop_valu_counts(asm: str) -> dict:
    """{kernel name: [vector instructions of each innermost loop body]} from gfx950
    assembly: a loop runs from its 'Inner Loop Header' label to the branch back to it."""
    import re
    out, fn, lines, i = {}, None, asm.split("\n"), 0
    while i < len(lines):
        f = re.match(r"^(_Z\w+):", lines[i])
        if f:
            fn = f.group(1)
        m = re.match(r"^(\.LBB\w+):.*Inner Loop Header", lines[i])
        if m and fn:
            lab, n, j = m.group(1), 0, i + 1
            while j < len(lines) and not re.match(r"^\s+s_cbranch\w*\s+" + re.escape(lab) + r"\s*$", lines[j]):
                t = lines[j].split()
                n += bool(t) and t[0].startswith("v_")
                j += 1
            out.setdefault(fn, []).append(n)
            i = j
        i += 1
    return out


def build_probe() -> str:
    """libdust_probe.so (the vector-ALU issue-rate probes the benchmark times) and
    libdust_probe.json (the vector instructions per loop trip of each probe, counted
    from the same source's assembly)."""
    import json
    os.makedirs(BUILD, exist_ok=True)
    asm = os.path.join(BUILD, "valu_mix.s")
    r = subprocess.run([HIPCC, *CFLAGS, "--cuda-device-only", "-S", PROBE_SRC, "-o", asm], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed on {PROBE_SRC}:\n{r.stderr}")
    counts = loop_valu_counts(open(asm).read())
    per_mix = {}
    for name, n in counts.items():
        for k, mix in PROBE_KERNELS.items():
            if k in name:
                if len(n) != 1:
                    raise RuntimeError(f"{k}: expected one loop, found {len(n)}")
                per_mix[mix] = n[0]
    if sorted(per_mix) != sorted(PROBE_KERNELS.values()):
        raise RuntimeError(f"probe loops not found in the assembly: {counts}")
    tmp = PROBE_LIB + ".tmp"
    r = subprocess.run([HIPCC, *CFLAGS, "-shared", PROBE_SRC, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {PROBE_SRC}:\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    with open(PROBE_COUNTS, "w") as f:
        json.dump({"valu_per_loop_trip": {str(k): v for k, v in sorted(per_mix.items())}}, f)
    return PROBE_LIB


if __name__ == "__main__":
    build(extra=sys.argv[1:], verbose=True)
    build_probe()
