"""Benchmark of the Dust gradient estimator on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--no-cpu-baseline]

A step is one full estimate (every stage of the hot path) over one batch of
synthetic inputs already resident in HBM: for the LM-head workloads, the
per-token estimator kernel (noise, clean statistics, perturbed losses,
rewards, reward-weighted noise sum) followed by the weight-gradient outer
product.  The default workload is the fp32 LM head with T=4096 tokens (2x2048),
d=512, V=8192, K=256 draws, sigma=1e-2.

Prints one JSON line: token-draws/s (T*K per step), the per-stage times, the
roofline of the dominant kernel and the oracle timed on the host cores on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks and unit counts.
HBM_PEAK_GBS = 8000.0
N_CU, CLOCK_GHZ, LANES_PER_CU = 256, 2.4, 64
VALU_PEAK_GSLOT = N_CU * LANES_PER_CU * CLOCK_GHZ  # 39321.6 G lane-slots/s (full-rate, unpacked)

# Algorithmic VALU work of one channel-draw of the head estimator, in full-rate
# lane-slots (a quarter-rate instruction counts 4): Philox4x32-10 gives four
# channels for 10 rounds x (2 32x32->64 products at 4 slots + 2 three-way xors)
# = 100 slots -> 25; Box-Muller gives two channels for 4 transcendentals (log2,
# sqrt, sin, cos) at 4 slots + 2 int->float conversions + 2 scalings + 2
# products = 22 -> 11; the perturbed-loss term sum_v p_v expm1(sigma a_v) with
# a degree-5 polynomial = 5 fma + 1 mul + 1 fma = 7; the running sum r*a = 1.
SLOTS_PER_CHANNEL_DRAW = 25 + 11 + 7 + 1

WORKLOAD_NAMES = {
    1: "LM-head estimator fp32 logits: T=256, d=64, V=512, K=64, sigma=1e-2, uniform labels",
    2: "LM-head estimator fp32 logits: T=4096 (2x2048), d=512, V=8192, K=256, sigma=1e-2, Zipf(1.1) labels",
    4: "243M-shape LM head bf16 logits: T=8192 (4x2048), d=1024, V=50304, K=16, sigma=5e-3, Zipf(1.1) labels",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=2, choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    return ap.parse_args()


def cpu_baseline(case, target_s):
    """The oracle, as it stands, on a bounded sample of tokens of the same workload."""
    import oracle

    z = case["logits"].astype(np.float64) if "logits" in case else (
        (case["logits_bf16"].astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    K, sigma = case["K"], case["sigma"]
    ntok = 8
    while True:
        t0 = time.perf_counter()
        oracle.head_estimate(z[:ntok], case["labels"][:ntok], K, sigma, case["seed_noise"], case["layer"])
        el = time.perf_counter() - t0
        if el >= target_s / 3 or ntok >= case["T"]:
            break
        ntok = min(case["T"], int(ntok * max(2.0, target_s / max(el, 1e-3))))
    threads = oracle.num_threads()
    return {"value": ntok * K / el, "unit": "token-draws/s", "cores": threads, "kind": "oracle",
            "sample": f"first {ntok} of {case['T']} tokens x all {K} draws (full vocabulary), "
                      f"fp64 C loops, {el:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported by this build "
              "(the estimator shards by tokens or draws with one all-reduce of G_W; not built here)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import zeroth_order_activation_amd as dust

    def gpu_matmul(X, W):
        with torch.no_grad():
            return (torch.from_numpy(X).cuda() @ torch.from_numpy(W).cuda().T).cpu().numpy()

    c = synth.workload(args.workload, matmul=gpu_matmul)
    T, V, d, K, sigma = c["T"], c["V"], c["d"], c["K"], c["sigma"]
    if "logits" in c:
        z = torch.from_numpy(c["logits"]).cuda()
        dtype = "f32"
    else:
        z = torch.from_numpy(c["logits_bf16"].view(np.int16)).cuda().view(torch.bfloat16)
        dtype = "f32 (bf16 cached logits)"
    x = torch.from_numpy(c["x"]).cuda()
    y = torch.from_numpy(c["labels"]).cuda()
    gw = torch.empty((V, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(dust.head_workspace_bytes(T, V, d, K), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        dust.estimate_head(z, x, y, K, sigma, c["seed_noise"], c["layer"], grad_w=gw, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e3 in ev:  # torch creates the underlying hipEvent at its first record
        for e in e3:
            e.record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        ev[k][0].record(stream)
        dust.set_stage_event(0, ev[k][1])
        dust.set_stage_event(1, ev[k][2])
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dust.set_stage_event(0, None)
    dust.set_stage_event(1, None)
    est_ms = float(np.mean([dust.event_elapsed_ms(e[0], e[1]) for e in ev]))
    outer_ms = float(np.mean([dust.event_elapsed_ms(e[1], e[2]) for e in ev]))

    ms_per_step = wall * 1e3 / args.steps
    td = T * K
    value = td / (ms_per_step / 1e3)
    # dominant kernel: the per-token estimator
    ch_draws = T * K * V
    achieved = ch_draws * SLOTS_PER_CHANNEL_DRAW / (est_ms / 1e3) / 1e9
    logit_bytes = 4 if "logits" in c else 2
    hbm_bytes = T * V * logit_bytes + T * V * 4 + T * 4 + K * 0  # logits read, g_hat written, labels
    profiles = os.path.join(ROOT, "profiles")
    traffic = None
    tfile = os.path.join(profiles, f"traffic_head_workload{args.workload}.json")
    if os.path.exists(tfile):
        with open(tfile) as f:
            traffic = json.load(f).get("bytes_per_launch")
    out = {
        "metric": "token-draws/sec per Dust gradient estimate",
        "value": value,
        "unit": "token-draws/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded; stands in for FineWeb)",
        "config": {"workload": WORKLOAD_NAMES[args.workload], "T": T, "V": V, "d": d, "K": K, "sigma": sigma,
                   "noise_seed": c["seed_noise"], "layer": c["layer"], "data_seed": 1000 + args.workload},
        "stages_ms": {"estimator": est_ms, "outer_product": outer_ms},
        "roofline": {"bound": "alu", "kernel": "head_estimate_kernel",
                     "achieved": achieved, "peak": VALU_PEAK_GSLOT, "unit": "G lane-slots/s",
                     "frac": achieved / VALU_PEAK_GSLOT, "traffic": traffic,
                     "slots_per_channel_draw": SLOTS_PER_CHANNEL_DRAW},
        "hbm": {"algorithmic_bytes_per_step": hbm_bytes + (V * d + T * d) * 4 + T * V * 4,
                "GBps_per_step": (hbm_bytes + (V * d + T * d) * 4 + T * V * 4) / (ms_per_step / 1e3) / 1e9,
                "frac": (hbm_bytes + (V * d + T * d) * 4 + T * V * 4) / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(c, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
