"""Benchmark of the Dust gradient estimator on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--draws K5]
                    [--subset M] [--no-cpu-baseline]

A step is one full estimate -- every stage of the hot path -- over one batch of
synthetic inputs already resident in HBM:
  * LM-head workloads (1, 2, 4): the per-token estimator kernel (noise, clean
    statistics, perturbed losses, rewards, reward-weighted noise sum) and the
    weight-gradient outer product;
  * with --subset M on an LM-head workload: the vocabulary-subset estimator
    (a window of M channels per draw plus the label) and the outer product;
  * MLP-linear workloads (3, 5): GEMM1 with the noise/GELU prologue and the
    LayerNorm epilogue, GEMM2 with the log-sum-exp epilogue, the loss combine,
    the noise-regenerating reduce and the outer product.
The default workload is the 243M-shape LM head: bf16 cached logits, T=8192 tokens
(4x2048), d=1024, V=50304, K=16 full-vocabulary draws, sigma=5e-3.  The same JSON
line also carries, under "mlp_linear", the MLP-linear estimator (T=4096, d=512,
n=2048, V=8192, K=64) measured in the same process (skip with --no-mlp-line), and,
under "alu_probe", the sustained vector-ALU rate of the head's instruction mix.

Prints one JSON line: token-draws/s (T*K per step), per-stage times from HIP
events on the call's stream, the roofline of the dominant kernel and the oracle
timed on the host cores on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
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
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_F32_PEAK_TFLOPS = 157.3
N_CU, CLOCK_GHZ, LANES_PER_CU = 256, 2.4, 64
# 32-bit vector ALU: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 39.3 T lane-ops/s.
# The published fp32 vector figure, 157.3 TFLOP/s, is this times 2 (an FMA is two
# flops) times 2 (packed fp32 issues two lanes per op); the integer multiplies and
# xors of Philox and the per-channel float work here cannot use packed issue.
VALU_PEAK_GOPS = N_CU * LANES_PER_CU * CLOCK_GHZ  # 39321.6 G lane-ops/s


def head_lane_ops_per_channel_draw(deg):
    """Vector lane-ops one (token, vocabulary channel, draw) of the head estimator needs.

    Philox4x32-10 per 4 channels: the counter words token, draw and layer are the
    same across a workgroup, so round 1 costs one xor, round 2 one wide multiply
    and one xor, round 3 one multiply and two xors, round 4 two multiplies and two
    three-way xors, rounds 5-10 four ops each: 34 -> 8.5 per channel.
    Box-Muller per 2 channels: u1 (shift, convert, scale) 3, log2 1, sqrt 1,
    u2 (shift, convert, scale) 3, sin 1, cos 1, two products 2: 12 -> 6.
    Loss term p_v expm1(sigma a_v) by a degree-D Taylor polynomial with sigma
    folded into the coefficients: D-1 fma + 1 mul, then 1 fma into the sum: D + 1.
    Running sum of r a: 1.
    """
    return 8.5 + 6.0 + (deg + 1) + 1.0


def head_taylor_degree(sigma):
    """The library's choice: the lowest of 3, 4, 6 whose dropped terms stay below
    2e-5 sigma for |sigma a| <= 5.7683 sigma (else the library expm1, counted as
    degree 6)."""
    xm = sigma * 5.7683
    for D in (3, 4, 6):
        if xm ** (D + 1) / math.factorial(D + 1) * math.exp(xm) <= 2e-5 * sigma:
            return D
    return 6


# Sources that define each measured kernel: a traffic file stands only while they
# are unchanged.
KERNEL_SOURCES = {
    "head_estimate_kernel": ["head_impl.hpp", "head_f32.hip", "head_bf16.hip", "head.hip", "dust_device.hpp"],
    "head_stream_kernel": ["head_impl.hpp", "head_bf16.hip", "head.hip", "dust_device.hpp"],
    "mlp_gemm2_kernel": ["mlp.hip", "dust_device.hpp", "dust_internal.hpp"],
    "head_subset_kernel": ["head_subset.hip", "dust_device.hpp", "dust_internal.hpp"],
    "attn_v_kernel": ["attn.hip", "dust_device.hpp", "dust_internal.hpp", "launch_events.hpp"],
    "attn_k_kernel": ["attn.hip", "dust_device.hpp", "dust_internal.hpp", "launch_events.hpp"],
    "attn_q_kernel": ["attn.hip", "dust_device.hpp", "dust_internal.hpp", "launch_events.hpp"],
    "lm_gemm_x3_kernel": ["lm.hip", "lm_internal.hpp", "launch_events.hpp"],
    "lm_head_delta_kernel": ["lm.hip", "lm_internal.hpp", "launch_events.hpp"],
}


def head_kernel_name(T, V, d, logits_bf16):
    """The estimator kernel the library launches for a whole-row head call that asks for
    no fp32 g_hat (the benchmark's call): the persistent form for bf16 rows staged in LDS
    (8192 < V <= 65536, V a multiple of 8) when g_hat goes to the outer product as bf16
    pairs (2 T V d >= 4e9), else one workgroup per token."""
    stream = logits_bf16 and 8192 < V <= 65536 and V % 8 == 0 and 2.0 * T * V * d >= 4e9
    return "head_stream_kernel" if stream else "head_estimate_kernel"


def subset_kernel_name(V):
    """The subset estimator's kernels: one pass with the row in LDS up to 16384 channels,
    else a rewards pass and an accumulation pass."""
    return "head_subset_kernel" if V <= 16384 else "head_subset_rewards_kernel+head_subset_accum_kernel"


def sources_digest(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "zeroth_order_activation_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def traffic_path(kernel, workload, subset=0):
    tag = f"_m{subset}" if subset else ""
    return os.path.join(ROOT, "profiles", f"traffic_{kernel}_workload{workload}{tag}.json")


def load_traffic(kernel, workload, subset=0):
    """Measured HBM bytes per launch, or None when absent or taken on other sources."""
    p = traffic_path(kernel, workload, subset)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("sources_sha256") != sources_digest(kernel):
        return None
    return t["bytes_per_launch"]


def _counter_sums(d):
    """{(dispatch, kernel name): {counter: value}} from a rocprofv3 --pmc output folder."""
    import csv
    out = {}
    for root, _, files in os.walk(d):
        for fn in files:
            if fn.endswith("counter_collection.csv"):
                with open(os.path.join(root, fn)) as fh:
                    for r in csv.DictReader(fh):
                        k = (int(r["Dispatch_Id"]), r["Kernel_Name"])
                        out.setdefault(k, {}).setdefault(r["Counter_Name"], 0.0)
                        out[k][r["Counter_Name"]] += float(r["Counter_Value"])
    return out


def write_traffic(args):
    """Turn four rocprofv3 --pmc runs (kernel FETCH_SIZE, kernel WRITE_SIZE, and the
    same two counters on a plain copy of --copy-calibration MiB) into the traffic
    file of the workload's dominant kernel."""
    head_kernel = None
    if args.workload in (1, 2, 4):
        import synth
        w = synth.WORKLOADS[args.workload]
        if not args.subset:
            head_kernel = head_kernel_name(w["T"], w["V"], w["d"], w["logits_dtype"] == "bf16")
        elif w["V"] <= 16384:
            head_kernel = "head_subset_kernel"
        else:
            sys.exit("traffic files cover the one-pass subset kernel only (V <= 16384)")
    kernel = head_kernel if args.workload in (1, 2, 4) \
        else f"attn_{args.attn_proj}_kernel" if args.workload == 6 \
        else "lm_head_delta_kernel" if args.workload == 7 else "mlp_gemm2_kernel"
    copy_bytes = args.copy_calibration << 20
    if copy_bytes <= 0:
        sys.exit("--traffic-from needs --copy-calibration MIB (the size the copy runs used)")
    res = {}
    for ctr, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        k_runs = [v[ctr] for (_, name), v in _counter_sums(os.path.join(args.traffic_from,
                                                                       f"{sub}_w{args.workload}")).items()
                  if kernel in name and ctr in v]
        c_runs = [v[ctr] for (_, name), v in _counter_sums(os.path.join(args.traffic_from, "copy_" + sub)).items()
                  if ("copy" in name.lower() or "elementwise" in name) and ctr in v]
        if not k_runs or not c_runs:
            sys.exit(f"no {ctr} dispatches of {kernel} / the copy under {args.traffic_from}")
        kib = float(np.mean(k_runs))
        copy_kib = max(c_runs)
        factor = copy_bytes / (copy_kib * 1024.0)
        res[ctr] = {"kib_per_dispatch": kib, "dispatches": len(k_runs), "copy_kib": copy_kib,
                    "scale": factor, "bytes": kib * 1024.0 * factor}
    wl = (f"--workload {args.workload}" + (f" --subset {args.subset}" if args.subset else "")
          + (f" --attn-proj {args.attn_proj}" if args.workload == 6 else ""))
    prof = "cd /tmp && export TMPDIR=/tmp && timeout -s KILL 120 rocprofv3 --pmc {c} --output-format csv -d DIR/{n} -o {n} -- python3 $REPO/bench.py {a}"
    cmds = [prof.format(c="FETCH_SIZE", n="copy_fetch", a=f"--copy-calibration {args.copy_calibration}"),
            prof.format(c="WRITE_SIZE", n="copy_write", a=f"--copy-calibration {args.copy_calibration}"),
            prof.format(c="FETCH_SIZE", n=f"fetch_w{args.workload}",
                        a=f"{wl} --steps 1 --warmup 0 --no-cpu-baseline --no-alignment --no-mlp-line --no-alu-probe"),
            prof.format(c="WRITE_SIZE", n=f"write_w{args.workload}",
                        a=f"{wl} --steps 1 --warmup 0 --no-cpu-baseline --no-alignment --no-mlp-line --no-alu-probe"),
            f"python bench.py {wl} --traffic-from DIR --copy-calibration {args.copy_calibration}"]
    out = {"kernel": kernel, "workload": args.workload, "subset_m": args.subset, "commands": cmds,
           "copy_bytes": copy_bytes,
           "fetch": res["FETCH_SIZE"], "write": res["WRITE_SIZE"],
           "bytes_per_launch": res["FETCH_SIZE"]["bytes"] + res["WRITE_SIZE"]["bytes"],
           "sources_sha256": sources_digest(kernel)}
    with open(traffic_path(kernel, args.workload, args.subset), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def trace_summary(args):
    """Markdown summary of a rocprofv3 --kernel-trace --stats --output-format csv folder
    (the kernel stats table and each library kernel's launch shape), printed to stdout."""
    import csv
    import glob
    d = args.trace_summary
    stats = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    trace = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not stats:
        sys.exit(f"no kernel_stats.csv under {d}")
    print("| kernel | calls | total us | average us | min us | max us | % |")
    print("|---|---:|---:|---:|---:|---:|---:|")
    for r in csv.DictReader(open(stats[0])):
        nm = r["Name"] if len(r["Name"]) <= 100 else r["Name"][:97] + "..."
        print(f"| `{nm}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e3:.1f} | {float(r['AverageNs']) / 1e3:.1f} "
              f"| {float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} |")
    if trace:
        seen = {}
        for r in csv.DictReader(open(trace[0])):
            nm = r.get("Kernel_Name", "")
            if "dust" not in nm or nm in seen:
                continue
            def dims(key):
                if key in r:
                    return r[key]
                xyz = [r.get(f"{key}_{a}") for a in "XYZ"]
                return "x".join(v for v in xyz if v) if xyz[0] else "?"
            seen[nm] = (f"grid {dims('Grid_Size')}, workgroup {dims('Workgroup_Size')}, "
                        f"VGPR {r.get('VGPR_Count', r.get('Arch_VGPR_Count', '?'))}, "
                        f"AGPR {r.get('Accum_VGPR_Count', '?')}, LDS {r.get('LDS_Block_Size', r.get('Lds_Size', '?'))} B, "
                        f"scratch {r.get('Scratch_Size', r.get('Private_Segment_Size', '?'))} B")
        print()
        print("Launch shape of each library kernel:")
        print()
        for nm, shape in seen.items():
            print(f"- `{nm[:110]}`: {shape}")


def counter_summary(dirs):
    """Markdown table of rocprofv3 --pmc runs: per library kernel, each counter summed
    over the rows of a dispatch (the per-XCD and per-SE instances), averaged over the
    kernel's dispatches."""
    per = {}
    for d in dirs:
        for (disp, name), ctrs in _counter_sums(d).items():
            if "dust" not in name:
                continue
            nm = name.split("(")[0]
            for c, v in ctrs.items():
                per.setdefault(nm, {}).setdefault(c, []).append(v)
    for nm, ctrs in per.items():
        print(f"### `{nm}`")
        print()
        print("| counter | per dispatch | dispatches |")
        print("|---|---:|---:|")
        for c in sorted(ctrs):
            v = ctrs[c]
            print(f"| {c} | {sum(v) / len(v):.4g} | {len(v)} |")
        print()


WORKLOAD_NAMES = {
    1: "LM-head estimator fp32 logits: T=256, d=64, V=512, K=64, sigma=1e-2, uniform labels",
    2: "LM-head estimator fp32 logits: T=4096 (2x2048), d=512, V=8192, K=256, sigma=1e-2, Zipf(1.1) labels",
    3: "MLP-linear (W1) estimator, bf16 downstream GELU-W2-residual-LayerNorm-head: T=4096, d=512, n=2048, "
       "V=8192, K=64, sigma=1e-2, Zipf(1.1) labels",
    4: "243M-shape LM head bf16 logits: T=8192 (4x2048), d=1024, V=50304, K=16, sigma=5e-3, Zipf(1.1) labels",
    5: "MLP-linear population sweep point: T=2048, d=512, n=2048, V=8192, sigma=1e-2, K={K}",
    6: "attention {P} estimator, causal: T=4096 (2x2048), d=512, 8 heads of 64, K=64, sigma=1e-2",
    7: "full Dust step of a 2M-class causal LM (2.5M parameters: V=8192, d=128, 2 heads, 2 blocks, n=512): "
       "T=1024 (4x256), head + 4 layer-type passes + q/k/v per block, K=64 draws each, ES on the 4 residual "
       "scalars with 32 antithetic pairs, sigma=1e-2, SGD with momentum",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=4, choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--draws", type=int, default=1024, help="K for workload 5")
    ap.add_argument("--subset", type=int, default=0, metavar="M",
                    help="LM-head workloads: perturb a window of M vocabulary channels per draw (plus the "
                         "label) with the subset estimator; M a multiple of 4")
    ap.add_argument("--attn-proj", default="v", choices=("q", "k", "v"),
                    help="workload 6: the attention projection whose output is perturbed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mlp-line", action="store_true",
                    help="with the default 243M-shape head workload: skip the MLP-linear (workload 3) measurement "
                         "that the same JSON line carries under 'mlp_linear'")
    ap.add_argument("--no-alu-probe", action="store_true",
                    help="skip the vector-ALU issue-rate probe (the measured peak of the head's instruction mix)")
    ap.add_argument("--no-alignment", action="store_true",
                    help="MLP-linear workloads: skip the cosine to the backprop gradient")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a device-to-device copy of MIB MiB (to scale HBM traffic counters) and exit")
    ap.add_argument("--counter-summary", metavar="DIR", nargs="+",
                    help="print each library kernel's rocprofv3 --pmc counters (csv output under the DIRs), "
                         "summed over a dispatch and averaged over dispatches, as markdown, and exit")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="print a markdown summary of the rocprofv3 --kernel-trace --stats csv output under DIR "
                         "and exit")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="with --copy-calibration MIB: read the rocprofv3 --pmc folders DIR/fetch_wN, "
                         "DIR/write_wN (this workload) and DIR/copy_fetch, DIR/copy_write, and write the "
                         "workload's traffic file under profiles/")
    return ap.parse_args()


def cpu_baseline_head(case, target_s, subset=0):
    """The oracle, as it stands, on a bounded sample of tokens of the same workload."""
    import oracle

    z = case["logits"].astype(np.float64) if "logits" in case else (
        (case["logits_bf16"].astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    K, sigma = case["K"], case["sigma"]
    ntok = 8
    while True:
        t0 = time.perf_counter()
        if subset:
            oracle.head_estimate_subset(z[:ntok], case["labels"][:ntok], K, subset, sigma, case["seed_noise"],
                                        case["layer"])
        else:
            oracle.head_estimate(z[:ntok], case["labels"][:ntok], K, sigma, case["seed_noise"], case["layer"])
        el = time.perf_counter() - t0
        if el >= 0.7 * target_s or ntok >= case["T"]:
            break
        ntok = min(case["T"], int(ntok * max(2.0, 1.1 * target_s / max(el, 1e-3))))
    return {"value": ntok * K / el, "unit": "token-draws/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"first {ntok} of {case['T']} tokens x all {K} draws "
                      f"({f'window of {subset} channels + label' if subset else 'full vocabulary'}), "
                      f"fp64 C loops, {el:.1f} s"}


def cpu_baseline_linear(case, K, target_s):
    """The oracle on the first tokens of the workload, all their draws (beyond 1024 draws:
    the first 1024, the work being linear in K)."""
    import oracle

    Ku = min(K, 1024)
    ntok = 1
    while True:
        t0 = time.perf_counter()
        oracle.linear_estimate(case["h"], case["x_res"], case["w2_bf16"], case["w_head_bf16"], case["labels"], Ku,
                               case["sigma"], case["ln_eps"], case["seed_noise"], case["layer"],
                               tokens=np.arange(ntok))
        el = time.perf_counter() - t0
        if el >= 0.7 * target_s or ntok >= case["T"]:
            break
        ntok = min(case["T"], int(ntok * max(2.0, 1.1 * target_s / max(el, 1e-3))))
    draws = f"all {K} draws" if Ku == K else f"the first {Ku} of {K} draws (rate extrapolated: work is linear in K)"
    return {"value": ntok * Ku / el, "unit": "token-draws/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"first {ntok} of {case['T']} tokens x {draws} (clean + perturbed downstream rows), "
                      f"numpy fp64 with C noise, {el:.1f} s"}


def timed(dust, torch, step, nstage, steps):
    """Run ``steps`` steps with HIP events: [start, stage events 0..nstage-1] per step."""
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(1 + nstage)] for _ in range(steps)]
    for e_list in ev:  # torch creates the underlying hipEvent at its first record
        for e in e_list:
            e.record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        ev[k][0].record(stream)
        for s in range(nstage):
            dust.set_stage_event(s, ev[k][1 + s])
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for s in range(nstage):
        dust.set_stage_event(s, None)
    return wall, ev


class KernelTimer:
    """HIP events around every launch of chosen library kernels (the library records
    them on the stream it launches on), for per-launch durations."""

    def __init__(self, dust, torch, names, capacity):
        self.dust, self.names = dust, names
        stream = torch.cuda.current_stream()
        self.ev = {n: ([torch.cuda.Event(enable_timing=True) for _ in range(capacity)],
                       [torch.cuda.Event(enable_timing=True) for _ in range(capacity)]) for n in names}
        for a, b in self.ev.values():
            for e in a + b:
                e.record(stream)
        torch.cuda.synchronize()

    def __enter__(self):
        for n, (a, b) in self.ev.items():
            self.dust.set_kernel_events(n, a, b)
        return self

    def __exit__(self, *exc):
        self.ms = {}
        for n, (a, b) in self.ev.items():
            cnt = self.dust.kernel_event_count(n)
            self.dust.set_kernel_events(n, None, None)
            self.ms[n] = [self.dust.event_elapsed_ms(a[j], b[j]) for j in range(cnt)]
        return False


def run_head(args, c, dust, torch):
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
    m = args.subset
    if m:
        if m % 4 or m <= 0:
            sys.exit("--subset M needs a positive multiple of 4")
        ws = torch.empty(dust.head_subset_workspace_bytes(T, V, d, K), dtype=torch.uint8, device="cuda")

        def step():
            dust.estimate_head_subset(z, x, y, K, m, sigma, c["seed_noise"], c["layer"], grad_w=gw, workspace=ws)
    else:
        ws = torch.empty(dust.head_workspace_bytes(T, V, d, K), dtype=torch.uint8, device="cuda")

        def step():
            dust.estimate_head(z, x, y, K, sigma, c["seed_noise"], c["layer"], grad_w=gw, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    kern = "head_subset" if m and m // 4 < (V + 3) // 4 else "head"
    names = ["outer"] + ([kern] if kern == "head" else [])
    with KernelTimer(dust, torch, names, args.steps) as kt:
        wall, ev = timed(dust, torch, step, 2, args.steps)
    est_ms = float(np.mean([dust.event_elapsed_ms(e[0], e[1]) for e in ev]))
    outer_ms = float(np.mean([dust.event_elapsed_ms(e[1], e[2]) for e in ev]))
    ms_per_step = wall * 1e3 / args.steps
    # the estimator kernel's own launches (HIP events around each on the call's stream);
    # the subset estimator's passes are timed together by the stage events
    kern_ms = float(np.mean(kt.ms["head"])) if kt.ms.get("head") else est_ms
    outer_main_ms = float(np.mean(kt.ms["outer"])) if kt.ms.get("outer") else None
    deg = head_taylor_degree(sigma)
    ops = head_lane_ops_per_channel_draw(deg)
    # channels perturbed per (token, draw): the vocabulary, or the window (the label,
    # perturbed besides when it falls outside, is not counted)
    nq = (V + 3) // 4
    covers = not m or m // 4 >= nq
    per_draw = V if covers else m
    kernel = head_kernel_name(T, V, d, "logits" not in c) if covers else subset_kernel_name(V)
    achieved = T * K * per_draw * ops / (kern_ms / 1e3) / 1e9
    lb = 4 if "logits" in c else 2
    # bytes every step must move at least once: logits read, g_hat written and read back,
    # x read, grad_w written, labels read
    alg_bytes = T * V * lb + 2 * T * V * 4 + T * d * 4 + V * d * 4 + T * 4
    # the estimator kernel alone: logits and labels in, g_hat and rewards out
    kern_bytes = T * V * lb + T * V * 4 + T * 4 + K * T * 4
    out = {
        "dtype": dtype,
        "stages_ms": {"estimator": est_ms, "outer_product": outer_ms},
        "roofline": {"bound": "alu", "kernel": kernel, "achieved": achieved,
                     "peak": VALU_PEAK_GOPS, "unit": "G lane-ops/s", "frac": achieved / VALU_PEAK_GOPS,
                     "traffic": load_traffic(kernel, args.workload, 0 if covers else m),
                     "lane_ops_per_channel_draw": ops, "taylor_degree": deg,
                     "channel_draws_per_launch": T * K * per_draw, "kernel_ms": kern_ms,
                     "kernel_ms_source": "HIP events around each launch of the estimator kernel"
                     if kern_ms is not est_ms else "HIP stage events around the estimator passes",
                     "algorithmic_bytes_per_launch": kern_bytes,
                     "hbm_GBps": kern_bytes / (kern_ms / 1e3) / 1e9,
                     "hbm_frac": kern_bytes / (kern_ms / 1e3) / 1e9 / HBM_PEAK_GBS},
        "hbm": {"algorithmic_bytes_per_step": alg_bytes, "GBps": alg_bytes / (ms_per_step / 1e3) / 1e9,
                "frac": alg_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS,
                "estimator_kernel_GBps": kern_bytes / (kern_ms / 1e3) / 1e9},
    }
    if outer_main_ms is not None:
        fl = 2.0 * T * V * d
        out["outer_product"] = {"kernel": "outer_x3_kernel", "ms_main_kernel": outer_main_ms,
                                "ms_stage": outer_ms, "flops": fl,
                                "issued_bf16_TFLOPs": 3 * fl / (outer_ms / 1e3) / 1e12,
                                "frac_bf16_peak_issued": 3 * fl / (outer_ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                                "note": "G_W = G^T X as three bf16 products (hi/lo pairs) with fp32 accumulation"}
    return ms_per_step, out


def analytic_alignment(c, gw, K, torch):
    """Cosine of the estimate to the backprop gradient of sum_t CE_t w.r.t. W1 (fp64
    autograd through the unrounded downstream GELU -> W2 -> +x -> LayerNorm -> head -> CE),
    and the alignment law 1/sqrt(1 + c/K) of the TL;DR page (section 2, c_max = 1) with
    c = (n + 1) sum_t |u_t|^2 |g_t|^2 / |G|_F^2 (the estimator's covariance in the linear
    regime).  Measurement only; outside the timed region."""
    f64 = torch.float64
    dev = gw.device

    def bf16v(bits):
        return torch.from_numpy((bits.astype(np.uint32) << 16).view(np.float32)).to(dev, f64)

    h = torch.from_numpy(c["h"]).to(dev, f64).requires_grad_(True)
    xr = torch.from_numpy(c["x_res"]).to(dev, f64)
    u = torch.from_numpy(c["u"]).to(dev, f64)
    w2, wh = bf16v(c["w2_bf16"]), bf16v(c["w_head_bf16"])
    y = torch.from_numpy(c["labels"].astype(np.int64)).to(dev)
    m = 0.5 * h * (1.0 + torch.erf(h / math.sqrt(2.0)))
    f = torch.nn.functional.layer_norm(xr + m @ w2.T, (xr.shape[1],), eps=c["ln_eps"])
    loss = torch.nn.functional.cross_entropy(f @ wh.T, y, reduction="sum")
    (g,) = torch.autograd.grad(loss, h)
    G = g.T @ u
    n = g.shape[1]
    cl = float((n + 1) * ((u * u).sum(1) * (g * g).sum(1)).sum() / (G * G).sum())
    est = gw.to(f64)
    cos = float((est * G).sum() / (est.norm() * G.norm()))
    return {"cosine": cos, "predicted": 1.0 / math.sqrt(1.0 + cl / K), "c": cl, "K": K,
            "reference": "fp64 autograd gradient of sum_t CE_t w.r.t. W1 (unrounded downstream)"}


def cpu_baseline_attn(case, target_s, proj):
    """The oracle on all tokens of the workload and its first draws (the work is linear in K)."""
    import oracle

    K = case["K"]
    kd = 1
    while True:
        t0 = time.perf_counter()
        oracle.attn_estimate(proj, case["q"], case["k"], case["v"], case["e"], case["S"], case["H"], kd,
                             case["sigma"], case["seed_noise"], case["layer"])
        el = time.perf_counter() - t0
        if el >= 0.7 * target_s or kd >= K:
            break
        kd = min(K, int(kd * max(2.0, 1.1 * target_s / max(el, 1e-3))))
    return {"value": case["T"] * kd / el, "unit": "token-draws/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"all {case['T']} tokens x the first {kd} of {K} draws (two causal attentions per draw, "
                      f"numpy fp64; rate extrapolated: work is linear in K), {el:.1f} s"}


def cpu_baseline_lm(case, target_s):
    """The oracle's full step on the workload with the first draws of every pass (and as
    many ES pairs); the work is linear in K and M, so the rate is per token-draw."""
    import oracle
    from oracle import lm

    ocfg = lm.LMConfig(case["V"], case["d"], case["H"], case["L"], case["n"], case["S"])
    T, L = case["T"], case["L"]
    sig = dict.fromkeys(lm.ALL_TYPES, case["sigma"])
    kd = 1
    while True:
        t0 = time.perf_counter()
        lm.estimate(ocfg, case["params"], case["tokens"], case["labels"], kd, kd, sig, case["sigma_es"],
                    case["seed_noise"])
        el = time.perf_counter() - t0
        if el >= 0.7 * target_s or kd >= case["K"]:
            break
        kd = min(case["K"], int(kd * max(2.0, 1.1 * target_s / max(el, 1e-3))))
    td = ((5 + 3 * L) * kd + 2 * kd) * T
    return {"value": td / el, "unit": "token-draws/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"the full step on all {T} tokens with {kd} draws per pass and {kd} ES pairs "
                      f"({td} token-draws: per draw a full fp64 forward in numpy for the layer-type and ES "
                      f"passes, one causal attention for q/k/v, the C head estimator), {el:.1f} s"}


def lm_change_gemm_flops(c):
    """Flops of the change-row GEMMs of one step (2 x rows x out x in each): per draw of
    each layer-type pass the blocks after its first perturbed point (block 0 keeps only
    what follows the point), the ES members likewise (block 0's attention branch has no
    change yet).  The head's change is the fused head kernel's."""
    T, d, n, L, K, M = c["T"], c["d"], c["n"], c["L"], c["K"], c["M"]
    attn, mlp = 2 * 4 * d * d, 2 * 2 * n * d
    head = 0
    full = attn + mlp
    first = {"emb": full, "o": mlp, "up": mlp // 2, "down": 0, "es": mlp}
    per_draw = {k: v + (L - 1) * full + head for k, v in first.items()}
    passes = K * T * (per_draw["emb"] + per_draw["o"] + per_draw["up"] + per_draw["down"])
    return passes + 2 * M * T * per_draw["es"]


def lm_change_gemm_bytes(c):
    """HBM bytes of the change-row GEMMs of one step: each reads its change rows (K_in
    floats) and writes its output rows (N_out floats); the weights' bf16 parts are small and
    stay in cache.  The query, key and value changes are one product (d in, 3d out), then W_O
    (d in, d out).  Blocks as in lm_change_gemm_flops."""
    T, d, n, L, K, M = c["T"], c["d"], c["n"], c["L"], c["K"], c["M"]
    attn, mlp = (d + 3 * d) + (d + d), 2 * (d + n)
    full = attn + mlp
    first = {"emb": full, "o": mlp, "up": n + d, "down": 0, "es": mlp}
    per_draw = {k: v + (L - 1) * full for k, v in first.items()}
    rows = K * T * (per_draw["emb"] + per_draw["o"] + per_draw["up"] + per_draw["down"]) + 2 * M * T * per_draw["es"]
    return 4 * rows


def run_lm(args, c, dust, torch):
    """Full Dust step: clean forward, head, the four layer-type passes, attention
    internals, residual-scalar ES, SGD with momentum."""
    cfg = dust.lm_config(c["V"], c["d"], c["H"], c["L"], c["n"], c["S"], c["B"])
    # the estimates are gradients of the summed (not mean) loss over T tokens: small rates
    hp = dust.lm_hparams(c["K"], c["M"], c["sigma"], c["sigma_es"], lr=1e-5, lr_scalar=1e-7, momentum=0.9)
    params = torch.from_numpy(c["params"]).cuda()
    tok = torch.from_numpy(c["tokens"]).cuda()
    lab = torch.from_numpy(c["labels"]).cuda()
    mom = torch.zeros_like(params)
    grads = torch.empty_like(params)
    ws = torch.empty(dust.lm_workspace_bytes(cfg, hp), dtype=torch.uint8, device="cuda")

    def step():
        dust.lm_step(cfg, hp, params, mom, tok, lab, c["seed_noise"], grads=grads, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for el in ev:
        for x in el:
            x.record(stream)
    timed = {"lm_gemm": [[torch.cuda.Event(enable_timing=True) for _ in range(1024)] for _ in range(2)],
             "lm_head": [[torch.cuda.Event(enable_timing=True) for _ in range(64)] for _ in range(2)]}
    for pair in timed.values():
        for x in pair[0] + pair[1]:
            x.record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for kk in range(args.steps):
        ev[kk][0].record(stream)
        for j, st in enumerate((4, 5, 6, 7)):
            dust.set_stage_event(st, ev[kk][1 + j])
        if kk == args.steps - 1:  # the last timed step also times each launch of two kernels
            for name, (a, b) in timed.items():
                dust.set_kernel_events(name, a, b)
        step()
        ev[kk][5].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {}
    for name, (a, b) in timed.items():
        n_l = dust.kernel_event_count(name)
        dust.set_kernel_events(name, None, None)
        per[name] = (n_l, float(sum(dust.event_elapsed_ms(a[j], b[j]) for j in range(n_l))))
    for st in (4, 5, 6, 7):
        dust.set_stage_event(st, None)
    names = ("clean_forward", "head_pass", "layer_type_passes", "attention_internals", "es_and_sgd")
    stages = {nm: float(np.mean([dust.event_elapsed_ms(x[j], x[j + 1]) for x in ev])) for j, nm in enumerate(names)}
    ms_per_step = wall * 1e3 / args.steps
    T, L = c["T"], c["L"]
    td = ((5 + 3 * L) * c["K"] + 2 * c["M"]) * T
    ce = dust.lm_forward(cfg, params, tok, lab)
    torch.cuda.synchronize()
    # fused head change: per draw and token, d x Vp products on bf16 MFMA, three each (hi/lo)
    vp = -(-c["V"] // 128) * 128
    head_flops = (4 * c["K"] + 2 * c["M"]) * T * vp * c["d"] * 2 * 3
    lines = {
        "lm_head_delta_kernel": {"bound": "mfma", "flops": head_flops, "peak": MFMA_BF16_PEAK_TFLOPS,
                                 "launches": per["lm_head"][0], "ms": per["lm_head"][1],
                                 "note": "issued bf16 MFMA flops (three products per fp32 product) of the fused "
                                         "head change over its launches' durations (HIP events around each "
                                         "launch of the last timed step)"},
        "lm_gemm_x3_kernel": {"bound": "hbm", "bytes": lm_change_gemm_bytes(c), "peak": HBM_PEAK_GBS,
                              "launches": per["lm_gemm"][0], "ms": per["lm_gemm"][1],
                              "note": "change rows read and written by every launch of the change-row GEMM in one "
                                      "step (about 95 issued bf16 flops per byte: HBM-bound) over the summed "
                                      "durations of those launches (HIP events around each launch)"},
    }
    roof = {}
    for name, x in lines.items():
        nl = max(x["launches"], 1)
        if x["bound"] == "hbm":
            ach = x["bytes"] / (x["ms"] / 1e3) / 1e9
            unit, per_launch = "GB/s", {"bytes_per_launch": x["bytes"] / nl}
        else:
            ach = x["flops"] / (x["ms"] / 1e3) / 1e12
            unit, per_launch = "TFLOP/s", {"flops_per_launch": x["flops"] / nl}
        roof[name] = {"bound": x["bound"], "kernel": name, "achieved": ach, "peak": x["peak"], "unit": unit,
                      "frac": ach / x["peak"], "traffic": load_traffic(name, args.workload), **per_launch,
                      "launches_per_step": x["launches"], "kernel_ms": x["ms"] / nl, "kernel_ms_per_step": x["ms"],
                      "note": x["note"]}
    dom = max(roof, key=lambda k_: roof[k_]["kernel_ms_per_step"])
    out = {
        "dtype": "f32 (clean forward on fp32 MFMA; change rows on bf16x3 MFMA)",
        "token_draws_per_step": td,
        "stages_ms": stages,
        "loss_after": float(ce.mean()),
        "roofline": roof[dom],
        "roofline_other": [v_ for k_, v_ in roof.items() if k_ != dom],
    }
    return ms_per_step, td, out


def run_attn(args, c, dust, torch):
    """Attention projection estimator: rewards (attention passes), g_hat, outer product."""
    T, S, d, H, K, sigma = c["T"], c["S"], c["d"], c["H"], c["K"], c["sigma"]
    proj = args.attn_proj
    q, k, v, e, u = (torch.from_numpy(c[n]).cuda() for n in ("q", "k", "v", "e", "u"))
    gw = torch.empty((d, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(dust.attn_workspace_bytes(proj, T, S, d, H, K), dtype=torch.uint8, device="cuda")

    def step():
        dust.estimate_attn(proj, q, k, v, e, u, S, H, K, sigma, c["seed_noise"], c["layer"], grad_w=gw,
                           workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # stages: 2 after the rewards, 0 after g_hat, 1 after G_WV
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    ks, ke = ([torch.cuda.Event(enable_timing=True) for _ in range(64)] for _ in range(2))
    for x in [y for el in ev for y in el] + ks + ke:
        x.record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for kk in range(args.steps):
        ev[kk][0].record(stream)
        dust.set_stage_event(2, ev[kk][1])
        dust.set_stage_event(0, ev[kk][2])
        dust.set_stage_event(1, ev[kk][3])
        if kk == args.steps - 1:  # the last timed step also times each launch of the main kernel
            dust.set_kernel_events("attn_main", ks, ke)
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    nl = dust.kernel_event_count("attn_main")
    dust.set_kernel_events("attn_main", None, None)
    for st in (0, 1, 2):
        dust.set_stage_event(st, None)
    main_ms = float(sum(dust.event_elapsed_ms(ks[j], ke[j]) for j in range(nl)))
    att_ms = float(np.mean([dust.event_elapsed_ms(x[0], x[1]) for x in ev]))
    red_ms = float(np.mean([dust.event_elapsed_ms(x[1], x[2]) for x in ev]))
    out_ms = float(np.mean([dust.event_elapsed_ms(x[2], x[3]) for x in ev]))
    ms_per_step = wall * 1e3 / args.steps
    # bf16 MFMA work of the main kernel's launches: per (key tile <= query tile) pair of
    # 64-token tiles and head, 2 * 64^3 flops per product, three products (hi/lo pairs)
    # each: per draw one product (<a, e> for values, <a, q> or <k, a> for keys and queries);
    # per chunk of 8 draws the logits (and for keys and queries <v, e>)
    nkt = S // 64
    pairs = (T // S) * H * nkt * (nkt + 1) // 2
    per_pair = 2 * 64 ** 3 * 3
    part = {"v": nkt * H * 2 * T, "k": nkt * H * 4 * T, "q": H * T}[proj] * 4
    kc = max(1, min(64, (256 << 20) // part))
    chunks = sum(-(-min(kc, K - i0) // 8) for i0 in range(0, K, kc))
    per_chunk = 1 if proj == "v" else 2
    flops = pairs * per_pair * (K + per_chunk * chunks)
    achieved = flops / (main_ms / 1e3) / 1e12
    out = {
        "dtype": "f32 (bf16x3 MFMA products)",
        "stages_ms": {"attention_rewards": att_ms, "ghat_reduce": red_ms, "outer_product": out_ms},
        "roofline": {"bound": "mfma", "kernel": f"attn_{proj}_kernel", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": load_traffic(f"attn_{proj}_kernel", args.workload),
                     "flops_per_launch": flops / max(nl, 1), "launches_per_step": nl,
                     "kernel_ms": main_ms / max(nl, 1),
                     "note": "issued bf16 MFMA flops of the main kernel (three products per fp32 product) over "
                             "its launches' durations (HIP events around each launch of the last timed step)"},
    }
    return ms_per_step, out


def run_linear(args, c, K, dust, torch):
    T, d, n, V, sigma = c["T"], c["d"], c["n"], c["V"], c["sigma"]
    u, h, xr = (torch.from_numpy(c[k]).cuda() for k in ("u", "h", "x_res"))
    w2 = torch.from_numpy(c["w2_bf16"].view(np.int16)).cuda().view(torch.bfloat16)
    wh = torch.from_numpy(c["w_head_bf16"].view(np.int16)).cuda().view(torch.bfloat16)
    y = torch.from_numpy(c["labels"]).cuda()
    gw = torch.empty((n, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(dust.linear_workspace_bytes(T, d, n, V, K), dtype=torch.uint8, device="cuda")

    def step():
        dust.estimate_linear(u, h, xr, w2, wh, y, K, sigma, c["seed_noise"], c["layer"], ln_eps=c["ln_eps"],
                             grad_w=gw, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    rows = T * (K + 1)
    nchunks = -(-rows * d * 2 // (512 << 20)) + 2
    with KernelTimer(dust, torch, ["mlp_gemm1", "mlp_gemm2"], args.steps * nchunks) as kt:
        wall, ev = timed(dust, torch, step, 4, args.steps)
    # events: 0 start, 1 after g_hat, 2 after outer, 3 after (last) gemm1, 4 after (last) gemm2
    ms_per_step = wall * 1e3 / args.steps
    fl1 = 2.0 * rows * n * d
    fl2 = 2.0 * rows * d * V
    # per step: the sum of every row chunk's launch (HIP events around each launch)
    g1 = float(np.sum(kt.ms["mlp_gemm1"])) / args.steps
    g2 = float(np.sum(kt.ms["mlp_gemm2"])) / args.steps
    launches = len(kt.ms["mlp_gemm1"]) // args.steps
    red = float(np.mean([dust.event_elapsed_ms(e[4], e[1]) for e in ev]))
    outer = float(np.mean([dust.event_elapsed_ms(e[1], e[2]) for e in ev]))
    out = {"dtype": "bf16 GEMM operands with fp32 accumulate in the downstream; fp32 noise, rewards, g_hat, G_W"}
    out["stages_ms"] = {"gemm1_noise_gelu_w2_ln": g1, "gemm2_head_logsumexp": g2,
                        "combine_and_reduce_last_chunk": red, "outer_product": outer}
    both = (fl1 + fl2) / ((g1 + g2) / 1e3) / 1e12
    # the library's choice for the first product: at sigma 5.7683 <= 1/16 the GELU rows
    # (noise, GELU series) and the W2 + LayerNorm MFMA kernel, else one fused kernel
    g1_name = ("mlp_gelu_rows_kernel + mlp_w2ln_kernel" if sigma * 5.7683 <= 0.0625
               else "mlp_gemm1_kernel")
    out["roofline"] = {"bound": "mfma", "kernel": f"{g1_name} + mlp_gemm2_kernel", "achieved": both,
                       "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": both / MFMA_BF16_PEAK_TFLOPS,
                       "traffic": None, "flop_per_step": fl1 + fl2, "kernel_ms": g1 + g2,
                       "launches_per_step": 2 * launches,
                       "note": "the two downstream GEMMs together: their algorithmic flops (2 rows n d + 2 rows d V, "
                               "rows = T (K + 1)) over the sum of their launch durations (HIP events around each "
                               "launch, every row chunk)"}
    out["mfma_downstream"] = {
        "mlp_gemm1_kernel": {"TFLOPs": fl1 / (g1 / 1e3) / 1e12, "frac": fl1 / (g1 / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                             "ms_per_step": g1, "flop_per_step": fl1, "kernels": g1_name},
        "mlp_gemm2_kernel": {"TFLOPs": fl2 / (g2 / 1e3) / 1e12, "frac": fl2 / (g2 / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                             "ms_per_step": g2, "flop_per_step": fl2,
                             "traffic": load_traffic("mlp_gemm2_kernel", args.workload),
                             "algorithmic_bytes_per_step": rows * d * 2 + V * d * 2 + rows * 4
                             + (V + 255) // 256 * rows * 8},
        "launches_per_step_each": launches,
    }
    # bytes the step must move at least once: its inputs and G_W (F stays on chip in
    # principle; its HBM round trip is not counted)
    alg_bytes = 4 * T * (d + n + d) + 2 * d * n + 2 * V * d + 4 * T + 4 * n * d
    out["hbm"] = {"algorithmic_bytes_per_step": alg_bytes, "GBps": alg_bytes / (ms_per_step / 1e3) / 1e9,
                  "frac": alg_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS}
    if not args.no_alignment:
        out["alignment"] = analytic_alignment(c, gw, K, torch)
    return ms_per_step, out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the estimator would shard by tokens or draws with one all-reduce of G_W)",
              file=sys.stderr)
        sys.exit(2)
    if args.traffic_from:
        write_traffic(args)
        return
    if args.trace_summary:
        trace_summary(args)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    import torch
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "read_bytes": n, "write_bytes": n}), flush=True)
        return
    import synth
    import zeroth_order_activation_amd as dust

    def gpu_matmul(X, W):
        with torch.no_grad():
            return (torch.from_numpy(X).cuda() @ torch.from_numpy(W).cuda().T).cpu().numpy()

    out = measure(args, args.workload, dust, torch, synth, gpu_matmul)
    head_default = out["config"].get("V") == 50304 and not args.subset
    if out.pop("_kind") == "head" and not args.no_alu_probe:
        probe = alu_probe(torch)
        if probe is not None:
            out["alu_probe"] = probe
            r = out["roofline"]
            mix = probe["head_mix"]["channel_draws_per_s"]
            r["peak_measured_mix_G_lane_ops"] = probe["head_mix"]["G_lane_ops_per_s"]
            r["frac_of_measured_mix"] = (r["channel_draws_per_launch"] / (r["kernel_ms"] / 1e3)) / mix
            r["measured_mix_note"] = ("the estimator's channel-draws/s over those of the probe that runs the same "
                                      "per-channel-draw arithmetic (Philox, Box-Muller, degree-4 expm1 term, running "
                                      "sums) from registers only")
    if args.workload == 4 and head_default and not args.no_mlp_line:
        print("bench: 243M-shape head done; MLP-linear workload 3 next", file=sys.stderr, flush=True)
        mlp = measure(args, 3, dust, torch, synth, gpu_matmul)
        mlp.pop("_kind")
        for k in ("n_gpus", "higher_is_better", "scaling", "data", "warmup", "steps"):
            mlp.pop(k, None)
        if "alu_probe" in out:
            sus = out["alu_probe"]["mfma_bf16"]["TFLOP_per_s"]
            mlp["roofline"]["peak_measured_mfma_TFLOPs"] = sus
            mlp["roofline"]["frac_of_measured_mfma"] = mlp["roofline"]["achieved"] / sus
        out["mlp_linear"] = mlp
    print(json.dumps(out), flush=True)


def alu_probe(torch):
    """Sustained vector-ALU rates on this chip: each probe loop's vector instructions
    (counted from its own assembly at build time) x 64 lanes x waves x trips, over the
    time of a launch that fills every CU many times over."""
    lib_path = os.path.join(ROOT, "zeroth_order_activation_amd", "libdust_probe.so")
    cnt_path = os.path.join(ROOT, "zeroth_order_activation_amd", "libdust_probe.json")
    if not (os.path.exists(lib_path) and os.path.exists(cnt_path)):
        print("bench: libdust_probe.so not built; no ALU probe", file=sys.stderr, flush=True)
        return None
    import ctypes
    L = ctypes.CDLL(lib_path)
    L.dust_probe_valu_mix.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p]
    L.dust_probe_valu_mix.restype = ctypes.c_int
    with open(cnt_path) as f:
        per_trip = {int(k): v for k, v in json.load(f)["valu_per_loop_trip"].items()}
    blocks = N_CU * 32
    gin = torch.rand(2048, device="cuda") + 0.5
    gout = torch.empty(blocks * 256, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    names = {0: "fma_f32", 1: "mad_u64_u32_and_xor", 2: "log_sqrt_sin_cos_mul", 3: "head_mix"}
    iters = {0: 2048, 1: 1024, 2: 2048, 3: 32}
    res = {}
    for mix in (0, 1, 2, 3):
        for rep in range(2):  # the first launch warms up; the second is timed
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            rc = L.dust_probe_valu_mix(mix, blocks, iters[mix], ctypes.c_void_p(gin.data_ptr()),
                                       ctypes.c_void_p(gout.data_ptr()), stream)
            b.record()
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"probe mix {mix} failed: {rc}")
        ms = a.elapsed_time(b)
        waves = blocks * 4
        lane_ops = per_trip[mix] * 64 * waves * iters[mix]
        res[names[mix]] = {"valu_per_loop_trip": per_trip[mix], "ms": ms,
                           "G_lane_ops_per_s": lane_ops / (ms / 1e3) / 1e9,
                           "frac_of_unit_count_peak": lane_ops / (ms / 1e3) / 1e9 / VALU_PEAK_GOPS}
    # the head mix: 8 channel quads = 32 channel-draws per lane and loop trip
    res["head_mix"]["channel_draws_per_s"] = 32 * 256 * blocks * iters[3] / (res["head_mix"]["ms"] / 1e3)
    res["head_mix"]["valu_per_channel_draw"] = per_trip[3] / 32
    # the matrix cores: 8 independent v_mfma_f32_32x32x16_bf16 chains per wave on non-zero data
    mf_iters = 64
    for rep in range(2):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        rc = L.dust_probe_valu_mix(4, blocks, mf_iters, ctypes.c_void_p(gin.data_ptr()),
                                   ctypes.c_void_p(gout.data_ptr()), stream)
        b.record()
        torch.cuda.synchronize()
        if rc != 0:
            raise RuntimeError(f"probe mix 4 failed: {rc}")
    ms = a.elapsed_time(b)
    tf = 2.0 * 32 * 32 * 16 * 8 * mf_iters * blocks * 4 / (ms / 1e3) / 1e12
    res["mfma_bf16"] = {"ms": ms, "TFLOP_per_s": tf, "frac_of_peak": tf / MFMA_BF16_PEAK_TFLOPS,
                        "note": "register-only loop of v_mfma_f32_32x32x16_bf16, 8 independent accumulators per "
                                "wave, operands from random data: the sustained matrix-core rate"}
    res["note"] = ("register-only loops over 8192 workgroups of 256 lanes; rates are vector instructions x 64 lanes "
                   "per second (one issue slot per instruction), against 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz")
    return res


def measure(args, wid, dust, torch, synth, gpu_matmul):
    """One workload: its timed steps, roofline and (unless --no-cpu-baseline) the oracle
    timed on the host cores.  Returns the JSON object of its line."""
    print(f"bench: workload {wid}: inputs", file=sys.stderr, flush=True)
    args = argparse.Namespace(**{**vars(args), "workload": wid})
    c = synth.workload(wid, matmul=gpu_matmul)
    name = WORKLOAD_NAMES[wid]
    if args.subset and c["kind"] != "head":
        sys.exit("--subset applies to the LM-head workloads (1, 2, 4)")
    sub = args.subset
    if c["kind"] == "head":
        K = c["K"]
        ms, extra = run_head(args, c, dust, torch)
        cfg = {"workload": name, "T": c["T"], "V": c["V"], "d": c["d"], "K": K, "sigma": c["sigma"]}
        if sub:
            cfg["workload"] = name + f"; vocabulary subset: window of {sub} channels per draw + label"
            cfg["subset_m"] = sub
    elif c["kind"] == "lm":
        ms, td, extra = run_lm(args, c, dust, torch)
        cfg = {"workload": name, "T": c["T"], "V": c["V"], "d": c["d"], "H": c["H"], "L": c["L"], "n": c["n"],
               "S": c["S"], "K": c["K"], "M": c["M"], "sigma": c["sigma"], "sigma_es": c["sigma_es"]}
        c["layer"] = "per pass (1 embedding, 2 head, 3 ES, 16 (l + 1) + type)"
    elif c["kind"] == "attn_v":
        K = c["K"]
        name = name.format(P={"q": "query-projection (W_Q)", "k": "key-projection (W_K)",
                              "v": "value-projection (W_V)"}[args.attn_proj])
        ms, extra = run_attn(args, c, dust, torch)
        cfg = {"workload": name, "T": c["T"], "S": c["S"], "d": c["d"], "H": c["H"], "K": K, "sigma": c["sigma"],
               "projection": args.attn_proj}
    else:
        K = c["K"] if isinstance(c["K"], int) else args.draws
        name = name.format(K=K)
        ms, extra = run_linear(args, c, K, dust, torch)
        cfg = {"workload": name, "T": c["T"], "d": c["d"], "n": c["n"], "V": c["V"], "K": K, "sigma": c["sigma"]}
    print(f"bench: workload {wid}: {ms:.3f} ms per step", file=sys.stderr, flush=True)
    cfg.update({"noise_seed": c["seed_noise"], "layer": c["layer"], "data_seed": 1000 + wid})
    out = {
        "metric": "token-draws/sec per Dust gradient estimate; % of HBM BW / MFMA peak",
        "value": (td if c["kind"] == "lm" else c["T"] * K) / (ms / 1e3),
        "unit": "token-draws/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": extra.pop("dtype"),
        "data": "synthetic (seeded; stands in for FineWeb)",
        "config": cfg,
        "_kind": c["kind"],
    }
    out.update(extra)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = (cpu_baseline_lm(c, args.cpu_seconds) if c["kind"] == "lm"
                               else cpu_baseline_head(c, args.cpu_seconds, sub) if c["kind"] == "head"
                               else cpu_baseline_attn(c, args.cpu_seconds, args.attn_proj) if c["kind"] == "attn_v"
                               else cpu_baseline_linear(c, K, args.cpu_seconds))
    return out


if __name__ == "__main__":
    main()
