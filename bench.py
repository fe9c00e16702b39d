#!/usr/bin/env python3
"""Benchmark of the block-scaled FP4 MoE layer on one MI355X.

Metric: microseconds per MoE layer at M=1 with cold caches, plus the fraction
of HBM peak achieved on the unique routed FP4 weight + scale bytes.  With a
many-token workload (--workload mxfp4_prefill_e128) the same contract runs the
grouped path and prices its dominant kernel against the bf16 matrix-core peak;
with --act mxfp8 (the W4A8-MX variant: MXFP8 activations on the scaled
matrix instruction) against the fp8 matrix-core peak.

A step is one layer call (both kernels) on one batch of synthetic inputs
already resident in HBM.  Steps rotate through groups of disjoint experts
(each group has the workload's top-k size and weights from the workload's own
softmax routing), so that between two uses of an expert every other group
has streamed through: with the 512-expert NVFP4 workload that is ~700 MB of
other weights, more than L2 plus the 256 MB Infinity Cache, so every step
reads its experts from HBM.  A timed region is K back-to-back steps (graph
replays) between two HIP events on the launch stream (one event pair per
region, since a pair around a single launch adds ~4 us of its own); it runs
in several rounds, each right after a 1 GiB read + write scrub that evicts L2
and the Infinity Cache, and the median round is reported with every round's
value.  FC1-only and FC2-only regions over the same rotation give each
kernel's time per launch.  The roofline's `achieved` comes from the
rocprofv3 mean duration of the dominant kernel recorded for this same
command under profiles/ (used only while the kernel's HIP sources are
unchanged), with this run's event-timed figure beside it.  Correctness
against the CPU oracle gates the timing.

The default workload is the metric's configuration: the E256/H7168/I256
MXFP4 layer shard at M = 1, top-8 (the largest M = 1 configuration).

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--rounds 7] [--workload NAME] [--act bf16|mxfp8]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, published
MFMA_FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 matrix cores, published (fp8 x fp4 runs at this rate)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mxfp4_shard_e256_m1")
    ap.add_argument("--act", default="bf16", choices=("bf16", "mxfp8"),
                    help="activation format of the grouped path (mxfp8: W4A8-MX, MXFP4 weights)")
    ap.add_argument("--scales", default=None, choices=("plain", "csf"),
                    help="resident scale format (default: the workload's; csf = compressed scales)")
    ap.add_argument("--rounds", type=int, default=7,
                    help="timed rounds per region, each after a cache scrub; the median is reported")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-check", action="store_true", help="skip the oracle check (profiling runs)")
    ap.add_argument("--shape", default=None,
                    help="launch shape kl1,r1,r2 (FC1 chunks per wave, FC1 rows, FC2 rows; 0 = built-in)")
    ap.add_argument("--extra", action="store_true", help="also time warm-cache calls and a copy probe")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run 5 copies of a 256 MiB buffer (reference for profiler byte counters)")
    return ap.parse_args()


def copy_probe():
    """A plain device copy of known size: 256 MiB read + 256 MiB written per
    dispatch.  Profiler byte counters of this run calibrate the ones of the
    layer's kernels."""
    import torch
    src = torch.ones(1 << 26, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_per_dispatch": {"read": src.numel() * 4, "write": dst.numel() * 4}}))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def routed_bytes(wl, ids, d=None, csf=False):
    """Unique valid experts and their algorithmic weight bytes: codes plus
    scales.  With compressed scales (csf) a row's scales cost its CSF words
    (4 bytes per 24 chunks of 32 elements for MXFP4, per 3 chunks for NVFP4:
    the base byte and the offsets), and an exception row its plain scale
    bytes too."""
    import numpy as np
    flat = ids.reshape(-1).astype(np.int64)
    uniq = np.unique(flat[(flat >= 0) & (flat < wl.E)])
    G = wl.G
    glob = 4 if wl.fmt == "nvfp4" else 0
    U = len(uniq)
    if not csf:
        w13 = 2 * wl.I * (wl.H // 2 + wl.H // G)
        w2 = wl.H * (wl.I // 2 + wl.I // G)
        return U, U * (w13 + glob), U * (w2 + glob)
    reach = 1 if wl.fmt == "mxfp4" else 15
    out = []
    for key, K in (("w13_scales", wl.H), ("w2_scales", wl.I)):
        sc = d[key][uniq].astype(np.int32)
        rows = sc.shape[0] * sc.shape[1]
        lo, hi = sc.min(axis=2), sc.max(axis=2)
        exc = int(np.count_nonzero((lo == 255) | (hi - lo > reach)))
        nC = K // 32
        per_row = K // 2 + 4 * -(-nC // (24 if wl.fmt == "mxfp4" else 3))
        out.append(rows * per_row + exc * (K // G) + U * glob)
    return U, out[0], out[1]


def cold_groups(wl, d, dev):
    """Route tables for the rotation: the workload's own table first, then
    tables whose valid ids are disjoint groups of experts not used by it."""
    import numpy as np
    import torch

    ids0, w0 = d["ids"], d["w"]
    flat = ids0.reshape(-1)
    valid = flat[(flat >= 0) & (flat < wl.E)]
    per = len(np.unique(valid))
    rest = np.setdiff1d(np.arange(wl.E), valid)
    rng = np.random.default_rng(wl.seed & 0xFFFF)
    rest = rng.permutation(rest)
    tables = [(ids0, w0)]
    if per:
        first_slot = {}
        for pos, e in enumerate(flat):
            if 0 <= e < wl.E and e not in first_slot:
                first_slot[e] = pos
        for g in range(len(rest) // per):
            repl = dict(zip(first_slot.keys(), rest[g * per:(g + 1) * per]))
            ids = np.array([repl.get(int(e), e) if 0 <= e < wl.E else e for e in flat],
                           dtype=ids0.dtype).reshape(ids0.shape)
            tables.append((ids, w0))
    return [(torch.from_numpy(np.ascontiguousarray(i)).to(dev), torch.from_numpy(np.ascontiguousarray(w)).to(dev))
            for i, w in tables]


def run_env(torch) -> dict:
    """GPU and host identity for the record (the commit when a git checkout is present)."""
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    commit = None
    try:
        import subprocess
        commit = subprocess.run(["git", "rev-parse", "--short", "HEAD"], capture_output=True, text=True,
                                cwd=os.path.dirname(os.path.abspath(__file__)), timeout=10).stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        pass
    props = torch.cuda.get_device_properties(0)
    return {"gpu": torch.cuda.get_device_name(0), "gpu_arch": getattr(props, "gcnArchName", None),
            "gpu_cus": props.multi_processor_count, "host_cpu": cpu_model, "host_cpus": os.cpu_count(),
            "commit": commit}


def main():
    args = parse()
    if args.copy_probe:
        copy_probe()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}); "
              "the layer would shard by experts or by I with one exchange of the [M, H] output.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_scaled_fp4_gather_amd import moe, synth

    wl = synth.WORKLOADS[args.workload]
    log(f"[bench] workload {wl.name}: {wl.description}")
    d = synth.generate(wl)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    scales = args.scales or wl.scales
    desc = moe.Desc(wl.fmt, wl.E, wl.H, wl.I, wl.k, max(wl.M, 1), args.act, scales=scales)

    def dt(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    layer = moe.Fp4MoE(desc, dt(d["w13_codes"]), dt(d["w13_scales"]), dt(d["w2_codes"]),
                       dt(d["w2_scales"]), dt(d["g13"]) if d["g13"] is not None else None,
                       dt(d["g2"]) if d["g2"] is not None else None, device=dev)
    x = dt(d["x"]).view(torch.bfloat16)
    ids = dt(d["ids"])
    w = dt(d["w"])
    out = torch.empty((wl.M, wl.H), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    log("[bench] prepared")
    tuning = moe.Tuning(*[int(v) for v in args.shape.split(",")], 0) if args.shape else None
    plan = moe.plan(desc, wl.M, tuning)
    log(f"[bench] {'grouped' if plan.path == moe.PATH_GROUPED else 'decode'} path, "
        f"shape kl1={plan.fc1_chunks_per_wave} r1={plan.fc1_rows} r2={plan.fc2_rows}")

    # the library's choice of path for this M (moe_fp4_plan)
    grouped = plan.path == moe.PATH_GROUPED
    a8 = grouped and args.act == "mxfp8"  # the decode path keeps bf16 activations
    sample = np.arange(wl.M)
    if grouped:
        rs = np.random.default_rng(wl.seed & 0xFFFF)
        sample = np.unique(np.concatenate([[0, wl.M - 1], rs.integers(0, wl.M, 6)]))

    check = None
    if not args.no_check:
        import oracle
        sub = dict(d, x=d["x"][sample], ids=d["ids"][sample], w=d["w"][sample])
        acc = oracle.forward_w4a8(wl.fmt, sub) if a8 else oracle.forward_f32(wl.fmt, sub)[0]
        layer(x, ids, w, out=out, tuning=tuning)
        torch.cuda.synchronize()
        g = oracle.bf16_bits_to_f32(out.view(torch.int16).cpu().numpy().view(np.uint16)[sample]).astype(np.float64).ravel()
        r = acc.astype(np.float64).ravel()
        rms = float(np.sqrt(np.mean(r * r)))
        cos = float(g @ r / (np.linalg.norm(g) * np.linalg.norm(r)))
        err = np.abs(g - r)
        _, ex = np.frexp(np.abs(r))
        half_ulp = np.where(r == 0, 0.0, np.ldexp(1.0, ex - 9))
        mx = float(err.max() / rms)
        beyond = float(np.max(err - half_ulp) / rms)
        check = {"tokens_checked": int(len(sample)), "cos": round(cos, 8), "maxabs_over_rms": round(mx, 6),
                 "beyond_bf16_rounding_over_rms": round(beyond, 6),
                 "pass": bool(cos >= 0.99995 and beyond <= (0.1 if a8 else 2e-2))}
        log(f"[bench] oracle check {check}")
        if not check["pass"]:
            print(json.dumps({"error": "correctness check failed", "check": check}))
            sys.exit(1)

    K, W = args.steps, args.warmup
    # decode: rotate through disjoint expert groups so weights come from HBM;
    # grouped: every expert is active and all weights together exceed the caches
    groups = cold_groups(wl, d, dev) if not grouped else [(ids, w)]
    log(f"[bench] {len(groups)} disjoint expert groups in rotation")

    def call(g, phases=None):
        layer(x, g[0], g[1], out=out, tuning=tuning, phases=phases)

    def graph_len(K):
        """Steps per captured graph: K itself up to 512, else the largest
        divisor of K in [64, 512] (so exactly K steps run), else 512 with a
        final shorter graph for the rest."""
        if K <= 512:
            return K
        for n in range(512, 63, -1):
            if K % n == 0:
                return n
        return 512

    # A read + write pass over 1 GiB between replays evicts the 8 x 4 MB L2s
    # and the 256 MB Infinity Cache, so every timed replay starts cold.
    scrub = torch.zeros(1 << 28, dtype=torch.float32, device=dev)

    def region(phases=None, rotate=True, rounds=None, cold=True):
        """Exactly K steps as graph replays (steps cycle through the expert
        rotation), between one event pair on the launch stream, in `rounds`
        rounds each preceded by a cache scrub (cold=True).  Returns (median
        us per step over the rounds, the rounds' us per step, median wall s
        per step)."""
        rounds = args.rounds if rounds is None else rounds
        n = graph_len(K)
        sizes = [n] * (K // n) + ([K % n] if K % n else [])
        graphs = {}
        pos = 0
        plan = []
        for sz in sizes:
            key = (sz, pos % len(groups))
            if key not in graphs:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for i in range(sz):
                        call(groups[(pos + i) % len(groups)] if rotate else groups[0], phases)
                if cold:
                    scrub.add_(1.0)
                g.replay()  # first replay of a fresh graph, untimed
                graphs[key] = g
            plan.append(graphs[key])
            pos += sz
        torch.cuda.synchronize()
        samples = []
        for _ in range(rounds):
            # the scrub is still running while the host submits the graphs,
            # so the event pair times the K steps on the GPU, not the
            # host's submission of the first graph
            if cold:
                scrub.add_(1.0)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for g in plan:
                g.replay()
            b.record()
            torch.cuda.synchronize()
            samples.append(a.elapsed_time(b) * 1e3 / K)
        # host wall clock per step: the same K steps, synchronised on both sides
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for g in plan:
            g.replay()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / K
        return statistics.median(samples), samples, wall

    def launch_floor():
        """Per step, K steps of two trivial kernels (one-element adds) as
        graph replays: the floor of any two-launch layer step."""
        t = torch.zeros(1, dtype=torch.float32, device=dev)
        g = torch.cuda.CUDAGraph()
        n = min(K, 512)
        with torch.cuda.graph(g):
            for _ in range(n):
                t.add_(1.0)
                t.add_(1.0)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(max(1, K // n)):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (n * max(1, K // n))

    for i in range(W):
        call(groups[i % len(groups)])
    torch.cuda.synchronize()
    log("[bench] warm-up done")
    value, layer_rounds, wall_step = region()
    log(f"[bench] layer, cold: {value:.3f} us/step (median of {len(layer_rounds)} rounds: "
        f"{', '.join(f'{v:.3f}' for v in layer_rounds)})")
    floor_us = launch_floor()
    log(f"[bench] two trivial kernels per step: {floor_us:.3f} us/step")
    fc1_us, fc1_rounds, _ = region(phases=1)
    fc2_us, fc2_rounds, _ = region(phases=2)
    log(f"[bench] fc1 only {fc1_us:.3f} us/launch, fc2 only {fc2_us:.3f} us/launch")
    aux = {}
    if grouped:
        # the grouped halves also hold the routing (with FC1) and the combine
        # (with FC2): time those alone and take them out of the GEMM figures
        route_us, _, _ = region(phases=4)
        comb_us, _, _ = region(phases=8)
        aux = {"routing": round(route_us, 3), "combine": round(comb_us, 3),
               "fc1_half": round(fc1_us, 3), "fc2_half": round(fc2_us, 3)}
        fc1_us, fc2_us = fc1_us - route_us, fc2_us - comb_us
        log(f"[bench] routing {route_us:.3f} us, combine {comb_us:.3f} us; "
            f"fc1_gemm {fc1_us:.3f} us, fc2_gemm {fc2_us:.3f} us")

    csf = scales == "csf" and not grouped  # the grouped path reads the plain scales
    U, b13, b2 = routed_bytes(wl, groups[0][0].cpu().numpy(), d, csf)
    layer_bytes = b13 + b2
    from block_scaled_fp4_gather_amd import profsum
    if grouped:
        # algorithmic flops: 2 per multiply-add; FC1 is 2I x H and FC2 H x I per valid route
        flat = d["ids"].reshape(-1).astype(np.int64)
        routes = int(np.count_nonzero((flat >= 0) & (flat < wl.E)))
        f1, f2 = 2.0 * routes * 2 * wl.I * wl.H, 2.0 * routes * wl.H * wl.I
        sfx = "_a8" if a8 else ""
        dom, dom_work, dom_us = ("fc1_gemm" + sfx, f1, fc1_us) if f1 >= f2 else ("fc2_gemm" + sfx, f2, fc2_us)
        achieved = dom_work / (dom_us * 1e-6) / 1e12
        peak, unit, bound = (MFMA_FP8_PEAK_TFLOPS if a8 else MFMA_BF16_PEAK_TFLOPS), "TFLOP/s", "mfma"
    else:
        dom, dom_work, dom_us = ("fc1_kernel", b13, fc1_us) if b13 >= b2 else ("fc2_kernel", b2, fc2_us)
        achieved = dom_work / (dom_us * 1e-6) / 1e9
        peak, unit, bound = HBM_PEAK_GBPS, "GB/s", "hbm"
    prof = profsum.lookup(dom, wl.name) if args.shape is None and scales == wl.scales else None
    traffic = prof["hbm_bytes_per_dispatch"] if prof else None
    # `achieved` from the rocprofv3 mean duration of the kernel (the summary
    # of this same command in profiles/, while its HIP sources are
    # unchanged); the event-timed figure of this run is kept beside it
    scale = 1e12 if grouped else 1e9
    event_achieved = achieved
    if prof:
        achieved = dom_work / (prof["duration_us"]["mean_us"] * 1e-6) / scale
    extra = {}
    if args.extra:
        warm_us, _, _ = region(rotate=False)
        extra["warm_us_per_step"] = round(warm_us, 3)
        scrub = torch.zeros(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        ev = []
        for i in range(50):
            scrub.add_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            call(groups[0])
            e1.record()
            ev.append((e0, e1))
        torch.cuda.synchronize()
        extra["scrub_single_event_pair_us_median"] = round(statistics.median(a.elapsed_time(b) * 1e3 for a, b in ev), 3)
        dst = torch.empty_like(scrub)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        dst.copy_(scrub)
        c0.record()
        for _ in range(10):
            dst.copy_(scrub)
        c1.record()
        torch.cuda.synchronize()
        extra["copy_probe_GBps"] = round(2 * scrub.numel() * 4 * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9, 1)
        del scrub, dst

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        # whole layer calls; for many tokens, single tokens of the batch, scaled to M
        n, t_cpu, M_cpu = 0, 0.0, (1 if grouped else wl.M)
        while t_cpu < args.cpu_seconds and n < 1000:
            if grouped:
                t = int(sample[n % len(sample)])
                dd = dict(d, x=d["x"][t:t + 1], ids=d["ids"][t:t + 1], w=d["w"][t:t + 1])
            else:
                dd = d
            s0 = time.perf_counter()
            if a8:
                oracle.forward_w4a8(wl.fmt, dd)
            else:
                oracle.forward_f32(wl.fmt, dd)
            t_cpu += time.perf_counter() - s0
            n += 1
        per_call = t_cpu / n * wl.M / M_cpu
        what = (f"{n} single-token calls of {wl.name} (tokens of the batch), scaled by M={wl.M}" if grouped
                else f"{n} full layer calls of {wl.name} (M={wl.M})")
        cpu = {"value": round(per_call * 1e6, 1), "unit": "us", "cores": 1, "kind": "oracle",
               "sample": what + ", single-threaded C++ oracle"}
        log(f"[bench] cpu oracle {cpu['value']} us/layer over {n} calls")

    line = {
        "metric": ("us per MoE layer, grouped path, weights from HBM" if grouped else
                   "us per MoE layer @M=1 cold-L2 + % HBM peak on routed FP4 weight bytes"),
        "value": round(value, 3),
        "unit": "us",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(wall_step * 1e3, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("e2m1 weights x mxfp8 activations, f32 accumulate" if a8 else
                  "e2m1 weights x bf16 activations, f32 accumulate"),
        "data": "synthetic",
        "config": {"workload": wl.name, "format": wl.fmt, "E": wl.E, "H": wl.H, "I": wl.I,
                   "M": wl.M, "top_k": wl.k, "unique_experts": U, "activations": "mxfp8" if a8 else "bf16",
                   "scales": scales,
                   "path": "grouped" if plan.path == moe.PATH_GROUPED else "decode"},
        "hbm_frac_layer": round(layer_bytes / (value * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "routed_bytes": {"fc1": b13, "fc2": b2},
        "kernel_us": {"fc1": round(fc1_us, 3), "fc2": round(fc2_us, 3), **aux},
        "two_kernel_graph_floor_us": round(floor_us, 3),
        "roofline": {"bound": bound, "achieved": round(achieved, 1), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel": dom, ("algorithmic_flops" if grouped else "algorithmic_bytes"): dom_work,
                     "achieved_from": "rocprof_mean_us" if prof else "event_us",
                     "rocprof_mean_us": prof["duration_us"]["mean_us"] if prof else None,
                     "event_us": round(dom_us, 3), "event_achieved": round(event_achieved, 1),
                     "event_frac": round(event_achieved / peak, 4)},
        "rounds_us": {"layer": [round(v, 3) for v in layer_rounds], "fc1": [round(v, 3) for v in fc1_rounds],
                      "fc2": [round(v, 3) for v in fc2_rounds]},
        "cpu_baseline": cpu,
        "check": check,
        "env": run_env(torch),
    }
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
