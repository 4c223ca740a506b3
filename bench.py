#!/usr/bin/env python3
"""Benchmark of the Evoformer biased-attention forward pass on one MI355X.

One step = one evo_attn_fwd launch over the whole workload (every (b, n, h)
slice, every query), default: triangle attention around the starting node,
B=1, N=L=384, H=4, D=32, bf16, mask on the last 16 keys, pair bias projected
from a seeded pair tensor.  Throughput counts the dense work 4*B*N*H*L^2*D.

Timing: about a second of untimed launches (clock spin-up), W untimed
warm-up steps, then exactly K timed steps bracketed by
torch.cuda.synchronize(); inputs are resident in device memory before the
timed region.  In the default "cold" mode each step reads a different one of R
copies of the inputs (R chosen so the copies exceed the 256 MB Infinity
Cache), so every step streams its operands from HBM; "warm" reuses one copy.
A pair of HIP events on the launch stream brackets the K launches; their
elapsed time / K is the kernel time used for the roofline.  After the timed
region, 100 more launches, each between its own pair of events, give the
distribution of single-launch times (median, min, p90).  The fp64 CPU oracle
is timed on the host cores for the cpu_baseline field.  The line also names
the host CPU model, the GPU and the ROCm / HIP / PyTorch versions.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA, AMD public specification
# What a loop of independent v_mfma_f32_16x16x32_bf16 sustains on this part, two
# waves per SIMD on all 256 CUs (micro/micro.hip; profiles/micro_peaks_gfx950.md)
MEASURED_BF16_MFMA_TFLOPS = 1905.0
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
MALL_BYTES = 256 * 2 ** 20
METRIC = "biased-attention fwd TFLOP/s + % bf16 MFMA peak, triangle attn N=L=384"
KERNEL_SOURCES = {"bf16": "evoformer_biased_attention_amd/csrc/evo_attn_bf16.hip",
                  "f16": "evoformer_biased_attention_amd/csrc/evo_attn_bf16.hip",
                  "f32": "evoformer_biased_attention_amd/csrc/evo_attn_f32.hip"}


def metric_name(base, workload_name):
    """The headline metric names the triangle workload (N=L=384); other workloads name themselves."""
    return base if workload_name == "tri_start_bf16_384" else base.split(", triangle attn")[0] + ", " + workload_name


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def launch_stats(torch, launch, R, n=100):
    """Distribution of single-launch times: n launches, each bracketed by its own pair of HIP events on the
    launch stream (the marker packets add a little to each), inputs rotating over the R sets as in the timed
    region."""
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        launch(i % R)
        b.record(stream)
    torch.cuda.synchronize()
    t = sorted(1e3 * a.elapsed_time(b) for a, b in evs)
    pick = lambda q: t[min(n - 1, int(round(q * (n - 1))))]
    return {"n": n, "median_us": round(pick(0.5), 3), "min_us": round(t[0], 3), "p90_us": round(pick(0.9), 3),
            "max_us": round(t[-1], 3), "mean_us": round(sum(t) / n, 3)}


def environment(torch):
    """Host CPU model, GPU, and the versions of the tools behind the numbers."""
    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    cpu = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    rocm = None
    for path in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        if os.path.exists(path):
            with open(path) as f:
                rocm = f.read().strip()
            break
    props = torch.cuda.get_device_properties(0)
    return {"cpu_model": cpu, "host_threads": len(os.sched_getaffinity(0)), "gpu": props.name or None,
            "gcn_arch": getattr(props, "gcnArchName", None), "compute_units": props.multi_processor_count,
            "rocm": rocm, "hip_runtime": torch.version.hip, "torch": torch.__version__,
            "numpy": __import__("numpy").__version__, "python": sys.version.split()[0]}


def source_hash(dtype):
    with open(os.path.join(ROOT, KERNEL_SOURCES[dtype]), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def algorithmic_bytes(shape, dtype, has_mask, has_pair):
    """Q, K, V, O once, LSE once, the mask once per (b, n), the pair bias once per (b, h)."""
    B, N, L, H, D = shape
    es = 4 if dtype == "f32" else 2
    return 4 * B * N * L * H * D * es + 4 * B * N * H * L + (B * N * L * es if has_mask else 0) + (
        B * H * L * L * es if has_pair else 0)


def measured_counters(workload_name, dtype):
    """MFMA-busy fraction, vector issue slots per score element and engine clock from the committed
    rocprofv3 SQ counter summary, if it matches this kernel source."""
    path = os.path.join(ROOT, "profiles", f"sq_counters_{workload_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != source_hash(dtype):
        return None
    keys = ("mfma_busy_frac", "valu_slots_per_score", "mfma_per_wave_block", "valu_per_wave_block",
            "exp_per_wave_block", "engine_clock_ghz", "wait_frac_of_wave_time")
    return {k: t[k] for k in keys} | {"source": f"profiles/sq_counters_{workload_name}.json"}


def measured_traffic(workload_name, dtype):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it matches this kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != source_hash(dtype):
        return None
    return t.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=4, help="named workload 1..5 (default 4)")
    ap.add_argument("--dtype", choices=["bf16", "f16", "f32"], default=None,
                    help="store the workload's values in this format instead of its own")
    ap.add_argument("--mode", choices=["cold", "warm"], default="cold")
    ap.add_argument("--pass", dest="which", choices=["fwd", "bwd"], default="fwd",
                    help="fwd (default): the forward pass; bwd: one evo_attn_bwd call per step, every gradient")
    ap.add_argument("--no-workspace", action="store_true", help="bwd: run without the pair-gradient workspace")
    ap.add_argument("--op", choices=["attention", "trimul"], default="attention",
                    help="trimul: time evo_trimul on the named triangle-multiplication size instead")
    ap.add_argument("--direction", choices=["outgoing", "incoming"], default="outgoing", help="trimul orientation")
    ap.add_argument("--sweep", choices=["ds4sci"], default=None,
                    help="ds4sci: forward and backward over batch 1..16 at N=L=256, H=4, D=32, fp16 "
                         "(the DS4Sci guide's benchmark shape); prints one JSON line with every batch")
    ap.add_argument("--layout", choices=["dense", "transposed"], default="dense",
                    help="fwd: transposed stores Q/K/V/O as X[B, L, N, H, D] and reads them in place through "
                         "evo_attn_fwd_strided (triangle attention around the ending node without a copy)")
    ap.add_argument("--no-pair-bias", action="store_true",
                    help="drop the workload's pair bias (to price the pair-bias stream by difference)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="wall-time budget of the oracle leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-warm", action="store_true", help="skip the secondary warm-cache measurement")
    ap.add_argument("--spinup-seconds", type=float, default=1.0,
                    help="untimed launches for this long before the warm-up steps, so the timed steps run at "
                         "steady-state clocks (a fresh process starts them lower)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed steps, run one plain copy kernel (torch.neg, out=) over this many MiB, "
                         "a known-size reference for the HBM byte counters")
    ap.add_argument("--summarize-sq", nargs=2, metavar=("SQ_A_DIR", "SQ_B_DIR"),
                    help="read the two rocprofv3 SQ counter passes of this script (see sq_commands) and write "
                         "profiles/sq_counters_<workload>.json; runs on the host only")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="read two rocprofv3 --pmc runs of this script (FETCH_SIZE, WRITE_SIZE) and write "
                         "profiles/traffic_<workload>.json; runs on the host only")
    args = ap.parse_args()
    if args.summarize_sq:
        summarize_sq(args.workload, *args.summarize_sq)
        return
    if args.summarize_traffic:
        if args.copy_probe_mib <= 0:
            raise SystemExit("--summarize-traffic needs the --copy-probe-mib value the counter runs used")
        summarize_traffic(args.workload, args.copy_probe_mib, *args.summarize_traffic)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the forward pass shards over "
                                   "B*N with no exchange, so per-GPU work is the one-GPU figure; "
                                   f"--gpus {args.gpus} is not supported"}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import evoformer_biased_attention_amd as E
    import synthetic as S

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)

    if args.op == "trimul":
        return bench_trimul(args, torch, E, S)
    if args.sweep:
        return bench_sweep(args, torch, E, S)

    log(f"bench: generating workload {args.workload}")
    w = S.workload(args.workload, dtype=args.dtype)
    if args.no_pair_bias:
        w.pair = None
    B, N, L, H, D = w.shape
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.dtype]
    dcode = E.torch_dtype_code(tdt)

    def dev(x):
        if x is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(x))
        return (t if w.dtype == "f32" else t.view(tdt)).to("cuda")

    if args.which == "bwd":
        return bench_bwd(args, w, dev, torch, E, S)

    base = [dev(x) for x in (w.q, w.k, w.v, w.mask, w.pair)]
    if args.layout == "transposed":
        # X[B, L, N, H, D] in memory; the kernel sees its [B, N, L, H, D] view
        base[:3] = [t.permute(0, 2, 1, 3, 4).contiguous().permute(0, 2, 1, 3, 4) for t in base[:3]]
    set_bytes = sum(t.numel() * t.element_size() for t in base if t is not None) * 4 // 3 + B * N * H * L * 4
    R = 1 if args.mode == "warm" else max(2, math.ceil(2.5 * MALL_BYTES / set_bytes))
    sets = []
    for r in range(R):
        # clone keeps the strides (preserve_format), so every copy has the chosen layout
        ins = [t if (t is None or r == 0) else t.clone() for t in base]
        out = torch.empty_like(base[0])
        lse = torch.empty((B, N, H, L), dtype=torch.float32, device="cuda")
        sets.append((*ins, out, lse))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    layouts = [E.layout_of(s_[0], s_[1], s_[2], s_[5], s_[3], s_[4]) for s_ in sets]

    def launch(r):
        q, k, v, m, p, o, l = sets[r]
        if args.layout == "dense":
            return E.evo_attn_fwd(q, k, v, m, p, o, l, w.shape, dcode, sh)
        return E.evo_attn_fwd_strided(q, k, v, m, p, o, l, layouts[r], w.shape, dcode, sh)

    st = launch(0)
    if st != E.EVO_OK:
        raise E.EvoAttnError(st)
    log(f"bench: {R} input set(s) of {set_bytes / 2**20:.1f} MiB, warmup {args.warmup}, steps {args.steps}")
    t_spin = time.perf_counter()
    while time.perf_counter() - t_spin < args.spinup_seconds:
        for i in range(20):
            launch(i % R)
        torch.cuda.synchronize()
    for i in range(args.warmup):
        launch(i % R)
    torch.cuda.synchronize()

    # Timed region: K launches back to back on the launch stream, one pair of
    # HIP events around them (events between launches would add a marker
    # packet and a gap before every kernel).  kernel_us = region / K, so it
    # includes the short dispatch gaps between consecutive kernels.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        launch(i % R)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_us = 1e3 * ev0.elapsed_time(ev1) / args.steps
    flops = w.flops
    value = flops * args.steps / wall / 1e12
    achieved = flops / (kern_us * 1e-6) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype != "f32" else PEAK_F32_TFLOPS
    log(f"bench: {kern_us:.2f} us/launch (events), {wall / args.steps * 1e6:.2f} us/step (wall), "
        f"{achieved:.1f} TFLOP/s = {100 * achieved / peak:.1f}% of peak")

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * 2 ** 20 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    stats = launch_stats(torch, launch, R)
    log(f"bench: single launches median {stats['median_us']} us, min {stats['min_us']}, p90 {stats['p90_us']}")

    # secondary: the same launches reading one input set (operands may sit in the Infinity Cache)
    warm = None
    if R > 1 and not args.no_warm:
        nw = 50
        ev0.record(stream)
        for i in range(nw):
            launch(0)
        ev1.record(stream)
        torch.cuda.synchronize()
        wu = 1e3 * ev0.elapsed_time(ev1) / nw
        warm = {"kernel_us": round(wu, 3), "tflops": round(flops / (wu * 1e-6) / 1e12, 2)}

    alg_bytes = algorithmic_bytes(w.shape, w.dtype, w.mask is not None, w.pair is not None)
    traffic = measured_traffic(w.name, w.dtype)
    result = {
        "metric": metric_name(METRIC, w.name),
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; see synthetic/)",
        "config": {"workload": w.name, "variant": w.meta.get("variant"), "B": B, "N": N, "L": L, "H": H, "D": D,
                   "mask": w.mask is not None, "pair_bias": w.pair is not None, "mode": args.mode,
                   "input_sets": R, "flop_per_step": flops, "layout": args.layout},
        "pct_of_bf16_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic},
        "measured_mfma_peak": None if w.dtype == "f32" else {
            "tflops": MEASURED_BF16_MFMA_TFLOPS, "frac": round(achieved / MEASURED_BF16_MFMA_TFLOPS, 4),
            "source": "profiles/micro_peaks_gfx950.md"},
        "kernel_us": round(kern_us, 3),
        "launch_us": stats,
        "hbm": {"algorithmic_bytes": alg_bytes,
                "achieved_GBps": round(alg_bytes / (kern_us * 1e-6) / 1e9, 1),
                "frac_of_8TBps": round(alg_bytes / (kern_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
        "warm": warm,
        "counters": measured_counters(w.name, w.dtype),
        "env": environment(torch),
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, sets[0], args.cpu_seconds)
    print(json.dumps(result), flush=True)


TRIMUL_METRIC = "triangle multiplication TFLOP/s (x[c,i,j] = sum_k a[c,i,k] w[c,j,k]), bf16, L=384, C=128"


def bench_trimul(args, torch, E, S):
    """One step = one evo_trimul call over the named size (B=1, C=128, L=384).  Work 2*B*C*L^3; algorithmic
    bytes 3*B*C*L^2*2 (a and w read once, x written once), so the call is bound by HBM (128 FLOP/B, below
    the 315 FLOP/B ridge)."""
    import numpy as np
    c = dict(S.TRIMUL_WORKLOAD)
    if args.dtype:
        c["dtype"] = args.dtype
    B, C, L, dt = c["B"], c["C"], c["L"], c["dtype"]
    if dt not in ("bf16", "f16"):
        raise SystemExit("trimul runs in bf16 or f16")
    a, w = S.trimul_problem(B, C, L, dt, seed=384)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float16
    base = [torch.from_numpy(x).view(tdt).to("cuda") for x in (a, w)]
    set_bytes = 3 * B * C * L * L * 2
    R = 1 if args.mode == "warm" else max(2, math.ceil(2.5 * MALL_BYTES / set_bytes))
    sets = [([t if r == 0 else t.clone() for t in base], torch.empty_like(base[0])) for r in range(R)]
    code = E.torch_dtype_code(tdt)
    d = {"outgoing": E.EVO_TRIMUL_OUTGOING, "incoming": E.EVO_TRIMUL_INCOMING}[args.direction]
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def launch(r):
        (ta, tw), x = sets[r]
        return E.evo_trimul(ta, tw, x, (B, C, L), d, code, sh)

    st = launch(0)
    if st != E.EVO_OK:
        raise E.EvoAttnError(st)
    t_spin = time.perf_counter()
    while time.perf_counter() - t_spin < args.spinup_seconds:
        for i in range(20):
            launch(i % R)
        torch.cuda.synchronize()
    for i in range(args.warmup):
        launch(i % R)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        launch(i % R)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_us = 1e3 * ev0.elapsed_time(ev1) / args.steps
    stats = launch_stats(torch, launch, R)
    flops = 2 * B * C * L ** 3
    alg_bytes = set_bytes
    gbs = alg_bytes / (kern_us * 1e-6) / 1e9
    log(f"bench trimul: {kern_us:.2f} us/launch, {flops / (kern_us * 1e-6) / 1e12:.1f} TFLOP/s, {gbs:.0f} GB/s")
    result = {
        "metric": TRIMUL_METRIC.replace("sum_k a[c,i,k] w[c,j,k]", "sum_k a[c,i,k] w[c,j,k]" if d == 0
                                        else "sum_k a[c,k,i] w[c,k,j]"),
        "value": round(flops * args.steps / wall / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic (seeded; see synthetic/)",
        "config": {"workload": c["name"], "direction": args.direction, "B": B, "C": C, "L": L, "mode": args.mode,
                   "input_sets": R, "flop_per_step": flops},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None},
        "kernel_us": round(kern_us, 3),
        "mfma": {"tflops": round(flops / (kern_us * 1e-6) / 1e12, 2),
                 "frac_of_bf16_peak": round(flops / (kern_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4)},
        "launch_us": stats,
        "env": environment(torch),
    }
    if not args.no_cpu_baseline:
        import oracle
        threads = len(os.sched_getaffinity(0))
        ch, t = 0, 0.0
        while ch == 0 or (t < args.cpu_seconds and ch < C):
            t0 = time.perf_counter()
            ref = oracle.trimul(a[:, ch:ch + 1], w[:, ch:ch + 1], dt, args.direction, nthreads=threads)
            t += time.perf_counter() - t0
            ch += 1
        got = sets[0][1][:, :1].float().cpu().numpy()
        ref0 = oracle.trimul(a[:, :1], w[:, :1], dt, args.direction, nthreads=threads)
        result["cpu_baseline"] = {"value": round(2 * B * ch * L ** 3 / t / 1e12, 6), "unit": "TFLOP/s",
                                  "cores": threads, "kind": "oracle",
                                  "sample": f"{ch} of {C} channels of {c['name']} in fp64, {t:.1f} s",
                                  "parity_vs_gpu_channel0_max_err_over_max_ref":
                                      float(np.abs(got - ref0).max() / np.abs(ref0).max())}
    print(json.dumps(result), flush=True)


BWD_METRIC = "biased-attention bwd TFLOP/s (dq, dk, dv, mask and pair gradients), triangle attn N=L=384"


def bench_bwd(args, w, dev, torch, E, S):
    """One step = one evo_attn_bwd call: dq, dk, dv, the mask gradient and the
    pair gradient (a sum over N), from the forward pass's out and lse.
    Throughput counts the backward's dense work 10*B*N*H*L^2*D: the score
    recomputation Q.K^T, dP = dO.V^T, dV = P^T.dO, dQ = dS.K and dK = dS^T.Q."""
    B, N, L, H, D = w.shape
    dcode = {"f32": E.EVO_DTYPE_F32, "bf16": E.EVO_DTYPE_BF16, "f16": E.EVO_DTYPE_F16}[w.dtype]
    dout = S.random_dout(w.shape, w.dtype, seed=2026)
    base = [dev(x) for x in (w.q, w.k, w.v, w.mask, w.pair, dout)]
    out, lse = E.fwd(*base[:5])
    base += [out, lse]
    in_bytes = sum(t.numel() * t.element_size() for t in base if t is not None)
    set_bytes = 2 * in_bytes
    R = 1 if args.mode == "warm" else max(2, math.ceil(2.5 * MALL_BYTES / set_bytes))
    sets = []
    for r in range(R):
        ins = [t if (t is None or r == 0) else t.clone() for t in base]
        q, k, v, m, p, do, o, l = ins
        grads = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                 None if m is None else torch.empty_like(m), None if p is None else torch.empty_like(p),
                 torch.empty((B, N, H, L), dtype=torch.float32, device="cuda")]
        sets.append((ins, grads))
    # one workspace serves every step: the steps run one after another on one stream
    ws_bytes = E.evo_attn_bwd_workspace_size(w.shape, dcode) if not args.no_workspace else 0
    ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device="cuda") if ws_bytes else None
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def launch(r):
        (q, k, v, m, p, do, o, l), (dq, dk, dv, dm, dp, delta) = sets[r]
        return E.evo_attn_bwd(q, k, v, m, p, o, l, do, dq, dk, dv, dm, dp, delta, w.shape, dcode, sh,
                              workspace=ws, workspace_bytes=ws_bytes)

    st = launch(0)
    if st != E.EVO_OK:
        raise E.EvoAttnError(st)
    log(f"bench bwd: {R} input set(s) of {set_bytes / 2**20:.1f} MiB, warmup {args.warmup}, steps {args.steps}")
    t_spin = time.perf_counter()
    while time.perf_counter() - t_spin < args.spinup_seconds:
        for i in range(5):
            launch(i % R)
        torch.cuda.synchronize()
    for i in range(args.warmup):
        launch(i % R)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        launch(i % R)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pass_us = 1e3 * ev0.elapsed_time(ev1) / args.steps
    stats = launch_stats(torch, launch, R, n=60)
    flops = 10 * B * N * H * L * L * D
    value = flops * args.steps / wall / 1e12
    achieved = flops / (pass_us * 1e-6) / 1e12
    log(f"bench bwd: {pass_us:.2f} us/pass (events), {achieved:.2f} TFLOP/s")
    result = {
        "metric": metric_name(BWD_METRIC, w.name),
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; see synthetic/)",
        "config": {"workload": w.name, "variant": w.meta.get("variant"), "B": B, "N": N, "L": L, "H": H, "D": D,
                   "mask": w.mask is not None, "pair_bias": w.pair is not None, "mode": args.mode,
                   "input_sets": R, "flop_per_step": flops, "workspace_bytes": ws_bytes},
        # 16-bit inputs: every product on the matrix cores, priced against the dense bf16/f16 MFMA peak;
        # f32 inputs: the fp32 matrix-core kernels (every head dimension and bias stride of the dense and
        # transposed layouts), priced against the 157.3 TFLOP/s fp32 matrix peak
        "roofline": {"bound": "mfma",
                     "achieved": round(achieved, 3),
                     "peak": PEAK_BF16_TFLOPS if w.dtype != "f32" else PEAK_F32_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / (PEAK_BF16_TFLOPS if w.dtype != "f32" else PEAK_F32_TFLOPS), 4),
                     "traffic": None, "scope": "whole pass"},
        "measured_mfma_peak": None if w.dtype == "f32" else {
            "tflops": MEASURED_BF16_MFMA_TFLOPS, "frac": round(achieved / MEASURED_BF16_MFMA_TFLOPS, 4),
            "source": "profiles/micro_peaks_gfx950.md"},
        "pass_us": round(pass_us, 3),
        "launch_us": stats,
        "env": environment(torch),
    }
    if not args.no_cpu_baseline:
        import numpy as np
        import oracle
        threads = len(os.sched_getaffinity(0))
        passes, t = 0, 0.0
        while passes == 0 or (t < args.cpu_seconds and passes < 50):
            t0 = time.perf_counter()
            ref = oracle.bwd(w.q, w.k, w.v, w.mask, w.pair, dout, dtype=w.dtype, nthreads=threads)
            t += time.perf_counter() - t0
            passes += 1
        got = [None if g is None else g.float().cpu().numpy() for g in sets[0][1][:5]]
        err = {n: float(np.abs(g - r).max() / np.abs(r).max())
               for n, g, r in zip(("dq", "dk", "dv", "dmask", "dpair"), got, ref) if g is not None}
        result["cpu_baseline"] = {"value": round(flops * passes / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
                                  "kind": "oracle",
                                  "sample": f"{passes} full backward pass(es) over workload {w.name} in fp64, "
                                            f"{t:.1f} s",
                                  "parity_vs_gpu_max_err_over_max_ref": err}
    print(json.dumps(result), flush=True)


SWEEP_METRIC = "biased-attention fwd+bwd TFLOP/s over batch 1..16, N=L=256, H=4, D=32, fp16"


def _event_time_us(torch, launch, R, steps, warmup):
    """Average time per launch (HIP events around `steps` back-to-back launches), inputs rotating over R sets."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        launch(i % R)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(steps):
        launch(i % R)
    ev1.record(stream)
    torch.cuda.synchronize()
    return 1e3 * ev0.elapsed_time(ev1) / steps


def bench_sweep(args, torch, E, S):
    """The DS4Sci guide's benchmark shape (section 4 of its page): N=L=256,
    H=4, D=32, fp16, with a mask and a pair bias, batch 1 to 16.  Per batch:
    the forward (4*B*N*H*L^2*D flops) and the backward (10*B*N*H*L^2*D) each
    timed with HIP events over the launch stream, inputs rotated over enough
    copies to miss the Infinity Cache.  `value` is the fwd+bwd throughput at
    batch 16.  The guide prints no MI355X or absolute figure for this shape, so
    vs_baseline is null."""
    batches = [1, 2, 4, 8, 16]
    N, L, H, D, dt = 256, 256, 4, 32, "f16"
    log(f"sweep: generating B={batches[-1]} N={N} L={L} H={H} D={D} {dt}")
    w = S.random_problem(batches[-1], N, L, H, D, dtype=dt, seed=4781, mask="tail", pair="normal")
    dout = S.random_dout(w.shape, dt, seed=2026)
    dcode = E.EVO_DTYPE_F16

    def dev(x):
        return torch.from_numpy(x).view(torch.float16).to("cuda")

    full = [dev(x) for x in (w.q, w.k, w.v, w.mask, w.pair, dout)]
    stream_h = torch.cuda.current_stream().cuda_stream
    rows = []
    t_total = {"fwd": 0.0, "bwd": 0.0}
    for B in batches:
        shape = (B, N, L, H, D)
        base = [t[:B].contiguous() for t in full]
        in_bytes = sum(t.numel() * t.element_size() for t in base)
        R = max(2, math.ceil(2.5 * MALL_BYTES / (2 * in_bytes)))
        sets = []
        for r in range(R):
            q, k, v, m, p, do = base if r == 0 else [t.clone() for t in base]
            o, l = E.fwd(q, k, v, m, p)
            grads = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(m),
                     torch.empty_like(p), torch.empty((B, N, H, L), dtype=torch.float32, device="cuda")]
            sets.append(((q, k, v, m, p, do, o, l), grads))
        ws_bytes = E.evo_attn_bwd_workspace_size(shape, dcode)
        ws = torch.empty(max(ws_bytes, 4) // 4, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()

        def fwd(r):
            (q, k, v, m, p, _, o, l), _g = sets[r]
            return E.evo_attn_fwd(q, k, v, m, p, o, l, shape, dcode, stream_h)

        def bwd(r):
            (q, k, v, m, p, do, o, l), (dq, dk, dv, dm, dp, delta) = sets[r]
            return E.evo_attn_bwd(q, k, v, m, p, o, l, do, dq, dk, dv, dm, dp, delta, shape, dcode, stream_h,
                                  workspace=ws, workspace_bytes=ws_bytes)

        for f in (fwd, bwd):
            st = f(0)
            if st != E.EVO_OK:
                raise E.EvoAttnError(st)
        steps = max(10, args.steps // B)
        fu = _event_time_us(torch, fwd, R, steps, max(3, args.warmup // B))
        bu = _event_time_us(torch, bwd, R, steps, max(3, args.warmup // B))
        ff, bf = 4 * B * N * H * L * L * D, 10 * B * N * H * L * L * D
        rows.append({"B": B, "fwd_us": round(fu, 2), "fwd_tflops": round(ff / fu / 1e6, 2),
                     "bwd_us": round(bu, 2), "bwd_tflops": round(bf / bu / 1e6, 2),
                     "fwd_bwd_tflops": round((ff + bf) / (fu + bu) / 1e6, 2), "input_sets": R})
        log(f"sweep: B={B} fwd {fu:.1f} us ({rows[-1]['fwd_tflops']} TFLOP/s), "
            f"bwd {bu:.1f} us ({rows[-1]['bwd_tflops']} TFLOP/s)")
        t_total["fwd"], t_total["bwd"] = fu, bu
        del sets, ws
        torch.cuda.empty_cache()
    last = rows[-1]
    result = {
        "metric": SWEEP_METRIC,
        "value": last["fwd_bwd_tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round((t_total["fwd"] + t_total["bwd"]) / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic (seeded; see synthetic/)",
        "config": {"workload": "ds4sci_benchmark_256x256_h4_d32_f16", "N": N, "L": L, "H": H, "D": D,
                   "batches": batches, "mask": True, "pair_bias": True, "mode": "cold"},
        "roofline": {"bound": "mfma", "achieved": last["fwd_bwd_tflops"], "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(last["fwd_bwd_tflops"] / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "scope": "forward + backward at batch 16"},
        "sweep": rows,
    }
    print(json.dumps(result), flush=True)


def _counter_means(directory, counter, name_part):
    """Mean per-dispatch value of one counter over the kernels whose name contains name_part."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]:
                    key = (f, r.get("Dispatch_Id", r.get("Correlation_Id")))
                    vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} rows for kernels matching {name_part!r} under {directory}")
    return sum(vals.values()) / len(vals), len(vals)


def traffic_commands(fetch_dir, write_dir, probe_mib):
    """The three commands behind a traffic summary: one counter run per counter (each writes its CSV under
    the given directory), then this summary."""
    run = (f"-o tri -- python3 bench.py --steps 5 --warmup 1 --no-cpu-baseline --no-warm --spinup-seconds 0 "
           f"--copy-probe-mib {probe_mib}")
    return [f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} {run}",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} {run}",
            f"python3 bench.py --summarize-traffic {fetch_dir} {write_dir} --copy-probe-mib {probe_mib}"]


def summarize_traffic(workload, probe_mib, fetch_dir, write_dir):
    """HBM traffic per launch of the attention kernel from FETCH_SIZE / WRITE_SIZE (KiB per dispatch).

    Each counter is scaled by the factor that maps what it reads for the copy
    probe (torch.neg over --copy-probe-mib MiB, reading and writing exactly
    that many bytes) onto the probe's true byte count.
    """
    import synthetic as S
    w = S.workload(workload)
    kname = {"bf16": "Bf16Fmt", "f16": "F16Fmt", "f32": "fwd_f32"}[w.dtype]  # in the kernel's demangled name
    probe_name = "neg_kernel"
    fk, nfk = _counter_means(fetch_dir, "FETCH_SIZE", kname)
    wk, nwk = _counter_means(write_dir, "WRITE_SIZE", kname)
    fp, _ = _counter_means(fetch_dir, "FETCH_SIZE", probe_name)
    wp, _ = _counter_means(write_dir, "WRITE_SIZE", probe_name)
    probe_bytes = probe_mib * 2 ** 20
    f_scale = probe_bytes / (fp * 1024)
    w_scale = probe_bytes / (wp * 1024)
    fetch_b = fk * 1024 * f_scale
    write_b = wk * 1024 * w_scale
    B, N, L, H, D = w.shape
    out = {
        "workload": w.name,
        "commands": traffic_commands(fetch_dir, write_dir, probe_mib),
        "note": "FETCH_SIZE's formula counts a 128-byte read request as 64 bytes on this device; the copy "
                "probe (all 128-byte requests) reads back half its size, hence fetch_scale ~2",
        "kernel_name_contains": kname,
        "kernel_source_sha256": source_hash(w.dtype),
        "dispatches": {"fetch": nfk, "write": nwk},
        "fetch_kib_per_dispatch": round(fk, 1),
        "write_kib_per_dispatch": round(wk, 1),
        "copy_probe": {"bytes_read": probe_bytes, "bytes_written": probe_bytes,
                       "fetch_kib": round(fp, 1), "write_kib": round(wp, 1),
                       "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
        "hbm_fetch_bytes_per_launch": int(fetch_b),
        "hbm_write_bytes_per_launch": int(write_b),
        "hbm_bytes_per_launch": int(fetch_b + write_b),
        "algorithmic_bytes": algorithmic_bytes(w.shape, w.dtype, w.mask is not None, w.pair is not None),
    }
    path = os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


SQ_A = ["SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_ANY",
        "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"]
SQ_B = ["SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_VALU_TRANS_F32", "SQ_WAVES",
        "SQ_INSTS_SALU", "SQ_WAIT_INST_LDS"]


def sq_commands(dir_a, dir_b):
    """The three commands behind an SQ counter summary (one counter pass each, then the summary)."""
    run = "-o tri -- python3 bench.py --steps 5 --warmup 1 --no-cpu-baseline --no-warm --spinup-seconds 0"
    return [f"rocprofv3 --pmc {' '.join(SQ_A)} --output-format csv -d {dir_a} {run}",
            f"rocprofv3 --pmc {' '.join(SQ_B)} --output-format csv -d {dir_b} {run}",
            f"python3 bench.py --summarize-sq {dir_a} {dir_b}"]


def summarize_sq(workload, dir_a, dir_b):
    """MFMA-busy fraction, vector issue slots per score element and the engine clock of the attention
    kernel, from two rocprofv3 SQ counter passes (means per dispatch; the clock from GRBM_GUI_ACTIVE per
    XCD over the dispatches' own durations in the counter CSV)."""
    import csv
    import glob
    import synthetic as S
    w = S.workload(workload)
    kname = {"bf16": "Bf16Fmt", "f16": "F16Fmt", "f32": "fwd_f32"}[w.dtype]
    c = {n: _counter_means(dir_a, n, kname)[0] for n in SQ_A}
    c.update({n: _counter_means(dir_b, n, kname)[0] for n in SQ_B})
    durations = {}
    for f in glob.glob(os.path.join(dir_a, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if kname in r["Kernel_Name"]:
                    durations[(f, r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    dur_ns = sum(durations.values()) / len(durations)
    xcds, simds = 8, 1024
    grbm_per_xcd = c["GRBM_GUI_ACTIVE"] / xcds
    B, N, L, H, D = w.shape
    waves = c["SQ_WAVES"]
    blocks_per_wave = -(-L // 64)  # 64-key blocks each wave visits
    scores_per_wave_block = 32 * 64  # 32 queries x 64 keys
    per_block = lambda x: x / waves / blocks_per_wave
    valu_other = c["SQ_INSTS_VALU"] - c["SQ_INSTS_MFMA"]  # vector instructions, exponentials included
    out = {
        "workload": w.name,
        "commands": sq_commands(dir_a, dir_b),
        "kernel_name_contains": kname,
        "kernel_source_sha256": source_hash(w.dtype),
        "dispatches": len(durations),
        "dispatch_ns_under_counters": round(dur_ns, 1),
        "counters_per_dispatch": {k: round(v, 1) for k, v in c.items()},
        "engine_clock_ghz": round(grbm_per_xcd / dur_ns, 3),
        "mfma_busy_frac": round(c["SQ_VALU_MFMA_BUSY_CYCLES"] / (grbm_per_xcd * simds), 4),
        "mfma_per_wave_block": round(per_block(c["SQ_INSTS_MFMA"]), 2),
        "valu_per_wave_block": round(per_block(valu_other), 2),
        "exp_per_wave_block": round(per_block(c["SQ_INSTS_VALU_TRANS_F32"]), 2),
        # issue slots of the vector port per score element: each wave64 instruction covers 64 lanes, and a
        # wave-block holds 32 x 64 score elements, i.e. 32 per lane
        "valu_slots_per_score": round(per_block(valu_other) / (scores_per_wave_block / 64), 3),
        "wait_frac_of_wave_time": round(c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"], 4),
        "note": "per wave-block: one wave's 32 queries against one 64-key block; the vector counts include the "
                "exponentials and exclude the MFMAs",
    }
    path = os.path.join(ROOT, "profiles", f"sq_counters_{w.name}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def cpu_baseline(w, gpu_set, budget_s):
    """The fp64 oracle (oracle/evo_ref.c, OpenMP over slices) on the host cores.

    Runs whole passes over the same workload until the wall-time budget is
    used (at least one pass), and compares its result with the GPU output of
    the first input set.
    """
    import numpy as np

    import oracle
    threads = len(os.sched_getaffinity(0))
    log(f"bench: oracle on {threads} host threads")
    passes, t = 0, 0.0
    ref = None
    while passes == 0 or (t < budget_s and passes < 200):
        t0 = time.perf_counter()
        ref = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype=w.dtype, nthreads=threads)
        t += time.perf_counter() - t0
        passes += 1
    out, lse = gpu_set[5], gpu_set[6]
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    do = np.abs(o - ref[0])
    dl = np.abs(l - ref[1])
    return {"value": round(w.flops * passes / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{passes} full pass(es) over workload {w.name} in fp64, {t:.1f} s",
            "parity_vs_gpu": {"max_abs_o": float(do.max()), "mean_abs_o": float(do.mean()),
                              "max_abs_lse": float(dl.max())}}


if __name__ == "__main__":
    main()
