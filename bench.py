"""Benchmark: fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long_yat]
                    [--no-cpu-baseline] [--backward]

A step is one Yat forward (|k|^2 pre-pass + fused kernel, i.e. every step of
the hot path) over the resident synthetic batch B=4, H=16, T=4096, d=128,
bf16, causal.  The softmax branch of the same kernel skeleton is timed on the
same inputs for the side-by-side figure.  Prints one JSON line.

Algorithmic work per allowed (query, key) pair: 2*d_k + 2*d_v MFMA flops
(elementwise maps and reductions not counted); causal pairs per head
T(T+1)/2.  Durations are HIP events recorded on the stream the kernels run on.

--backward times attn_bwd instead (the gradients of the same forward, with
the forward's row statistics and dL/dout resident): five products per pair,
2*(3 d_k + 2 d_v) flops (S, dP, dV, dK, dQ; the kernels' recomputation of S
and dP is not counted).  Its line carries its own metric name.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s and % bf16 MFMA peak (Yat vs softmax), B4 h16 T4096 d128"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published


def alg_flops(wl) -> float:
    return float(wl.allowed_pairs) * 2.0 * (wl.dk + wl.dv)


def uses_decode_kernel(wl, args) -> bool:
    """The library's plan: the decode kernel runs when a key/value head has
    at most 8 query rows and no launch option overrides it, or when
    block_rows = 8 forces it."""
    packed = wl.Hq // wl.Hkv * wl.Tq
    return args.block_rows == 8 or (args.block_rows == 0 and args.kv_splits == 0 and packed <= 8)


def kernels_timed(wl, args, variant) -> str:
    """The kernels one timed forward call runs: the decode kernel and its
    merge, or the fused tile kernel after the |k|^2 pre-pass for Yat (at
    d_k <= 32 the small-grid tile kernels form |k|^2 themselves)."""
    if uses_decode_kernel(wl, args):
        return f"attn_decode_bf16 ({variant}) + combine_partials"
    if variant != "yat":
        return f"attn_fwd_bf16 ({variant})"
    if wl.dk <= 32:
        return "attn_fwd_bf16 (yat; |k|^2 in-kernel in the small-grid kernels, else a pre-pass)"
    return "|k|^2 pre-pass + attn_fwd_bf16 (yat)"


def alg_bytes(wl) -> float:
    e = 2 if wl.dtype == "bf16" else 4
    q = wl.B * wl.Hq * wl.Tq * wl.dk * e
    kv = wl.B * wl.Hkv * wl.Tk * (wl.dk + wl.dv) * e
    o = wl.B * wl.Hq * wl.Tq * wl.dv * e
    stats = 2 * wl.B * wl.Hq * wl.Tq * 4
    return float(q + kv + o + stats)


# sources the fused forward kernel is compiled from
# sources of the dominant kernel: the fused tile kernels, or the decode kernel
KERNEL_SOURCES = {
    False: ("attn_bf16.hip", "bf16_common.h", "attn_launch.h"),
    True: ("attn_decode.hip", "bf16_common.h", "attn_launch.h"),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash(decode: bool = False) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[decode]:
        with open(os.path.join(ROOT, "softmax_free_score_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, variant: str, decode: bool = False):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by the same counter on a
    plain copy of known size), or None when there is none for this workload and
    variant or the kernel source changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    r = rec.get(f"{workload}/{variant}")
    if not r or r.get("kernel_source_sha256_16") != kernel_source_hash(decode):
        return None
    return r.get("bytes_per_launch")


def bwd_flops(wl) -> float:
    return float(wl.allowed_pairs) * 2.0 * (3 * wl.dk + 2 * wl.dv)


def settle(fn, ms):
    """Run `fn` untimed for about `ms` milliseconds of wall time and wait for
    it: the GPU leaves the idle power state it sat in while the inputs were
    generated on the host, so the warm-up and timed calls that follow run at
    the engine clock this load holds (a handful of warm-up calls, a few
    milliseconds, is shorter than that ramp)."""
    import torch
    if ms <= 0:
        return 0
    n, t0 = 0, time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            fn()
        n += 8
        torch.cuda.synchronize()
    return n


def time_calls(fn, stream, steps, warmup, per_call=None, settle_ms=0):
    """Average per-call duration (ms) by HIP events on `stream`, plus the
    wall time of the whole timed region.  `per_call`, a list, receives every
    call's duration.  `settle_ms`: untimed calls before the warm-up (settle)."""
    import torch
    settle(fn, settle_ms)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    if per_call is not None:
        per_call.extend(per)
    return float(np.mean(per)), float(np.median(per)), wall


def spread(per):
    """Spread of the per-call durations of the timed region (ms)."""
    a = np.asarray(per, dtype=np.float64)
    return {"min_ms": round(float(a.min()), 4), "p10_ms": round(float(np.percentile(a, 10)), 4),
            "median_ms": round(float(np.median(a)), 4),
            "p90_ms": round(float(np.percentile(a, 90)), 4), "max_ms": round(float(a.max()), 4),
            "cv": round(float(a.std() / a.mean()), 4)}


def engine_clock(fn, warm=1.0, readings_n=3, gap=0.25):
    """The GFX engine clock under this load: the timed call is enqueued in a
    loop by a second thread (after the timed region); after `warm` seconds of
    it, `amd-smi metric --clock` is read `readings_n` times, `gap` apart.
    Returns the mean clock over the XCDs of each reading (MHz) and their
    median, or None where amd-smi is missing or its output does not parse."""
    import re
    import shutil
    import subprocess
    import threading
    import torch
    exe = shutil.which("amd-smi")
    if not exe:
        return None
    stop = threading.Event()

    def load():
        while not stop.is_set():
            fn()

    th = threading.Thread(target=load, daemon=True)
    th.start()
    readings = []
    try:
        time.sleep(warm)
        for _ in range(readings_n):
            try:
                out = subprocess.run([exe, "metric", "-g", "0", "--clock"], capture_output=True,
                                     text=True, timeout=20).stdout
            except (OSError, subprocess.SubprocessError):
                continue
            clk = [int(m) for m in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*(\d+)\s*MHz", out)]
            if clk:
                readings.append(round(float(np.mean(clk)), 1))
            time.sleep(gap)
    finally:
        stop.set()
        th.join()
        torch.cuda.synchronize()
    if not readings:
        return None
    return {"gfx_mhz_mean_over_xcds": readings, "median_mhz": float(np.median(readings)),
            "source": f"amd-smi metric --clock, read {len(readings)} times while the timed "
                      f"call ran in a loop (after {warm:.1f} s of it, following the timed region)"}


def cpu_baseline(inp, variant, target_s=25.0):
    """The fp64 C oracle on a strided sample of the query rows, timed on the
    host cores; scaled to TFLOP/s with the same algorithmic count."""
    import oracle
    wl = inp.wl
    q, k, v = inp.f64()
    prm = {n: a.astype(np.float64) for n, a in inp.params().items()}
    n_rows = wl.B * wl.Hq * wl.Tq

    def pairs_of(rows):
        i = rows % wl.Tq
        return float(np.sum(i + 1)) if wl.causal else float(len(rows) * wl.Tk)

    # calibrate on a small sample, then size the timed sample to ~target_s
    # (4096 rows: enough per thread that the causal row-length spread averages out)
    probe = np.arange(0, n_rows, max(1, n_rows // 4096), dtype=np.int64)
    t0 = time.perf_counter()
    oracle.attn_fwd_c(q, k, v, variant, causal=wl.causal, rows=probe, **prm)
    t_probe = max(time.perf_counter() - t0, 1e-3)
    stride = max(1, int(np.ceil(n_rows * t_probe / len(probe) / target_s)))
    rows = np.arange(stride // 2, n_rows, stride, dtype=np.int64)
    t0 = time.perf_counter()
    oracle.attn_fwd_c(q, k, v, variant, causal=wl.causal, rows=rows, **prm)
    dt = time.perf_counter() - t0
    flops = pairs_of(rows) * 2.0 * (wl.dk + wl.dv)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{variant}, "
                      + ("every query row" if stride == 1 else f"1 query row in {stride}")
                      + f" of {wl.name} ({len(rows)} rows, "
                      f"{pairs_of(rows):.3e} allowed pairs) in {dt:.1f} s, fp64 C loops, OpenMP"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long_yat")
    ap.add_argument("--variant", default="yat")
    ap.add_argument("--settle-ms", type=int, default=300,
                    help="before each branch's warm-up, run its call untimed for this many "
                         "milliseconds so that the engine clock has left the idle state")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the engine-clock reading after the timed region")
    ap.add_argument("--rotate-mib", type=int, default=0,
                    help="cycle over enough distinct copies of the inputs and outputs to "
                         "span this many MiB (larger than the 256 MB Infinity Cache, so "
                         "small workloads are measured from HBM)")
    ap.add_argument("--block-rows", type=int, default=0, choices=(0, 8, 64, 128, 256),
                    help="query rows per workgroup of the bf16 kernel (0: the library's "
                         "choice from the grid size)")
    ap.add_argument("--kv-splits", type=int, default=0,
                    help="key chunks per workgroup of the small-grid kernels (0: the library's "
                         "choice, 1: none)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward (attn_bwd) of the workload instead of the forward")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (the "
                         "reference that scales the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the attention "
              "forward shards over (batch, kv-head) with no exchange step; only the one-GPU "
              "kernel is built)", file=sys.stderr)
        sys.exit(2)

    import torch
    from softmax_free_score_amd import attn
    from softmax_free_score_amd.workloads import WORKLOADS, make_inputs

    wl = WORKLOADS[args.workload]
    inp = make_inputs(wl)
    if args.backward:
        return bench_backward(args, wl, inp)
    dev = torch.device("cuda:0")
    if wl.dtype == "bf16":
        t = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
        q, k, v = t(inp.q_bits), t(inp.k_bits), t(inp.v_bits)
    else:
        q, k, v = (torch.from_numpy(a).to(dev) for a in (inp.q, inp.k, inp.v))
    prm = {n: torch.from_numpy(a).to(dev) for n, a in inp.params().items()}
    out = torch.empty((wl.B, wl.Hq, wl.Tq, wl.dv), dtype=q.dtype, device=dev)
    mass = torch.empty((wl.B, wl.Hq, wl.Tq), dtype=torch.float32, device=dev)
    mx = torch.empty_like(mass)
    sets = [(q, k, v, out, mass, mx)]
    if args.rotate_mib:
        n_sets = max(1, -(-(args.rotate_mib << 20) // int(alg_bytes(wl))))
        sets += [tuple(t.clone() for t in sets[0]) for _ in range(n_sets - 1)]
    stream = torch.cuda.current_stream(dev)
    ws = {}
    for var in ("yat", "softmax", "stau"):
        n = attn.workspace_bytes(q, k, v, var, args.block_rows, args.kv_splits)
        ws[var] = torch.empty(n, dtype=torch.uint8, device=dev) if n else None

    def call(var):
        it = [0]

        def run():
            q_, k_, v_, o_, m_, x_ = sets[it[0] % len(sets)]
            it[0] += 1
            attn.attn_fwd(q_, k_, v_, var, causal=wl.causal, out=o_, mass=m_, max_score=x_,
                          workspace=ws[var], stream=stream.cuda_stream,
                          block_rows=args.block_rows, kv_splits=args.kv_splits, **prm)
        return run

    flops = alg_flops(wl)
    primary = args.variant
    torch.cuda.synchronize()
    per_call = []
    mean_ms, med_ms, wall = time_calls(call(primary), stream, args.steps, args.warmup, per_call,
                                       settle_ms=args.settle_ms)
    others = {}
    for var in wl.variants:
        if var != primary:
            m2, md2, _ = time_calls(call(var), stream, args.steps, args.warmup,
                                    settle_ms=args.settle_ms)
            others[var] = {"ms": m2, "tflops": flops / (m2 * 1e-3) / 1e12,
                           "frac_bf16_peak": flops / (m2 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    value = flops / (mean_ms * 1e-3) / 1e12
    ai = flops / alg_bytes(wl)
    hbm_bound = ai < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if hbm_bound:   # below the ridge point: the HBM roofline bounds the kernel
        gbs = alg_bytes(wl) / (mean_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(value, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(value / PEAK_BF16_TFLOPS, 4)}
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(mean_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: B{wl.B} Hq{wl.Hq} Hkv{wl.Hkv} Tq{wl.Tq} Tk{wl.Tk} "
                               f"dk{wl.dk} dv{wl.dv} {wl.dtype} "
                               f"{'causal' if wl.causal else 'non-causal'}",
                   "variant": primary, "global_batch": wl.B, "seq_len": wl.Tq,
                   "input_sets_rotated": len(sets), "block_rows": args.block_rows,
                   "kv_splits": args.kv_splits,
                   "parallelism": "none (1 GPU)"},
        "roofline": {**roof,
                     "scope": "step: the whole call, every kernel it launches, event-timed "
                              "(kernel-level figures from the trace are in profiles/)",
                     "traffic": recorded_traffic(wl.name, primary, uses_decode_kernel(wl, args)),
                     "traffic_unit": "bytes per launch of "
                                     f"{'attn_decode_bf16' if uses_decode_kernel(wl, args) else 'attn_fwd_bf16'}"
                                     " (HBM, counters)",
                     "kernel": f"{kernels_timed(wl, args, primary)}; flops = "
                               f"{flops:.4e} per launch ({wl.allowed_pairs} allowed pairs x "
                               f"2(dk+dv))",
                     "median_ms": round(med_ms, 4),
                     "arithmetic_intensity_flop_per_byte": round(ai, 1)},
        "alg_bytes_gbs": round(alg_bytes(wl) / (mean_ms * 1e-3) / 1e9, 1),
        "wall_s_timed_region": round(wall, 3),
        "settle_ms_per_branch": args.settle_ms,
        "spread": spread(per_call),
    }
    for var, r in others.items():
        line[var] = {k2: round(v2, 4) for k2, v2 in r.items()}
    if "softmax" in others:
        # > 1 means the primary branch is faster than softmax on the same inputs
        line[f"{primary}_speed_vs_softmax"] = round(others["softmax"]["ms"] / mean_ms, 4)
    if not args.no_clock:
        line["engine_clock"] = engine_clock(call(primary))
    line["roofline"]["alg_bytes_per_launch"] = alg_bytes(wl)
    line["kernel_source_sha256_16"] = kernel_source_hash(uses_decode_kernel(wl, args))
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = n
        del src, dst
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp, primary)
    print(json.dumps(line), flush=True)


def cpu_baseline_bwd(inp, variant, target_s=10.0):
    """The fp64 numpy oracle backward over whole (batch, kv head) groups, in
    order, until about target_s seconds have passed (its own five-product flop
    count over the pairs it covered)."""
    import oracle
    from softmax_free_score_amd.workloads import make_grad_out
    wl = inp.wl
    g = wl.Hq // wl.Hkv
    q, k, v = inp.f64()
    dout = make_grad_out(inp)[0].astype(np.float64)
    groups, dt = 0, 0.0
    while dt < target_s and groups < wl.B * wl.Hkv:
        b, hk = divmod(groups, wl.Hkv)
        hs = slice(hk * g, (hk + 1) * g)
        prm = {n: a[hs].astype(np.float64) for n, a in inp.params().items()}
        t0 = time.perf_counter()
        oracle.attn_bwd_np(q[b:b + 1, hs], k[b:b + 1, hk:hk + 1], v[b:b + 1, hk:hk + 1],
                           dout[b:b + 1, hs], variant, causal=wl.causal, **prm)
        dt += time.perf_counter() - t0
        groups += 1
    pairs = groups * g * (wl.Tq * (wl.Tq + 1) // 2 if wl.causal else wl.Tq * wl.Tk)
    flops = pairs * 2.0 * (3 * wl.dk + 2 * wl.dv)
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except ImportError:
        cores = os.cpu_count()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{variant}, {groups} of {wl.B * wl.Hkv} (batch, kv head) groups "
                      f"({groups * g} query heads, {pairs} pairs) of {wl.name} in {dt:.1f} s, "
                      f"fp64 numpy (BLAS threads for the products)"}


def bench_backward(args, wl, inp):
    import torch
    from softmax_free_score_amd import attn
    from softmax_free_score_amd.workloads import make_grad_out

    dev = torch.device("cuda:0")
    t = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    if wl.dtype != "bf16":
        print("the backward is built for bf16 storage", file=sys.stderr)
        sys.exit(2)
    q, k, v = t(inp.q_bits), t(inp.k_bits), t(inp.v_bits)
    dout = t(make_grad_out(inp)[1])
    prm = {n: torch.from_numpy(a).to(dev) for n, a in inp.params().items()}
    stream = torch.cuda.current_stream(dev)
    grads = {n: torch.empty_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v))}

    def call(var):
        _, mass, mx = attn.attn_fwd(q, k, v, var, causal=wl.causal, **prm)
        n = attn.bwd_workspace_bytes(q, k, v, var)
        ws = torch.empty(n, dtype=torch.uint8, device=dev) if n else None

        def run():
            attn.attn_bwd(q, k, v, dout, var, mass, mx, causal=wl.causal, workspace=ws,
                          stream=stream.cuda_stream, **grads, **prm)
        return run

    flops = bwd_flops(wl)
    primary = args.variant
    torch.cuda.synchronize()
    per_call = []
    mean_ms, med_ms, wall = time_calls(call(primary), stream, args.steps, args.warmup, per_call,
                                       settle_ms=args.settle_ms)
    others = {}
    for var in wl.variants:
        if var != primary:
            m2, _, _ = time_calls(call(var), stream, args.steps, args.warmup,
                                    settle_ms=args.settle_ms)
            others[var] = {"ms": m2, "tflops": flops / (m2 * 1e-3) / 1e12,
                           "frac_bf16_peak": flops / (m2 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    value = flops / (mean_ms * 1e-3) / 1e12
    line = {
        "metric": "attn bwd TFLOP/s (5-product count) and % bf16 MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(mean_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: B{wl.B} Hq{wl.Hq} Hkv{wl.Hkv} Tq{wl.Tq} Tk{wl.Tk} "
                               f"dk{wl.dk} dv{wl.dv} {wl.dtype} "
                               f"{'causal' if wl.causal else 'non-causal'}, backward",
                   "variant": primary, "global_batch": wl.B, "seq_len": wl.Tq,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(value, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(value / PEAK_BF16_TFLOPS, 4),
                     "traffic": None,
                     "kernel": f"attn_bwd ({primary}): row prep, D pass, dK/dV and dQ kernels; "
                               f"flops = {flops:.4e} per call ({wl.allowed_pairs} allowed "
                               f"pairs x 2(3 dk + 2 dv))",
                     "median_ms": round(med_ms, 4),
                     "scope": "step: the whole attn_bwd call, every kernel it launches"},
        "wall_s_timed_region": round(wall, 3),
        "settle_ms_per_branch": args.settle_ms,
        "spread": spread(per_call),
    }
    for var, r in others.items():
        line[var] = {k2: round(v2, 4) for k2, v2 in r.items()}
    if "softmax" in others:
        line[f"{primary}_speed_vs_softmax"] = round(others["softmax"]["ms"] / mean_ms, 4)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_bwd(inp, primary)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
