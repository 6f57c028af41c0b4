#!/usr/bin/env python3
"""Benchmark of the LittleBit factorised-linear forward on one MI355X.

Default workload: the Llama-2-70B-shaped stack at 0.1 sign bits per weight
(80 layers x {q, k, v, o, gate, up, down}, both paths, 560 linears, 0.91 GB
of packed signs + fp16 scales), decode at batch 1, run as one lb_stack_forward
per step (HIP graph replay of the three decode kernels, V stage, mid stage
and U stage, each over every linear of the stack).  Inputs are seeded synthetic data
resident in HBM before timing starts.

Prints one JSON line: the decode step's microseconds per token and achieved
HBM GB/s (algorithmic bytes), the roofline of the dominant kernel, the
prefill stack's effective TFLOP/s (Llama-2-13B shape, 2048 tokens) when the
prefill kernels are available, and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time
from fractions import Fraction

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6       # MI355X dense bf16 MFMA
METRIC = "decode µs/token + HBM GB/s on layer stack; prefill TFLOP/s vs MFMA peak"

WORKLOADS = {
    # name: (synth workload, tokens, regime)
    "cfg5-decode": ("llama2-70b-0.1bpw", 1, "decode"),
    "cfg5-decode8": ("llama2-70b-0.1bpw", 8, "decode"),
    "cfg5-decode64": ("llama2-70b-0.1bpw", 64, "decode"),
    "cfg2-decode": ("llama2-7b-0.1bpw", 1, "decode"),
    "cfg4-decode": ("llama3-8b-0.3bpw", 16, "decode"),
    "cfg3-prefill": ("llama2-13b-0.55bpw", 2048, "prefill"),
    "cfg4-prefill": ("llama3-8b-0.3bpw", 2048, "prefill"),
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def ranks_for(wl, spec, lb):
    if wl.bpw is None:
        return [wl.fixed_rank, wl.fixed_rank]
    r = lb.rank_for_bpw(spec.m, spec.n, wl.bpw.numerator, wl.bpw.denominator) * spec.rank_mult
    return [r, r]


def algorithmic(wl, ranks_of, T):
    """Bytes and flops the method itself must move / compute per step (both paths)."""
    byts = flops = 0
    for _, j, s in wl.entries():
        for r in ranks_of[j]:
            byts += (s.m + s.n) * r / 8 + 2 * (s.m + s.n + r)
            flops += 2 * T * (s.m + s.n) * r
        byts += T * (s.n + s.m) * 2
    return byts, flops


def build_stack(wl, T, lb, torch, limit_layers=None):
    import synth
    ranks_of = [ranks_for(wl, s, lb) for s in wl.mats]
    lins, xs, ys = [], [], []
    layers = wl.layers if limit_layers is None else min(limit_layers, wl.layers)
    t0 = time.time()
    for l in range(layers):
        for j, s in enumerate(wl.mats):
            paths = synth.layer_tensors(wl.wid, l, j, s.m, s.n, ranks_of[j])
            lins.append(lb.Linear.from_numpy(s.m, s.n, paths))
            x = synth.layer_activations(wl, l, j, s.n, T, io="bf16")
            xs.append(torch.from_numpy(x.view(np.int16).copy()).cuda().view(torch.bfloat16))
            ys.append(torch.empty((T, s.m), dtype=torch.bfloat16, device="cuda"))
        if l % 10 == 9:
            log(f"  built {l + 1}/{layers} layers ({time.time() - t0:.0f}s)")
    torch.cuda.synchronize()
    return lins, xs, ys, ranks_of


def time_steps(fn, steps, warmup, torch):
    """Warm up, then time exactly `steps` calls: wall clock between two device
    synchronisations, and one pair of HIP events on the launch stream around
    the same region (per-step events would add their own gaps to the stream)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(st)
    for _ in range(steps):
        fn()
    ev1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, ev0.elapsed_time(ev1) / steps   # seconds; ms per step on the stream


def cpu_baseline(wl, ranks_of, T, budget_s=15.0):
    """The oracle (explicit W, fp64) on whole layers of the workload until the
    time budget is spent; scaled to the full stack per token."""
    import oracle
    import synth
    t_start = time.perf_counter()
    done_layers = 0
    elapsed = 0.0
    for l in range(wl.layers):
        for j, s in enumerate(wl.mats):
            paths = synth.layer_tensors(wl.wid, l, j, s.m, s.n, ranks_of[j])
            x = oracle.decode_bf16(synth.layer_activations(wl, l, j, s.n, T, io="bf16"))
            t0 = time.perf_counter()
            oracle.forward(x, paths, s.m, s.n)
            elapsed += time.perf_counter() - t0
        done_layers += 1
        if time.perf_counter() - t_start > budget_s:
            break
    per_layer = elapsed / done_layers
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max(int(i.get("num_threads", 1)) for i in threadpool_info()) if threadpool_info() else None
    except Exception:
        pass
    if threads is None:
        threads = len(os.sched_getaffinity(0))
    return dict(value=per_layer * wl.layers * 1e6 / T, unit="us/token", cores=threads, kind="oracle",
                sample=f"{done_layers} of {wl.layers} layers ({done_layers * len(wl.mats)} linears), "
                       f"T={T}, explicit fp64 W then x W^T; scaled to the full stack",
                seconds=round(elapsed, 2))


def read_traffic(kernel_file, workload):
    """HBM bytes per launch from committed rocprofv3 counters, if they were taken
    on the current kernel source (else null)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = open(os.path.join(ROOT, "binary_rank_gemm_amd", "csrc", kernel_file), "rb").read()
    if rec.get("kernel_source_sha256") != hashlib.sha256(src).hexdigest():
        return None
    return rec.get("hbm_bytes_per_launch")


def run_decode(args, lb, torch):
    import synth
    wl_name, T, _ = WORKLOADS[args.workload]
    wl = synth.WORKLOADS[wl_name]
    log(f"building {wl.name}: {wl.count} linears, T={T}")
    lins, xs, ys, ranks_of = build_stack(wl, T, lb, torch, args.layers)
    if args.layers:
        wl = dataclasses.replace(wl, layers=min(args.layers, wl.layers))
    S = lb.Stack(lins)
    fn = lambda: S.forward(xs, ys, regime=lb.REGIME_DECODE, use_graph=True)
    wall, kern_ms = time_steps(fn, args.steps, args.warmup, torch)
    byts, flops = algorithmic(wl, ranks_of, T)
    ms = wall * 1e3 / args.steps
    gbps = byts / (kern_ms * 1e-3) / 1e9
    return dict(wl=wl, T=T, ranks_of=ranks_of, ms=ms, kern_ms=kern_ms, bytes=byts, flops=flops,
                gbps=gbps, stack=S, lins=lins)


def run_prefill(args, lb, torch, workload):
    import synth
    wl_name, T, _ = WORKLOADS[workload]
    wl = synth.WORKLOADS[wl_name]
    log(f"building {wl.name}: {wl.count} linears, T={T}")
    lins, xs, ys, ranks_of = build_stack(wl, T, lb, torch, args.layers)
    if args.layers:
        wl = dataclasses.replace(wl, layers=min(args.layers, wl.layers))
    S = lb.Stack(lins)
    fn = lambda: S.forward(xs, ys, regime=lb.REGIME_PREFILL, use_graph=True)
    wall, kern_ms = time_steps(fn, max(2, args.steps // 10), max(1, args.warmup // 5), torch)
    byts, flops = algorithmic(wl, ranks_of, T)
    return dict(workload=f"{wl.name} prefill, {wl.count} linears, {T} tokens", tokens=T, ms_per_step=kern_ms,
                tflops=flops / (kern_ms * 1e-3) / 1e12, frac_of_bf16_peak=flops / (kern_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                algorithmic_tflop=flops / 1e12)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # the GPU's clocks take some tens of milliseconds of load to settle
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="cfg5-decode", choices=sorted(WORKLOADS))
    ap.add_argument("--layers", type=int, default=None, help="limit the stack to this many layers (not for reports)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-only", action="store_true", help="time only the prefill stack (for profiling)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="before timing, run one device-to-device copy of this many MiB (a known-size "
                         "reference for the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (this build has no multi-GPU path)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import binary_rank_gemm_amd as lb
    lb.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_probe_mb:
        nb = args.copy_probe_mb << 20
        src = torch.empty(nb, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy probe: {nb} bytes read + {nb} bytes written")

    if args.prefill_only:
        p = run_prefill(args, lb, torch, "cfg3-prefill")
        log(f"prefill: {p['ms_per_step']:.2f} ms/step, {p['tflops']:.0f} TFLOP/s")
        print(json.dumps({"prefill": p}), flush=True)
        return
    r = run_decode(args, lb, torch)
    wl, T = r["wl"], r["T"]
    log(f"decode: {r['kern_ms'] * 1e3:.1f} us/step (events), {r['ms'] * 1e3:.1f} us/step (wall), {r['gbps']:.0f} GB/s")
    us_per_token = r["ms"] * 1e3 / T
    out = {
        "metric": METRIC,
        "value": round(us_per_token, 3),
        "unit": "us/token",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 I/O; fp8(e4m3 x2) x fp4 MFMA, fp32 accumulate",
        "data": "synthetic (seeded +-1 signs, lognormal fp16 scales, N(0,1) bf16 activations)",
        "config": {"workload": f"{wl.name} decode stack: {wl.layers} layers x 7 linears, both paths, batch {T}",
                   "tokens": T, "linears": wl.count, "ranks": {s.name: r["ranks_of"][j][0] for j, s in enumerate(wl.mats)}},
        "hbm_gbps": round(r["gbps"], 1),
        "hbm_frac": round(r["gbps"] / HBM_PEAK_GBPS, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": "decode step: k_decode_v, k_decode_mid, k_decode_u over all linears (one graph launch)",
            "achieved": round(r["gbps"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(r["gbps"] / HBM_PEAK_GBPS, 4),
            "traffic": read_traffic("lb_decode.hip", args.workload),
            "algorithmic_bytes_per_launch": int(r["bytes"]),
            "kernel_ms_mean": round(r["kern_ms"], 5),
        },
    }
    if not args.no_prefill and args.layers is None:
        try:
            p = run_prefill(args, lb, torch, "cfg3-prefill")
            out["prefill"] = p
            log(f"prefill: {p['ms_per_step']:.2f} ms/step, {p['tflops']:.0f} TFLOP/s")
        except lb.LittleBitError as e:
            out["prefill"] = {"error": str(e)}
    if not args.no_cpu:
        del r["stack"], r["lins"]
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(wl, r["ranks_of"], T)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
