#!/usr/bin/env python3
"""Benchmark of the LittleBit factorised-linear forward on one MI355X.

Default workload: the Llama-2-70B-shaped stack at 0.1 sign bits per weight
(80 layers x {q, k, v, o, gate, up, down}, both paths, 560 linears, 0.91 GB
of packed signs + fp16 scales), decode at batch 1, run as one lb_stack_forward
per step (three kernel launches, V stage, mid stage and U stage, each over
every linear of the stack; the HIP-graph replay of the same three is timed
beside it).  Inputs are seeded synthetic data
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
    "llama2-70b-decode-t1": ("llama2-70b-0.1bpw", 1, "decode"),
    "llama2-70b-decode-t8": ("llama2-70b-0.1bpw", 8, "decode"),
    "llama2-70b-decode-t64": ("llama2-70b-0.1bpw", 64, "decode"),
    "llama2-7b-decode-t1": ("llama2-7b-0.1bpw", 1, "decode"),
    "llama3-8b-decode-t16": ("llama3-8b-0.3bpw", 16, "decode"),
    "llama2-13b-prefill-t2048": ("llama2-13b-0.55bpw", 2048, "prefill"),
    "llama3-8b-prefill-t2048": ("llama3-8b-0.3bpw", 2048, "prefill"),
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


def replay_stats(fn, torch, n=50, cold_mb=0):
    """n replays enqueued back to back, each bracketed by its own pair of HIP
    events on the launch stream (the host runs ahead, so a bracket holds the
    replay's GPU time, not the host's launch latency); with cold_mb, a scratch
    buffer of that size (written once) is read before each replay, outside its
    bracket, so the replay finds none of its data in the 256 MB Infinity Cache
    (and no dirty scratch lines are left to write back during it).
    Returns p10 / p50 / p90 in microseconds."""
    st = torch.cuda.current_stream()
    scratch = torch.ones((cold_mb << 20) // 4, dtype=torch.float32, device="cuda") if cold_mb else None
    evs = []
    fn()
    torch.cuda.synchronize()
    for i in range(n):
        if scratch is not None:
            scratch.sum()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        fn()
        e1.record(st)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    times = [a.elapsed_time(b) * 1e3 for a, b in evs]
    q = np.percentile(np.array(times), [10, 50, 90])
    return {"p10": round(float(q[0]), 2), "p50": round(float(q[1]), 2), "p90": round(float(q[2]), 2)}


def achievable_peaks(torch):
    """What this GPU reaches on plain work, measured in the same run: a graph
    replay of one tiny kernel (launch floor), a streaming read of 4 GiB (the
    library's plain-load probe; torch's sum and copy beside it), a large bf16
    GEMM (hipBLASLt through torch.matmul)."""
    out = {}
    st = torch.cuda.current_stream()
    tiny = torch.zeros(1, device="cuda")
    tiny.add_(1)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tiny.add_(1)
    torch.cuda.synchronize()
    out["launch_floor_us"] = replay_stats(g.replay, torch, n=50)["p50"]

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3   # seconds per call

    big = torch.ones(1 << 30, dtype=torch.float32, device="cuda")
    import binary_rank_gemm_amd as lb
    t = timed(lambda: lb.probe_stream_read(big), 10)
    out["probe_read_gbps"] = round(big.numel() * 4 / t / 1e9, 1)
    t = timed(lambda: big.sum(), 10)
    out["sum_read_gbps"] = round(big.numel() * 4 / t / 1e9, 1)
    dst = torch.empty_like(big)
    t = timed(lambda: dst.copy_(big), 10)
    out["copy_read_write_gbps"] = round(2 * big.numel() * 4 / t / 1e9, 1)
    del big, dst
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    t = timed(lambda: a @ b, 20)
    out["bf16_gemm_8192_tflops"] = round(2 * 8192 ** 3 / t / 1e12, 1)
    del a, b
    torch.cuda.empty_cache()
    return out


def dense_comparators(torch, wl_dec, ranks_dec, wl_pre, ranks_pre, T_pre):
    """The same shapes run the dense way, for the pages' comparison with an
    fp16 model and with decompress-then-compute: (1) dense bf16 weights, one
    GEMV per linear per token; (2) W rebuilt per forward from its factors as
    bf16 GEMMs, then the GEMV; (3) dense bf16 prefill GEMMs.  One layer's
    weights are generated and reused for every layer (each layer's weights
    exceed the Infinity Cache, so every GEMV still streams them from HBM).
    Dense weights are [m, n] as a PyTorch Linear holds them (F.linear: one 2-D
    GEMM per call, hipBLASLt's preferred NT form); no batched products."""
    st = torch.cuda.current_stream()

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    out = {}
    # (1) dense decode (weights [m, n] as a PyTorch Linear holds them; y = x W^T)
    wts = [torch.randn(s.m, s.n, device="cuda", dtype=torch.bfloat16, generator=gen) for s in wl_dec.mats]
    xs = [torch.randn(1, s.n, device="cuda", dtype=torch.bfloat16, generator=gen) for s in wl_dec.mats]

    def dense_step():
        for _ in range(wl_dec.layers):
            for x, w in zip(xs, wts):
                torch.nn.functional.linear(x, w)
    out["dense_bf16_decode_us_per_token"] = round(timed(dense_step, 3) * 1e6, 1)
    del wts
    # (2) decompress-then-compute: W = sum_p (h o U o l)(V o g)^T rebuilt as bf16 GEMMs, then the GEMV
    facs = []
    for j, s in enumerate(wl_dec.mats):
        per = []
        for r in ranks_dec[j]:
            a = torch.randn(s.m, r, device="cuda", dtype=torch.bfloat16, generator=gen)
            b = torch.randn(r, s.n, device="cuda", dtype=torch.bfloat16, generator=gen)
            per.append((a, b))
        facs.append(per)
    wbuf = [torch.empty(s.m, s.n, device="cuda", dtype=torch.bfloat16) for s in wl_dec.mats]
    xs_t = [x.t().contiguous() for x in xs]   # [n, 1]

    def rebuild_step():
        for _ in range(wl_dec.layers):
            for per, w, xt in zip(facs, wbuf, xs_t):
                torch.matmul(per[0][0], per[0][1], out=w)
                for a, b in per[1:]:
                    w.addmm_(a, b)
                torch.matmul(w, xt)
    out["decompress_then_compute_us_per_token"] = round(timed(rebuild_step, 1) * 1e6, 1)
    del facs, wbuf
    # (3) dense prefill
    wts = [torch.randn(s.m, s.n, device="cuda", dtype=torch.bfloat16, generator=gen) for s in wl_pre.mats]
    xs = [torch.randn(T_pre, s.n, device="cuda", dtype=torch.bfloat16, generator=gen) for s in wl_pre.mats]

    def dense_prefill():
        for _ in range(wl_pre.layers):
            for x, w in zip(xs, wts):
                torch.nn.functional.linear(x, w)
    out["dense_bf16_prefill_ms"] = round(timed(dense_prefill, 3) * 1e3, 2)
    del wts, xs
    torch.cuda.empty_cache()
    return out


def cpu_info():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            blas = f"{info[0].get('internal_api')} ({info[0].get('num_threads')} threads)"
    except Exception:
        pass
    return dict(cpu_model=model, cpu_count=os.cpu_count(), affinity=len(os.sched_getaffinity(0)), blas=blas)


def cpu_baseline(wl, ranks_of, T, budget_s=15.0):
    """The oracle (explicit W, fp64) on whole layers of the workload until the
    time budget is spent; scaled to the full stack per token."""
    import oracle
    import synth
    t_start = time.perf_counter()
    done_layers = 0
    elapsed = 0.0
    elapsed_f = 0.0
    for l in range(wl.layers):
        for j, s in enumerate(wl.mats):
            paths = synth.layer_tensors(wl.wid, l, j, s.m, s.n, ranks_of[j])
            x = oracle.decode_bf16(synth.layer_activations(wl, l, j, s.n, T, io="bf16"))
            t0 = time.perf_counter()
            oracle.forward(x, paths, s.m, s.n)
            t1 = time.perf_counter()
            oracle.forward_factored(x, paths, s.m, s.n)
            elapsed += t1 - t0
            elapsed_f += time.perf_counter() - t1
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
                seconds=round(elapsed, 2),
                factored_fp64_us_per_token=round(elapsed_f / done_layers * wl.layers * 1e6 / T, 1),
                **cpu_info())


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
    # direct launches of the decode kernels: on this ROCm a HIP graph replay
    # adds a few us of its own per replay (timed below and reported beside).
    # The stack is bound to its buffers once, so each step is one C-ABI call
    # with no per-call marshalling of the 560 pointers.
    fn = S.bind(xs, ys, regime=lb.REGIME_DECODE, use_graph=False).forward
    wall, kern_ms = time_steps(fn, args.steps, args.warmup, torch)
    fn_g = S.bind(xs, ys, regime=lb.REGIME_DECODE, use_graph=True).forward
    _, graph_ms = time_steps(fn_g, args.steps, args.warmup, torch)
    byts, flops = algorithmic(wl, ranks_of, T)
    ms = wall * 1e3 / args.steps
    gbps = byts / (kern_ms * 1e-3) / 1e9
    return dict(wl=wl, T=T, ranks_of=ranks_of, ms=ms, kern_ms=kern_ms, graph_ms=graph_ms, bytes=byts, flops=flops,
                gbps=gbps, stack=S, lins=lins, xs=xs, ys=ys)


def run_chained(r, lb, torch, steps=20, warmup=5):
    """The same linears listed in a model's real order and chained through
    their buffers (per layer: q, k, v read the layer input; o reads q's
    output; gate and up read o's; down reads gate's; the next layer reads
    down's), so the stack runs level after level: per-token latency of a real
    model's linears at batch 1, where the independent stack is a bandwidth
    figure.  Outputs of k, v and up are not consumed (attention and the MLP's
    elementwise product are not part of the method)."""
    wl, T, lins = r["wl"], r["T"], r["lins"]
    d_model = wl.mats[0].n
    x0 = torch.randn(T, d_model, device="cuda").to(torch.bfloat16)
    ys = [torch.empty((T, lins[i].d_out), dtype=torch.bfloat16, device="cuda") for i in range(len(lins))]
    xs = []
    names = [s.name for s in wl.mats]
    qi, oi, gi, di = names.index("q"), names.index("o"), names.index("gate"), names.index("down")
    for l in range(wl.layers):
        b = 7 * l
        inp = x0 if l == 0 else ys[b - 7 + di]
        src = {"q": inp, "k": inp, "v": inp, "o": ys[b + qi], "gate": ys[b + oi], "up": ys[b + oi],
               "down": ys[b + gi]}
        xs += [src[nm] for nm in names]
    S = lb.Stack(lins)
    out = {}
    for lab, g in (("direct", False), ("graph", True)):
        fn = S.bind(xs, ys, regime=lb.REGIME_DECODE, use_graph=g).forward
        _, ms = time_steps(fn, steps, warmup, torch)
        out[f"us_per_token_{lab}"] = round(ms * 1e3 / T, 1)
    out["levels"] = 4 * wl.layers
    out["workload"] = f"{wl.name}: {wl.count} linears chained in model order, batch {T}"
    S.close()
    return out


def run_prefill(args, lb, torch, workload):
    import synth
    wl_name, T, _ = WORKLOADS[workload]
    wl = synth.WORKLOADS[wl_name]
    log(f"building {wl.name}: {wl.count} linears, T={T}")
    lins, xs, ys, ranks_of = build_stack(wl, T, lb, torch, args.layers)
    if args.layers:
        wl = dataclasses.replace(wl, layers=min(args.layers, wl.layers))
    S = lb.Stack(lins)
    fn = S.bind(xs, ys, regime=lb.REGIME_PREFILL, use_graph=True).forward
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
    ap.add_argument("--workload", default="llama2-70b-decode-t1", choices=sorted(WORKLOADS))
    ap.add_argument("--layers", type=int, default=None, help="limit the stack to this many layers (not for reports)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-only", action="store_true", help="time only the prefill stack (for profiling)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the per-replay and cold-cache timings, the achievable-peak probes and the dense comparators")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="before timing, run one device-to-device copy of this many MiB (a known-size "
                         "reference for the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the library has no multi-GPU path)",
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
        # a prefill workload named by --workload, else the 13B stack at 2048 tokens
        wk = args.workload if WORKLOADS[args.workload][2] == "prefill" else "llama2-13b-prefill-t2048"
        p = run_prefill(args, lb, torch, wk)
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
            "kernel": "decode step: k_decode_v, k_decode_mid, k_decode_u over all linears (three direct launches)",
            "achieved": round(r["gbps"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(r["gbps"] / HBM_PEAK_GBPS, 4),
            "traffic": read_traffic("lb_decode.hip", args.workload),
            "algorithmic_bytes_per_launch": int(r["bytes"]),
            "kernel_ms_mean": round(r["kern_ms"], 5),
        },
        "graph_replay_us_per_step": round(r["graph_ms"] * 1e3, 2),
    }
    fn = r["stack"].bind(r["xs"], r["ys"], regime=lb.REGIME_DECODE, use_graph=False).forward
    if not args.no_context:
        out["decode_replays"] = {"n": 50, "warm_us": replay_stats(fn, torch, 50),
                                 "cold_us": replay_stats(fn, torch, 50, cold_mb=512), "cold_scratch_mb": 512}
        if args.layers is None:
            out["chained_decode"] = run_chained(r, lb, torch)
            log(f"chained decode: {out['chained_decode']}")
    if not args.no_prefill and args.layers is None:
        try:
            p = run_prefill(args, lb, torch, "llama2-13b-prefill-t2048")
            out["prefill"] = p
            log(f"prefill: {p['ms_per_step']:.2f} ms/step, {p['tflops']:.0f} TFLOP/s")
        except lb.LittleBitError as e:
            out["prefill"] = {"error": str(e)}
    del r["stack"], r["lins"], r["xs"], r["ys"], fn
    torch.cuda.empty_cache()
    if not args.no_context and args.layers is None:
        import synth
        ctx = achievable_peaks(torch)
        ctx["decode_frac_of_probe_read"] = round(r["gbps"] / ctx["probe_read_gbps"], 4)
        if "prefill" in out and "tflops" in out["prefill"]:
            ctx["prefill_frac_of_bf16_gemm"] = round(out["prefill"]["tflops"] / ctx["bf16_gemm_8192_tflops"], 4)
        out["achievable_peaks"] = ctx
        wl_pre_name, T_pre, _ = WORKLOADS["llama2-13b-prefill-t2048"]
        wl_pre = synth.WORKLOADS[wl_pre_name]
        cmp_ = dense_comparators(torch, wl, r["ranks_of"], wl_pre, [ranks_for(wl_pre, s, lb) for s in wl_pre.mats], T_pre)
        cmp_["speedup_vs_dense_bf16_decode"] = round(cmp_["dense_bf16_decode_us_per_token"] / us_per_token, 1)
        cmp_["speedup_vs_decompress_then_compute"] = round(cmp_["decompress_then_compute_us_per_token"] / us_per_token, 1)
        if "prefill" in out and "ms_per_step" in out["prefill"]:
            cmp_["speedup_vs_dense_bf16_prefill"] = round(cmp_["dense_bf16_prefill_ms"] / out["prefill"]["ms_per_step"], 2)
        out["comparators"] = cmp_
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(wl, r["ranks_of"], T)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
