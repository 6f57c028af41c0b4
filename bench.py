#!/usr/bin/env python3
"""Benchmark of the LittleBit factorised-linear forward on one MI355X.

Default workload (the headline): the Llama-2-70B-shaped stack at 0.1 sign
bits per weight (80 layers x {q, k, v, o, gate, up, down}, both paths, 560
linears, 0.91 GB of packed signs + fp16 scales), decode at batch 1, run as
one lb_stack_forward per step.  Inputs are seeded synthetic data resident in
HBM before timing starts.

Prints one JSON line: the decode step's microseconds per token and achieved
HBM GB/s (algorithmic bytes), the roofline of the dominant kernel, the sign-
and scale-bit budget of every workload, the token sweep of the same stack
(2 to 64 tokens, AUTO's choice and both regimes), the other stacks (Llama-2-7B at batch 1 warm and cold,
Llama-3-8B at 16 tokens), the prefill stack's effective TFLOP/s (Llama-2-13B
shape, 2048 tokens), the dense and decompress-then-compute comparators, and
the CPU oracle timed on a bounded sample.
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


def bit_budget(wl, ranks_of):
    """Sign bits and fp16 scale bits per original weight over the whole stack,
    from the shapes and ranks: two paths of rank r store r (m + n) sign bits
    each and 16 (m + n + r) scale bits each for m n weights.  The rank rule
    spends the sign-bit budget only; the scale bits come on top."""
    weights = sum(s.m * s.n for s in wl.mats)
    sign = sum(sum(r * (s.m + s.n) for r in ranks_of[j]) for j, s in enumerate(wl.mats))
    scale = sum(sum(16 * (s.m + s.n + r) for r in ranks_of[j]) for j, s in enumerate(wl.mats))
    return {"target_bpw": float(wl.bpw) if wl.bpw is not None else None,
            "sign_bpw": round(sign / weights, 5), "scale_bpw": round(scale / weights, 5),
            "total_bpw": round((sign + scale) / weights, 5)}


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
            xs.append(activations(wl, l, j, s.n, T, torch))
            ys.append(torch.empty((T, s.m), dtype=torch.bfloat16, device="cuda"))
        if l % 20 == 19:
            log(f"  built {l + 1}/{layers} layers ({time.time() - t0:.0f}s)")
    torch.cuda.synchronize()
    return lins, xs, ys, ranks_of


def activations(wl, l, j, n, T, torch):
    import synth
    x = synth.layer_activations(wl, l, j, n, T, io="bf16")
    return torch.from_numpy(x.view(np.int16).copy()).cuda().view(torch.bfloat16)


def settle(fn, seconds, torch):
    """Runs fn back to back for `seconds` of wall time (outside any timed
    region): the GPU's clocks need some tens of milliseconds of sustained load
    to settle, and a fixed count of warm-up steps is too short for a 0.2 ms
    step.  Returns the number of calls made."""
    n = 0
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
        n += 20
    return n


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


def alternating(fns, steps, rounds, torch):
    """Each named fn timed `rounds` times in alternating order (a, b, a, b, ...)
    after one settle pass of each, so clock ramps and drift weigh on all alike.
    Returns the median ms per step (HIP events) of each."""
    out = {k: [] for k in fns}
    for k, f in fns.items():
        settle(f, 0.3, torch)
    for _ in range(rounds):
        for k, f in fns.items():
            _, ms = time_steps(f, steps, 2, torch)
            out[k].append(ms)
    return {k: float(np.median(v)) for k, v in out.items()}


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


def timed_calls(fn, reps, torch):
    st = torch.cuda.current_stream()
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


def achievable_peaks(torch):
    """What this GPU reaches on plain work, measured in the same run: a graph
    replay of one tiny kernel (launch floor), a streaming read of 4 GiB (a
    plain-load probe kernel; torch's sum and copy beside it), a large bf16
    GEMM (hipBLASLt through torch.matmul)."""
    out = {}
    tiny = torch.zeros(1, device="cuda")
    tiny.add_(1)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tiny.add_(1)
    torch.cuda.synchronize()
    out["launch_floor_us"] = replay_stats(g.replay, torch, n=50)["p50"]
    big = torch.ones(1 << 30, dtype=torch.float32, device="cuda")
    import binary_rank_gemm_amd.probe as probe
    settle(lambda: probe.stream_read(big), 0.5, torch)
    t = timed_calls(lambda: probe.stream_read(big), 20, torch)
    out["probe_read_gbps"] = round(big.numel() * 4 / t / 1e9, 1)
    t = timed_calls(lambda: big.sum(), 10, torch)
    out["sum_read_gbps"] = round(big.numel() * 4 / t / 1e9, 1)
    dst = torch.empty_like(big)
    t = timed_calls(lambda: dst.copy_(big), 10, torch)
    out["copy_read_write_gbps"] = round(2 * big.numel() * 4 / t / 1e9, 1)
    del big, dst
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    t = timed_calls(lambda: a @ b, 20, torch)
    out["bf16_gemm_8192_tflops"] = round(2 * 8192 ** 3 / t / 1e12, 1)
    del a, b
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------
# comparators: the same layers the dense way and decompress-then-compute
# ----------------------------------------------------------------------------

def unpack_signs_torch(words, rank, torch):
    """Canonical packed sign words (int32 [rows, ceil(rank/32)] on the device)
    -> float32 +-1 [rows, rank]: entry j of a row is -1 iff bit j % 32 of its
    word j // 32 is set."""
    j = torch.arange(rank, device=words.device)
    bits = torch.bitwise_and(torch.bitwise_right_shift(words[:, j // 32], (j % 32).to(torch.int32)), 1)
    return (1 - 2 * bits).to(torch.float32)


def decompress_weight(paths_dev, torch):
    """W = sum_p diag(h_p) U_p diag(l_p) V_p^T diag(g_p) as a bf16 [m, n]
    tensor, rebuilt from the layer's packed signs and fp16 scales the way a
    dense framework would: unpack the bits, scale, one bf16 GEMM per path
    (fp32 accumulation), summed.  paths_dev: dicts of device tensors u, v
    (int32 words), h, g, l (int16 fp16 bits) and rank."""
    W = None
    for p in paths_dev:
        r = int(p["rank"])
        h = p["h"].view(torch.float16).float()
        g = p["g"].view(torch.float16).float()
        l = p["l"].view(torch.float16).float()
        A = (unpack_signs_torch(p["u"], r, torch) * h[:, None] * l[None, :]).to(torch.bfloat16)   # [m, r]
        B = (unpack_signs_torch(p["v"], r, torch) * g[:, None]).to(torch.bfloat16)                # [n, r]
        Wp = torch.matmul(A, B.t().contiguous())
        W = Wp if W is None else W + Wp
    return W


def decompress_then_compute(paths_dev, x, torch):
    """y = x W^T with W rebuilt from its factors first (the comparison the
    pages draw between a factorised forward and unpacking the weight)."""
    return torch.nn.functional.linear(x, decompress_weight(paths_dev, torch))


def upload_paths(paths, torch):
    dev = []
    for p in paths:
        dev.append(dict(rank=int(p["rank"]),
                        u=torch.from_numpy(np.ascontiguousarray(p["u_words"]).view(np.int32)).cuda(),
                        v=torch.from_numpy(np.ascontiguousarray(p["v_words"]).view(np.int32)).cuda(),
                        h=torch.from_numpy(np.ascontiguousarray(p["h"]).view(np.int16)).cuda(),
                        g=torch.from_numpy(np.ascontiguousarray(p["g"]).view(np.int16)).cuda(),
                        l=torch.from_numpy(np.ascontiguousarray(p["l"]).view(np.int16)).cuda()))
    return dev


def dense_comparators(torch, wl_dec, ranks_dec, wl_pre, T_pre):
    """The same shapes run the dense way: (1) dense bf16 weights, one GEMV per
    linear per token (one layer's weights generated and reused for every
    layer; each exceeds the Infinity Cache, so every GEMV streams it from
    HBM); (2) decompress-then-compute: layer 0's own packed signs and fp16
    scales unpacked and multiplied out into a bf16 W every forward, then the
    GEMV; timed on that layer and scaled by the layer count (every layer has
    the same shapes); (3) dense bf16 prefill GEMMs."""
    import synth
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    out = {}
    wts = [torch.randn(s.m, s.n, device="cuda", dtype=torch.bfloat16, generator=gen) for s in wl_dec.mats]
    xs = [torch.randn(1, s.n, device="cuda", dtype=torch.bfloat16, generator=gen) for s in wl_dec.mats]

    def dense_step():
        for _ in range(wl_dec.layers):
            for x, w in zip(xs, wts):
                torch.nn.functional.linear(x, w)
    out["dense_bf16_decode_us_per_token"] = round(timed_calls(dense_step, 3, torch) * 1e6, 1)
    del wts
    layer0 = [upload_paths(synth.layer_tensors(wl_dec.wid, 0, j, s.m, s.n, ranks_dec[j]), torch)
              for j, s in enumerate(wl_dec.mats)]

    def rebuild_layer():
        for p, x in zip(layer0, xs):
            decompress_then_compute(p, x, torch)
    t_layer = timed_calls(rebuild_layer, 3, torch)
    out["decompress_then_compute_us_per_token"] = round(t_layer * wl_dec.layers * 1e6, 1)
    out["decompress_then_compute_sample"] = (f"layer 0 of {wl_dec.name} ({len(wl_dec.mats)} linears, its own packed "
                                             f"signs and fp16 scales), {t_layer * 1e6:.0f} us per layer, "
                                             f"x {wl_dec.layers} layers")
    del layer0
    wts = [torch.randn(s.m, s.n, device="cuda", dtype=torch.bfloat16, generator=gen) for s in wl_pre.mats]
    xs = [torch.randn(T_pre, s.n, device="cuda", dtype=torch.bfloat16, generator=gen) for s in wl_pre.mats]

    def dense_prefill():
        for _ in range(wl_pre.layers):
            for x, w in zip(xs, wts):
                torch.nn.functional.linear(x, w)
    out["dense_bf16_prefill_ms"] = round(timed_calls(dense_prefill, 3, torch) * 1e3, 2)
    del wts, xs
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------
# CPU baseline (the oracle on the host cores)
# ----------------------------------------------------------------------------

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


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

REGIME_NAMES = {0: "auto", 1: "exact", 2: "decode", 3: "prefill"}


def run_decode(args, lb, torch):
    import synth
    wl_name, T, _ = WORKLOADS[args.workload]
    wl = synth.WORKLOADS[wl_name]
    log(f"building {wl.name}: {wl.count} linears, T={T}")
    lins, xs, ys, ranks_of = build_stack(wl, T, lb, torch, args.layers)
    if args.layers:
        wl = dataclasses.replace(wl, layers=min(args.layers, wl.layers))
    S = lb.Stack(lins)
    # The stack is bound to its buffers once, so each step is one C-ABI call
    # with no per-call marshalling of the 560 pointers; the library's own
    # choice of launch form (lb_stack_forward).
    regime = {"auto": lb.REGIME_AUTO, "decode": lb.REGIME_DECODE, "prefill": lb.REGIME_PREFILL}[args.regime]
    fn = S.bind(xs, ys, regime=regime, use_graph=None if regime == lb.REGIME_AUTO else False).forward
    n_settle = settle(fn, args.settle_s, torch)
    wall, kern_ms = time_steps(fn, args.steps, args.warmup, torch)
    byts, flops = algorithmic(wl, ranks_of, T)
    ms = wall * 1e3 / args.steps
    gbps = byts / (kern_ms * 1e-3) / 1e9
    return dict(wl=wl, T=T, ranks_of=ranks_of, ms=ms, kern_ms=kern_ms, bytes=byts, flops=flops, gbps=gbps,
                stack=S, lins=lins, xs=xs, ys=ys, settle_calls=n_settle)


def launch_forms(r, lb, torch, steps):
    """Direct launches against the same launches captured in a HIP graph,
    timed in alternating order (three rounds each, medians)."""
    S, xs, ys = r["stack"], r["xs"], r["ys"]
    fns = {"direct": S.bind(xs, ys, regime=lb.REGIME_DECODE, use_graph=False).forward,
           "graph": S.bind(xs, ys, regime=lb.REGIME_DECODE, use_graph=True).forward}
    med = alternating(fns, steps, 3, torch)
    return {f"{k}_us_per_step": round(v * 1e3, 2) for k, v in med.items()} | {"rounds": 3, "order": "alternating"}


def token_sweep(r, lb, torch, tokens=(2, 4, 8, 16, 32, 64), steps=20):
    """The same linears at other token counts: the regime AUTO picks, and each
    regime forced, µs per step and per token, with algorithmic GB/s and the
    fraction of the larger of the HBM and MFMA roofline times."""
    wl, lins, S = r["wl"], r["lins"], r["stack"]
    out = {}
    for T in tokens:
        xs = [activations(wl, i // len(wl.mats), i % len(wl.mats), lin.d_in, T, torch) for i, lin in enumerate(lins)]
        ys = [torch.empty((T, lin.d_out), dtype=torch.bfloat16, device="cuda") for lin in lins]
        byts, flops = algorithmic(wl, r["ranks_of"], T)
        t_roof = max(byts / (HBM_PEAK_GBPS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12))
        rec = {"algorithmic_bytes": int(byts), "algorithmic_gflop": round(flops / 1e9, 2),
               "roofline_us": round(t_roof * 1e6, 1)}
        for name, rg in (("auto", lb.REGIME_AUTO), ("decode", lb.REGIME_DECODE), ("prefill", lb.REGIME_PREFILL)):
            fn = S.bind(xs, ys, regime=rg, use_graph=None if rg == lb.REGIME_AUTO else False).forward
            settle(fn, 0.2, torch)
            _, ms = time_steps(fn, steps, 3, torch)
            rec[f"{name}_us_per_step"] = round(ms * 1e3, 1)
        rec["auto_picks"] = REGIME_NAMES[lb.auto_regime(lins, T)]
        rec["us_per_token"] = round(rec["auto_us_per_step"] / T, 2)
        rec["hbm_gbps"] = round(byts / (rec["auto_us_per_step"] * 1e-6) / 1e9, 1)
        rec["frac_of_roofline"] = round(t_roof * 1e6 / rec["auto_us_per_step"], 4)
        out[f"T{T}"] = rec
        log(f"  {wl.name} T={T}: {rec}")
        del xs, ys
    return out


def other_decode_stack(name, T, lb, torch, steps, cold_mb=0):
    """A whole decode stack at T tokens (library's choice of regime and launch
    form): µs per step, warm (back-to-back steps) and, with cold_mb, cold (a
    cold_mb scratch buffer read before each step, outside its timing)."""
    import synth
    wl = synth.WORKLOADS[name]
    log(f"building {wl.name}: {wl.count} linears, T={T}")
    lins, xs, ys, ranks_of = build_stack(wl, T, lb, torch)
    S = lb.Stack(lins)
    fn = S.bind(xs, ys).forward
    settle(fn, 0.3, torch)
    _, ms = time_steps(fn, steps, 5, torch)
    byts, flops = algorithmic(wl, ranks_of, T)
    t_roof = max(byts / (HBM_PEAK_GBPS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12))
    rec = {"workload": f"{wl.name}: {wl.count} linears, batch {T}", "tokens": T,
           "warm_us_per_step": round(ms * 1e3, 2), "warm_hbm_gbps": round(byts / (ms * 1e-3) / 1e9, 1),
           "algorithmic_bytes": int(byts), "roofline_us": round(t_roof * 1e6, 1),
           "bit_budget": bit_budget(wl, ranks_of)}
    if cold_mb:
        cold = replay_stats(fn, torch, 50, cold_mb=cold_mb)
        rec["cold_us"] = cold
        rec["cold_scratch_mb"] = cold_mb
        rec["cold_hbm_gbps_p50"] = round(byts / (cold["p50"] * 1e-6) / 1e9, 1)
        rec["cold_frac_of_hbm"] = round(byts / (cold["p50"] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
    S.close()
    del S, lins, xs, ys, fn
    torch.cuda.empty_cache()
    log(f"  {rec}")
    return rec


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
    # one stack runs the levels in one persistent launch, the other (the
    # default) as three launches per level; a graph replays the level launches
    S = lb.Stack(lins)
    S.set_persistent(1)
    SL = lb.Stack(lins)
    fns = {"persistent": S.bind(xs, ys, regime=lb.REGIME_DECODE, use_graph=False).forward,
           "levels": SL.bind(xs, ys, regime=lb.REGIME_DECODE, use_graph=False).forward,
           "graph": SL.bind(xs, ys, regime=lb.REGIME_DECODE, use_graph=True).forward,
           "auto": SL.bind(xs, ys).forward}
    med = alternating(fns, steps, 2, torch)
    st = S.persistent_status()
    out = {f"us_per_token_{k}": round(v * 1e3 / T, 1) for k, v in med.items()}
    out["levels"] = 4 * wl.layers
    out["us_per_level_persistent"] = round(med["persistent"] * 1e3 / (4 * wl.layers), 2)
    out["us_per_level_launches"] = round(med["levels"] * 1e3 / (4 * wl.layers), 2)
    out["persistent_active"] = st["active"]
    out["persistent_aborted"] = st["aborted"]
    out["workload"] = f"{wl.name}: {wl.count} linears chained in model order, batch {T}"
    S.close()
    SL.close()
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
    fn = S.bind(xs, ys).forward
    settle(fn, min(0.3, args.settle_s), torch)
    steps = max(10, args.steps // 10)
    wall, kern_ms = time_steps(fn, steps, 2, torch)
    byts, flops = algorithmic(wl, ranks_of, T)
    rec = dict(workload=f"{wl.name} prefill, {wl.count} linears, {T} tokens", tokens=T, steps=steps,
               ms_per_step=round(kern_ms, 4), tflops=round(flops / (kern_ms * 1e-3) / 1e12, 1),
               frac_of_bf16_peak=round(flops / (kern_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
               algorithmic_tflop=round(flops / 1e12, 3), bit_budget=bit_budget(wl, ranks_of))
    S.close()
    del S, lins, xs, ys, fn
    torch.cuda.empty_cache()
    return rec


FP32_PEAK_TFLOPS = 157.3       # MI355X dense fp32 (matrix cores and vector units alike)


def run_fp32_tiled(lb, torch, layers=2, T=2048):
    """fp32 I/O at many tokens (the exact regime's tiled fp32 matrix-core
    form): the first `layers` layers of the Llama-2-13B-shaped stack at 2048
    fp32 tokens, effective TFLOP/s against the fp32 peak."""
    import synth
    wl = synth.WORKLOADS["llama2-13b-0.55bpw"]
    ranks_of = [ranks_for(wl, s, lb) for s in wl.mats]
    lins, xs, ys = [], [], []
    for l in range(layers):
        for j, s in enumerate(wl.mats):
            lins.append(lb.Linear.from_numpy(s.m, s.n, synth.layer_tensors(wl.wid, l, j, s.m, s.n, ranks_of[j])))
            x = synth.activations((wl.wid, l, j, 88, T), T, s.n, io="fp32")
            xs.append(torch.from_numpy(x).cuda())
            ys.append(torch.empty((T, s.m), dtype=torch.float32, device="cuda"))
    S = lb.Stack(lins)
    fn = S.bind(xs, ys).forward
    settle(fn, 0.3, torch)
    _, ms = time_steps(fn, 3, 1, torch)
    flops = sum(2 * T * (s.m + s.n) * sum(ranks_of[j]) for j, s in enumerate(wl.mats)) * layers
    rec = {"workload": f"{wl.name}: first {layers} layers ({len(lins)} linears), {T} fp32 tokens, fp32 I/O",
           "ms_per_step": round(ms, 3), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
           "frac_of_fp32_peak": round(flops / (ms * 1e-3) / 1e12 / FP32_PEAK_TFLOPS, 4),
           "regime": REGIME_NAMES[lb.auto_regime(lins, T, lb.FP32)]}
    S.close()
    del S, lins, xs, ys, fn
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="seconds of untimed steps before the warm-up, so the clocks have settled whatever --warmup is")
    ap.add_argument("--workload", default="llama2-70b-decode-t1", choices=sorted(WORKLOADS))
    ap.add_argument("--layers", type=int, default=None, help="limit the stack to this many layers (not for reports)")
    ap.add_argument("--regime", default="auto", choices=["auto", "decode", "prefill"],
                    help="regime of the headline stack's timed steps (auto: the library's choice)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-only", action="store_true", help="time only the prefill stack (for profiling)")
    ap.add_argument("--fp32-tiled-only", action="store_true",
                    help="time only the fp32 tiled (exact regime, many tokens) stack (for profiling)")
    ap.add_argument("--chained-only", action="store_true",
                    help="time only the headline stack chained in model order (persistent launch, level launches)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the launch-form and replay timings, the token sweep, the other stacks, the "
                         "achievable-peak probes and the comparators")
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

    if args.fp32_tiled_only:
        rec = run_fp32_tiled(lb, torch)
        log(f"fp32 tiled: {rec}")
        print(json.dumps({"fp32_tiled": rec}), flush=True)
        return
    if args.prefill_only:
        # a prefill workload named by --workload, else the 13B stack at 2048 tokens
        wk = args.workload if WORKLOADS[args.workload][2] == "prefill" else "llama2-13b-prefill-t2048"
        p = run_prefill(args, lb, torch, wk)
        log(f"prefill: {p['ms_per_step']:.2f} ms/step, {p['tflops']:.0f} TFLOP/s")
        print(json.dumps({"prefill": p}), flush=True)
        return
    r = run_decode(args, lb, torch)
    wl, T = r["wl"], r["T"]
    if args.chained_only:
        c = run_chained(r, lb, torch, steps=max(5, args.steps // 10))
        log(f"chained decode: {c}")
        print(json.dumps({"chained_decode": c}), flush=True)
        return
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
        "clock_settle": {"seconds": args.settle_s, "steps": r["settle_calls"],
                         "note": "untimed steps run before the warm-up so the clocks have settled"},
        "bit_budget": bit_budget(wl, r["ranks_of"]),
        "hbm_gbps": round(r["gbps"], 1),
        "hbm_frac": round(r["gbps"] / HBM_PEAK_GBPS, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": "decode step of the stack (the decode kernels over all 560 linears, direct launches)",
            "achieved": round(r["gbps"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(r["gbps"] / HBM_PEAK_GBPS, 4),
            "traffic": read_traffic("lb_decode.hip", args.workload),
            "algorithmic_bytes_per_launch": int(r["bytes"]),
            "kernel_ms_mean": round(r["kern_ms"], 5),
        },
    }
    fn = r["stack"].bind(r["xs"], r["ys"]).forward
    full = args.layers is None
    if not args.no_context:
        out["launch_forms"] = launch_forms(r, lb, torch, max(20, args.steps // 4))
        out["decode_replays"] = {"n": 50, "warm_us": replay_stats(fn, torch, 50),
                                 "cold_us": replay_stats(fn, torch, 50, cold_mb=512), "cold_scratch_mb": 512}
        if full:
            out["token_sweep"] = token_sweep(r, lb, torch)
            out["chained_decode"] = run_chained(r, lb, torch)
            log(f"chained decode: {out['chained_decode']}")
    wl_dec, ranks_dec = wl, r["ranks_of"]
    del r["stack"], r["lins"], r["xs"], r["ys"], fn
    torch.cuda.empty_cache()
    if not args.no_context and full:
        out["other_stacks"] = {
            "llama2-7b-decode-t1": other_decode_stack("llama2-7b-0.1bpw", 1, lb, torch, 100, cold_mb=512),
            "llama3-8b-decode-t16": other_decode_stack("llama3-8b-0.3bpw", 16, lb, torch, 50),
        }
    if not args.no_prefill and full:
        try:
            p = run_prefill(args, lb, torch, "llama2-13b-prefill-t2048")
            out["prefill"] = p
            log(f"prefill: {p['ms_per_step']:.2f} ms/step, {p['tflops']:.0f} TFLOP/s")
        except lb.LittleBitError as e:
            out["prefill"] = {"error": str(e)}
    if not args.no_context and full:
        out["fp32_tiled"] = run_fp32_tiled(lb, torch)
        log(f"fp32 tiled: {out['fp32_tiled']}")
        import synth
        ctx = achievable_peaks(torch)
        ctx["decode_frac_of_probe_read"] = round(r["gbps"] / ctx["probe_read_gbps"], 4)
        if "prefill" in out and "tflops" in out["prefill"]:
            ctx["prefill_frac_of_bf16_gemm"] = round(out["prefill"]["tflops"] / ctx["bf16_gemm_8192_tflops"], 4)
        out["achievable_peaks"] = ctx
        wl_pre = synth.WORKLOADS[WORKLOADS["llama2-13b-prefill-t2048"][0]]
        cmp_ = dense_comparators(torch, wl_dec, ranks_dec, wl_pre, 2048)
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
