"""Full-size parity: whole layers of the benchmark stacks at their real shapes,
run the way the benchmark runs them (one stack forward, HIP graph, the
benchmark's regime), checked against the oracle on a seeded sample of output
channels for every token (the oracle forms only the sampled rows of W).

Workloads (shapes of "LittleBit: Ultra Low-Bit Quantization via Latent
Factorization", experiments section: Llama-2 7B / 13B / 70B and Llama-3 8B
linears; ranks from the sign-bit budget): decode at batch 1, 8, 16, 64 and
prefill at 2048 tokens.
"""
from fractions import Fraction

import numpy as np
import pytest

import binary_rank_gemm_amd as lb
import oracle
import synth
from lbtest import assert_bf16_close, assert_fp32_close, log, to_f64, x_f64, x_tensor

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SAMPLE_ROWS = 48

# (workload, tokens, regime, layers checked)
CASES = [
    ("llama2-70b-0.1bpw", 1, "decode", (0, 79)),
    ("llama2-70b-0.1bpw", 8, "decode", (41,)),
    ("llama2-70b-0.1bpw", 64, "decode", (7,)),
    ("llama2-7b-0.1bpw", 1, "decode", (0, 31)),
    ("llama3-8b-0.3bpw", 16, "decode", (3,)),
    ("llama3-8b-0.3bpw", 2048, "prefill", (0,)),
    ("llama2-13b-0.55bpw", 2048, "prefill", (39,)),
]


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu(gpu):
    return gpu


def ranks(wl, spec):
    if wl.bpw is None:
        return [wl.fixed_rank, wl.fixed_rank]
    r = oracle.rank_for_bpw(spec.m, spec.n, Fraction(wl.bpw), spec.rank_mult)
    return [r, r]


@pytest.mark.parametrize("name,T,regime,layers", CASES, ids=[f"{c[0]}-T{c[1]}-{c[2]}" for c in CASES])
def test_full_size_layers_sampled(name, T, regime, layers):
    wl = synth.WORKLOADS[name]
    reg = {"decode": lb.REGIME_DECODE, "prefill": lb.REGIME_PREFILL}[regime]
    entries = []
    for l in layers:
        for j, s in enumerate(wl.mats):
            entries.append((l, j, s, synth.layer_tensors(wl.wid, l, j, s.m, s.n, ranks(wl, s)),
                            synth.layer_activations(wl, l, j, s.n, T, io="bf16")))
    log(f"{name} T={T} {regime}: {len(entries)} linears")
    lins = [lb.Linear.from_numpy(s.m, s.n, p) for _, _, s, p, _ in entries]
    S = lb.Stack(lins)
    xd = [x_tensor(x) for *_, x in entries]
    ys = [torch.empty((T, s.m), dtype=torch.bfloat16, device="cuda") for _, _, s, _, _ in entries]
    S.forward(xd, ys, regime=reg, use_graph=True)
    torch.cuda.synchronize()
    first = [y.clone() for y in ys]
    for rep in range(3):                              # replays of the captured graph: bit-identical
        S.forward(xd, ys, regime=reg, use_graph=True)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(first, ys)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {rep}, entry {i} differs"
    rng = np.random.default_rng(T * 1000 + layers[0])
    for (l, j, s, p, x), y in zip(entries, ys):
        rows = np.sort(rng.choice(s.m, size=min(SAMPLE_ROWS, s.m), replace=False))
        ref = oracle.forward_rows(x_f64(x), p, s.m, s.n, rows)
        got = to_f64(y)[:, rows]
        st = assert_bf16_close(got, ref, f"{name} layer {l} {s.name} T={T}")
        log(f"  layer {l} {s.name:5s} {s.m}x{s.n} r={p[0]['rank']}: E_rms {st['erms']:.2e} "
            f"E_max/rms {st['emax_rel_rms']:.2e}")


@pytest.fixture(scope="module")
def stack70():
    """The whole Llama-2-70B-shaped stack (80 layers, 560 linears), built once
    for the tests that run it as the benchmark does; the parameters of three
    layers are kept for the oracle."""
    wl = synth.WORKLOADS["llama2-70b-0.1bpw"]
    rk = [ranks(wl, s) for s in wl.mats]
    lins, keep = [], {}
    for l in range(wl.layers):
        for j, s in enumerate(wl.mats):
            p = synth.layer_tensors(wl.wid, l, j, s.m, s.n, rk[j])
            lins.append(lb.Linear.from_numpy(s.m, s.n, p))
            if l in (0, 40, 79):
                keep[len(lins) - 1] = (l, j, s, p)
    log(f"70B stack: {len(lins)} linears")
    S = lb.Stack(lins)
    yield wl, lins, S, keep
    S.close()


def run_stack70(stack70, T, regime, seed):
    wl, lins, S, keep = stack70
    xs, ys = [], []
    for i, lin in enumerate(lins):
        l, j = divmod(i, len(wl.mats))
        xs.append(x_tensor(synth.layer_activations(wl, l, j, lin.d_in, T, io="bf16")))
        ys.append(torch.empty((T, lin.d_out), dtype=torch.bfloat16, device="cuda"))
    step = S.bind(xs, ys, regime=regime, use_graph=False)
    for _ in range(3):
        step.forward()
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    for i, (l, j, s, p) in keep.items():
        x = synth.layer_activations(wl, l, j, s.n, T, io="bf16")
        rows = np.sort(rng.choice(s.m, size=min(SAMPLE_ROWS, s.m), replace=False))
        ref = oracle.forward_rows(x_f64(x), p, s.m, s.n, rows)
        st = assert_bf16_close(to_f64(ys[i])[:, rows], ref, f"70B stack T={T} layer {l} {s.name}")
        log(f"  layer {l} {s.name:5s}: E_rms {st['erms']:.2e} E_max/rms {st['emax_rel_rms']:.2e}")
    del step


def test_full_70b_stack_decode_as_benchmarked(stack70):
    """The whole Llama-2-70B-shaped stack at batch 1, run exactly as the
    benchmark times it: one stack, bound to its buffers, three direct launches
    per step (so the work items are those of the timed configuration, not of a
    smaller stack).  Sampled output channels of three layers' linears are
    checked against the oracle."""
    run_stack70(stack70, 1, lb.REGIME_DECODE, 5601)


def test_full_70b_stack_t64_auto_as_benchmarked(stack70):
    """The whole stack at 64 tokens in the regime AUTO picks for it, as the
    benchmark's token sweep runs it (the work items and tile order are those
    of the timed 560-linear launch, not of one layer).  Sampled output
    channels of three layers' linears against the oracle."""
    log(f"70B stack T=64: AUTO picks {lb.auto_regime(stack70[1], 64)}")
    run_stack70(stack70, 64, lb.REGIME_AUTO, 6401)


def test_full_70b_layer_t64_auto_all_rows():
    """One whole layer of the Llama-2-70B-shaped stack (q, k, v, o, gate, up,
    down at 0.1 BPW) at 64 tokens, run through lb_stack_forward with the
    regime and launch form the library picks by itself (AUTO), and checked
    against the oracle on every output of every linear (the oracle rebuilds
    each W in full)."""
    wl = synth.WORKLOADS["llama2-70b-0.1bpw"]
    T, layer = 64, 11
    entries = []
    for j, s in enumerate(wl.mats):
        entries.append((s, synth.layer_tensors(wl.wid, layer, j, s.m, s.n, ranks(wl, s)),
                        synth.layer_activations(wl, layer, j, s.n, T, io="bf16")))
    lins = [lb.Linear.from_numpy(s.m, s.n, p) for s, p, _ in entries]
    S = lb.Stack(lins)
    xd = [x_tensor(x) for *_, x in entries]
    ys = [torch.empty((T, s.m), dtype=torch.bfloat16, device="cuda") for s, _, _ in entries]
    log(f"70B layer {layer}, T={T}, AUTO")
    S.forward(xd, ys)
    torch.cuda.synchronize()
    for (s, p, x), y in zip(entries, ys):
        ref = oracle.forward(x_f64(x), p, s.m, s.n)
        st = assert_bf16_close(to_f64(y), ref, f"70B layer {layer} {s.name} T={T} AUTO")
        log(f"  {s.name:5s} {s.m}x{s.n}: E_rms {st['erms']:.2e} E_max/rms {st['emax_rel_rms']:.2e}")
    S.close()


def test_full_13b_gate_fp32_tiled_t2048():
    """A Llama-2-13B-shaped gate projection (13824 x 5120, rank 1027 per path)
    with fp32 I/O at 2048 tokens: the tiled fp32 form against the oracle on
    every output, at the fp32 bound max|y - y_ref| <= 1e-5 rms(y_ref)."""
    wl = synth.WORKLOADS["llama2-13b-0.55bpw"]
    s = wl.mats[4]
    T = 2048
    p = synth.layer_tensors(wl.wid, 5, 4, s.m, s.n, ranks(wl, s))
    x = synth.activations((wl.wid, 5, 4, 77, T), T, s.n, io="fp32")
    lin = lb.Linear.from_numpy(s.m, s.n, p)
    y = lin.forward(x_tensor(x))
    torch.cuda.synchronize()
    st = assert_fp32_close(to_f64(y), oracle.forward(x_f64(x), p, s.m, s.n), "13B gate fp32 T=2048")
    log(f"13B gate fp32 T=2048: E_max/rms {st['emax_rel_rms']:.2e}")
