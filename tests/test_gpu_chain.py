"""The persistent chained decode (lb_stack_set_persistent): a chained stack's
levels in one cooperative launch, checked bit for bit against the same stack
run as launches per level, and against the oracle.

The layer is the factorised form of the paper notes "LittleBit: Ultra Low-Bit
Quantization via Latent Factorization" (section "Key design"), both paths
(section "Residual compensation"); the chain is a model's linears in their real
order (experiments section: Llama-2 70B shapes).
"""
from fractions import Fraction

import numpy as np
import pytest

import binary_rank_gemm_amd as lb
import oracle
import synth
from lbtest import assert_bf16_close, log, to_f64, x_f64, x_tensor

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu(gpu):
    return gpu


# per layer: q, k, v read the layer input; o reads q's output; gate and up
# read o's; down reads gate's; the next layer reads down's.  (m, n, ranks)
D, F = 256, 704
LAYER = [(D, D, [16, 12]), (D // 4, D, [9, 9]), (D // 4, D, [9, 9]), (D, D, [16, 12]),
         (F, D, [33, 20]), (F, D, [33, 20]), (D, F, [33, 20])]


def model_order_inputs(x0, ys, layers):
    xs = []
    for l in range(layers):
        b = 7 * l
        inp = x0 if l == 0 else ys[b - 1]
        xs += [inp, inp, inp, ys[b], ys[b + 3], ys[b + 3], ys[b + 4]]
    return xs


def run(S, xs, ys, **kw):
    for y in ys:
        y.zero_()
    S.forward(xs, ys, **kw)
    torch.cuda.synchronize()
    return [y.clone() for y in ys]


def same_bits(a, b, what):
    for i, (u, v) in enumerate(zip(a, b)):
        assert torch.equal(u.view(torch.int16), v.view(torch.int16)), f"{what}: entry {i} differs"


def stacks(lins):
    """The persistent launch (mode 1) and its plans run as level launches
    (mode 2, the bit-for-bit reference), as two stacks over the same linears."""
    S1, S2 = lb.Stack(lins), lb.Stack(lins)
    S1.set_persistent(1)
    S2.set_persistent(2)
    return S1, S2


@pytest.mark.parametrize("T", [1, 2, 3, 8, 16])
def test_persistent_chain_equals_level_launches(T):
    """Three layers in model order (12 levels), one new input per call: the
    persistent launch gives the bits of its plans run as level launches on
    every call (the launch epoch advances; a hand-over that read data of the
    previous call would differ), reports itself active and not aborted, and
    every link matches the oracle applied to the input it read -- as do the
    stack's own level launches (mode 0, planned for the whole GPU)."""
    layers = 3
    shapes = LAYER * layers
    paths = [synth.layer_tensors(41, i, 0, m, n, r) for i, (m, n, r) in enumerate(shapes)]
    lins = [lb.Linear.from_numpy(m, n, p) for (m, n, _), p in zip(shapes, paths)]
    x0 = x_tensor(synth.activations((41, 99, T), T, D))
    ys = [torch.empty((T, m), dtype=torch.bfloat16, device="cuda") for m, _, _ in shapes]
    xs = model_order_inputs(x0, ys, layers)
    S1, S2 = stacks(lins)
    log(f"persistent chain T={T}: {len(shapes)} linears, {4 * layers} levels")
    kw = dict(regime=lb.REGIME_DECODE, use_graph=False)
    for call in range(3):
        x0.copy_(x_tensor(synth.activations((41, 100 + call, T), T, D)))
        ref = run(S2, xs, ys, **kw)
        got = run(S1, xs, ys, **kw)
        st = S1.persistent_status()
        assert st["active"] and not st["aborted"], st
        same_bits(ref, got, f"call {call}")
    for i, (m, n, _) in enumerate(shapes):
        assert_bf16_close(to_f64(ys[i]), oracle.forward(to_f64(xs[i]), paths[i], m, n), f"T={T} link {i}")
    # mode 0 (the default): the stack's usual plans, level launches, within the same bound
    S0 = lb.Stack(lins)
    run(S0, xs, ys, **kw)
    assert not S0.persistent_status()["active"]
    for i, (m, n, _) in enumerate(shapes):
        assert_bf16_close(to_f64(ys[i]), oracle.forward(to_f64(xs[i]), paths[i], m, n), f"T={T} mode 0 link {i}")
    # lb_stack_forward (AUTO, no graph) takes the persistent launch once asked for, at these few tokens
    if T <= 2:
        ref = run(S2, xs, ys, **kw)
        got = run(S1, xs, ys)
        assert S1.persistent_status()["active"]
        same_bits(ref, got, "lb_stack_forward")
    # a captured graph holds the persistent plans' level launches: the same bits again
    ref = run(S1, xs, ys, **kw)
    got = run(S1, xs, ys, regime=lb.REGIME_DECODE, use_graph=True)
    same_bits(ref, got, "graph")
    for S in (S0, S1, S2):
        S.close()


def test_persistent_chain_falls_back_when_an_entry_does_not_fit():
    """An entry whose rows of x cannot be read with 16-byte loads (d_in not a
    multiple of 8) keeps the stack on level launches."""
    shapes = [(96, 100, [20, 7]), (64, 96, [12, 12]), (72, 64, [9, 30])]
    T = 2
    paths = [synth.layer_tensors(42, i, 0, m, n, r) for i, (m, n, r) in enumerate(shapes)]
    lins = [lb.Linear.from_numpy(m, n, p) for (m, n, _), p in zip(shapes, paths)]
    x0 = x_tensor(synth.activations((42, 99, T), T, 100))
    ys = [torch.empty((T, m), dtype=torch.bfloat16, device="cuda") for m, _, _ in shapes]
    xs = [x0, ys[0], ys[1]]
    S = lb.Stack(lins)
    run(S, xs, ys, regime=lb.REGIME_DECODE, use_graph=False)
    assert not S.persistent_status()["active"]
    for i, (m, n, _) in enumerate(shapes):
        assert_bf16_close(to_f64(ys[i]), oracle.forward(to_f64(xs[i]), paths[i], m, n), f"fallback link {i}")
    S.close()


def test_persistent_chain_abort_path(monkeypatch):
    """Failure handling of the persistent launch, forced from the host: with
    LITTLEBIT_CHAIN_STALL=1 at planning, the first barrier of every launch
    waits for one arrival more than take part, so its bounded wait times out
    (one second) and every participant leaves.  The stack then reports the
    launch aborted, no output is written (the U items of the first level come
    after that barrier), and a second launch of the plan leaves at once.
    Planned again without the variable, the kernel runs normally: the bits of
    its plans run as level launches."""
    shapes = LAYER                                   # one layer: 4 levels
    T = 1
    paths = [synth.layer_tensors(43, i, 0, m, n, r) for i, (m, n, r) in enumerate(shapes)]
    lins = [lb.Linear.from_numpy(m, n, p) for (m, n, _), p in zip(shapes, paths)]
    x0 = x_tensor(synth.activations((43, 99, T), T, D))
    ys = [torch.empty((T, m), dtype=torch.bfloat16, device="cuda") for m, _, _ in shapes]
    xs = model_order_inputs(x0, ys, 1)
    S1, S2 = stacks(lins)
    kw = dict(regime=lb.REGIME_DECODE, use_graph=False)
    monkeypatch.setenv("LITTLEBIT_CHAIN_STALL", "1")
    log("persistent chain abort path: two stalled launches")
    for call in range(2):
        for y in ys:
            y.fill_(7.0)
        S1.forward(xs, ys, **kw)
        torch.cuda.synchronize()
        st = S1.persistent_status()
        assert st["active"] and st["aborted"], (call, st)
        for i, y in enumerate(ys):
            assert bool((y == 7.0).all()), f"call {call}: entry {i} was written by an aborted launch"
    monkeypatch.delenv("LITTLEBIT_CHAIN_STALL")
    S1.set_persistent(0)
    S1.set_persistent(1)                             # plans again at the next forward
    ref = run(S2, xs, ys, **kw)
    got = run(S1, xs, ys, **kw)
    st = S1.persistent_status()
    assert st["active"] and not st["aborted"], st
    same_bits(ref, got, "after planning again")
    for i, (m, n, _) in enumerate(shapes):
        assert_bf16_close(to_f64(ys[i]), oracle.forward(to_f64(xs[i]), paths[i], m, n), f"link {i}")
    S1.close()
    S2.close()


def ranks70(s):
    r = oracle.rank_for_bpw(s.m, s.n, Fraction(1, 10), s.rank_mult)
    return [r, r]


def test_persistent_chain_70b_layers_and_a_wide_level():
    """Real Llama-2-70B shapes (0.1 sign bits per weight): two layers in model
    order, preceded by a level of eight gate-shaped linears (more V and U work
    items than the persistent grid has workgroups, so workgroups take several
    items per phase), at one token: bit for bit the level launches, and
    sampled rows of every link against the oracle."""
    wl = synth.WORKLOADS["llama2-70b-0.1bpw"]
    T = 1
    gate = wl.mats[4]
    specs, paths = [], []
    for k in range(8):                               # the wide first level: gates of layers 10..17
        specs.append(gate)
        paths.append(synth.layer_tensors(wl.wid, 10 + k, 4, gate.m, gate.n, ranks70(gate)))
    for l in range(2):
        for j, s in enumerate(wl.mats):
            specs.append(s)
            paths.append(synth.layer_tensors(wl.wid, l, j, s.m, s.n, ranks70(s)))
    lins = [lb.Linear.from_numpy(s.m, s.n, p) for s, p in zip(specs, paths)]
    x0 = x_tensor(synth.activations((5, 77, T), T, 8192))
    ys = [torch.empty((T, s.m), dtype=torch.bfloat16, device="cuda") for s in specs]
    # the gates read x0, as do layer 0's q, k and v: one wide first level of 11 entries
    xs = [x0] * 8
    for l in range(2):
        b = 8 + 7 * l
        inp = x0 if l == 0 else ys[b - 1]
        xs += [inp, inp, inp, ys[b], ys[b + 3], ys[b + 3], ys[b + 4]]
    S1, S2 = stacks(lins)
    log(f"70B chain: {len(specs)} linears")
    kw = dict(regime=lb.REGIME_DECODE, use_graph=False)
    for call in range(2):
        x0.copy_(x_tensor(synth.activations((5, 78 + call, T), T, 8192)))
        ref = run(S2, xs, ys, **kw)
        got = run(S1, xs, ys, **kw)
        st = S1.persistent_status()
        assert st["active"] and not st["aborted"], st
        same_bits(ref, got, f"70B call {call}")
    rng = np.random.default_rng(70)
    for i, (s, p) in enumerate(zip(specs, paths)):
        rows = np.sort(rng.choice(s.m, size=min(32, s.m), replace=False))
        ref_rows = oracle.forward_rows(to_f64(xs[i]), p, s.m, s.n, rows)
        assert_bf16_close(to_f64(ys[i])[:, rows], ref_rows, f"70B link {i} {s.name}")
    S1.close()
    S2.close()
