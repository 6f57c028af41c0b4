"""Parity with the oracle for scales of every sign and the edge values a
learned real scale can take (negative, +0, -0, fp16 subnormals), in all three
regimes, one- and two-path, at shapes that reach every kernel form.

The page ("LittleBit: Ultra Low-Bit Quantization via Latent Factorization",
paper notes, section "Key design / multi-scale compensation") defines h, g and
l as learned real-valued scales, so nothing restricts their sign.  The kernels
have code that depends on it: the prefill build folds the signs of g and h
into the stored sign bits and keeps only their magnitudes; the decode V stage
multiplies g by a per-class factor.  Also here: activations whose 32-element
blocks span 2^12 in magnitude (the decode path's two-term fp8 conversion with
one power-of-two scale per block), an all-zero token, and a residual path
whose row scale is zero everywhere (a dead path).
"""
import numpy as np
import pytest

import binary_rank_gemm_amd as lb
import oracle
import synth
from lbtest import assert_bf16_close, assert_fp32_close, log, to_f64, x_f64, x_tensor

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu(gpu):
    return gpu


def signed_paths(key, m, n, ranks):
    """Seeded sign words with signed / zero / subnormal fp16 scales."""
    out = []
    for p, r in enumerate(ranks):
        out.append(dict(rank=int(r),
                        u_words=synth.sign_words((key, m, n, p, 0), m, r),
                        v_words=synth.sign_words((key, m, n, p, 1), n, r),
                        h=synth.signed_scales_fp16_bits((key, m, n, p, 2), m),
                        g=synth.signed_scales_fp16_bits((key, m, n, p, 3), n),
                        l=synth.signed_scales_fp16_bits((key, m, n, p, 4), r)))
    return out


def _assert_edge_values_present(paths):
    for p in paths:
        for name in ("h", "g"):
            b = p[name]
            v = oracle.decode_fp16(b)
            assert np.any(v < 0) and np.any(b == 0x8000) and np.any(b == 0), name
            assert np.any((np.abs(v) < 2.0 ** -14) & (v != 0)), name


# (regime, m, n, ranks, T): which kernel form each reaches is noted
CASES = [
    (lb.REGIME_DECODE, 777, 2100, [319, 5], 1),      # n % 8 != 0: V stage with plain loads; unequal ranks
    (lb.REGIME_DECODE, 1024, 8192, [46, 46], 8),     # streamed V ring (n % 8 == 0), 70B k/v shape
    (lb.REGIME_DECODE, 1024, 4096, [246, 246], 16),  # GQA k/v at twice the formula rank, two token blocks
    (lb.REGIME_DECODE, 2000, 300, [600], 2),         # one path, rank above one column group
    (lb.REGIME_DECODE, 640, 512, [600, 600], 3),     # ten 128-latent units: U stage's plain form
    (lb.REGIME_DECODE, 513, 257, [33, 31], 17),      # two decode launches (16 + 1 tokens)
    (lb.REGIME_PREFILL, 1000, 1200, [149, 102], 300),  # a full and a partial row stripe; GEMM1 tiles across paths
    (lb.REGIME_PREFILL, 1024, 4096, [246, 246], 256),  # full stripe only, GQA rank
    (lb.REGIME_PREFILL, 2000, 300, [600], 129),        # partial stripe only, one path
    (lb.REGIME_PREFILL, 513, 257, [33, 31], 140),      # element-wise A loads (n % 8 != 0)
    (lb.REGIME_EXACT, 300, 700, [37, 45], 5),
    (lb.REGIME_EXACT, 1000, 64, [1], 1),
]


@pytest.mark.parametrize("regime,m,n,ranks,T", CASES)
def test_signed_and_edge_scales(regime, m, n, ranks, T):
    log(f"signed scales regime={regime} m={m} n={n} ranks={ranks} T={T}")
    paths = signed_paths(41, m, n, ranks)
    _assert_edge_values_present(paths)
    lin = lb.Linear.from_numpy(m, n, paths)
    if regime == lb.REGIME_EXACT:
        x = synth.activations((41, T, n), T, n, io="fp32")
        y = lin.forward(x_tensor(x), regime=regime)
        torch.cuda.synchronize()
        s = assert_fp32_close(to_f64(y), oracle.forward(x_f64(x), paths, m, n), "signed scales fp32")
    else:
        x = synth.activations((41, T, n), T, n)
        y = lin.forward(x_tensor(x), regime=regime)
        torch.cuda.synchronize()
        s = assert_bf16_close(to_f64(y), oracle.forward(x_f64(x), paths, m, n), "signed scales bf16")
    log(f"  E_rms={s['erms']:.2e} E_max/rms={s['emax_rel_rms']:.2e}")


@pytest.mark.parametrize("regime,T", [(lb.REGIME_DECODE, 4), (lb.REGIME_PREFILL, 300), (lb.REGIME_EXACT, 2)])
def test_signed_scales_in_a_stack(regime, T):
    """The same edge values through a stack forward (one launch per stage over
    every entry), with the graph and direct launches agreeing bit for bit."""
    shapes = [(256, 512, [16, 16]), (1024, 300, [33, 20]), (96, 96, [5]), (1024, 4096, [246, 246])]
    io = "fp32" if regime == lb.REGIME_EXACT else "bf16"
    dt = torch.float32 if io == "fp32" else torch.bfloat16
    lins, paths, xs = [], [], []
    for i, (m, n, rk) in enumerate(shapes):
        p = signed_paths(42 + i, m, n, rk)
        paths.append(p)
        lins.append(lb.Linear.from_numpy(m, n, p))
        xs.append(synth.activations((42, i, T), T, n, io=io))
    S = lb.Stack(lins)
    xd = [x_tensor(x) for x in xs]
    runs = []
    for g in (False, True):
        ys = [torch.empty((T, m), dtype=dt, device="cuda") for m, _, _ in shapes]
        S.forward(xd, ys, regime=regime, use_graph=g)
        torch.cuda.synchronize()
        runs.append(ys)
    close = assert_fp32_close if io == "fp32" else assert_bf16_close
    bits = torch.int32 if io == "fp32" else torch.int16
    for i, (m, n, _) in enumerate(shapes):
        close(to_f64(runs[0][i]), oracle.forward(x_f64(xs[i]), paths[i], m, n), f"stack entry {i}")
        assert torch.equal(runs[0][i].view(bits), runs[1][i].view(bits)), f"graph != direct, entry {i}"
    S.close()


@pytest.mark.parametrize("regime,T", [(lb.REGIME_DECODE, 3), (lb.REGIME_DECODE, 16), (lb.REGIME_PREFILL, 300),
                                      (lb.REGIME_EXACT, 3)])
def test_dead_residual_path(regime, T):
    """A residual path whose row scale h is zero everywhere adds nothing: the
    two-path layer matches the oracle and equals the primary path alone; in
    the prefill GEMMs the extra latents only add zero products, so the result
    is bit-identical to the one-path layer."""
    m, n = 700, 1024
    pri = signed_paths(43, m, n, [64])[0]
    res = signed_paths(44, m, n, [40])[0]
    res = dict(res, h=np.zeros(m, np.uint16))
    io = "fp32" if regime == lb.REGIME_EXACT else "bf16"
    x = synth.activations((43, T, n), T, n, io=io)
    two = lb.Linear.from_numpy(m, n, [pri, res])
    one = lb.Linear.from_numpy(m, n, [pri])
    y2 = two.forward(x_tensor(x), regime=regime)
    y1 = one.forward(x_tensor(x), regime=regime)
    torch.cuda.synchronize()
    ref = oracle.forward(x_f64(x), [pri, res], m, n)
    assert np.array_equal(ref, oracle.forward(x_f64(x), [pri], m, n))
    close = assert_fp32_close if io == "fp32" else assert_bf16_close
    close(to_f64(y2), ref, "dead residual, two paths")
    close(to_f64(y1), ref, "dead residual, one path")
    if regime == lb.REGIME_PREFILL:
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("m,n,ranks,T", [(1000, 4096, [102, 102], 1), (513, 2100, [46, 30], 5),
                                         (1024, 8192, [205, 205], 16)])
def test_decode_wide_range_blocks(m, n, ranks, T):
    """Decode with activations whose 32-element blocks span 2^12 in magnitude,
    so each block's power-of-two scale serves values far below its largest
    (the second fp8 term carries their bits).  Scales are the usual positive
    ones and signed ones."""
    x = synth.wide_range_activations((45, T, n), T, n, octaves=12)
    xv = x_f64(x)
    spans = []
    for t in range(T):
        blk = np.abs(xv[t, : n // 32 * 32].reshape(-1, 32))
        nz = np.where(blk > 0, blk, np.inf).min(axis=1)
        spans.append(np.max(blk.max(axis=1) / nz))
    assert max(spans) >= 2.0 ** 12
    for kind, paths in (("lognormal", synth.layer_tensors(45, 1, 0, m, n, ranks)), ("signed", signed_paths(45, m, n, ranks))):
        lin = lb.Linear.from_numpy(m, n, paths)
        y = lin.forward(x_tensor(x), regime=lb.REGIME_DECODE)
        torch.cuda.synchronize()
        s = assert_bf16_close(to_f64(y), oracle.forward(xv, paths, m, n), f"wide-range {kind}")
        log(f"wide range {kind} m={m} n={n} T={T}: E_rms={s['erms']:.2e} E_max/rms={s['emax_rel_rms']:.2e}")


@pytest.mark.parametrize("regime", [lb.REGIME_DECODE, lb.REGIME_PREFILL, lb.REGIME_EXACT])
def test_zero_token_rows(regime):
    """Tokens whose activations are all zero give exactly zero outputs; the
    other tokens are unaffected."""
    m, n, T = 300, 520, 140 if regime == lb.REGIME_PREFILL else 5
    paths = signed_paths(46, m, n, [40, 24])
    io = "fp32" if regime == lb.REGIME_EXACT else "bf16"
    x = synth.activations((46, T, n), T, n, io=io)
    x[1] = 0
    x[T - 1] = 0
    lin = lb.Linear.from_numpy(m, n, paths)
    y = to_f64(lin.forward(x_tensor(x), regime=regime))
    torch.cuda.synchronize()
    assert np.all(y[1] == 0) and np.all(y[T - 1] == 0)
    close = assert_fp32_close if io == "fp32" else assert_bf16_close
    close(y, oracle.forward(x_f64(x), paths, m, n), "zero tokens")
