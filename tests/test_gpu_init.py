"""Dual-SVID initialisation on the GPU (lb_init_dual_svid) against the fp64
oracle (oracle.dual_svid).

The SVD fixes each singular pair only up to a joint sign, so the sign factors
of the two sides may differ by whole columns negated in both U and V; the
effective weight, the scales and the layer's output do not.  Those are what
the tests compare.
"""
from __future__ import annotations

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


def host_paths(paths):
    """Device outputs of init_dual_svid as the oracle's path dicts."""
    out = []
    for p in paths:
        out.append(dict(rank=p["rank"], u_words=p["u"].cpu().numpy().view(np.uint32),
                        v_words=p["v"].cpu().numpy().view(np.uint32), h=p["h"].cpu().numpy().view(np.uint16),
                        g=p["g"].cpu().numpy().view(np.uint16), l=p["l"].cpu().numpy().view(np.uint16)))
    return out


def fp32_weight(key, m, n):
    rng = np.random.default_rng(key)
    return rng.standard_normal((m, n)).astype(np.float32)


@pytest.mark.parametrize("m,n,ranks", [(96, 64, [12, 12]), (64, 160, [20, 9]), (1024, 512, [64, 32]),
                                       (300, 257, [31])])
def test_dual_svid_matches_oracle(m, n, ranks):
    log(f"dual-svid m={m} n={n} ranks={ranks}")
    W = fp32_weight((m, n), m, n)
    got = host_paths(lb.init_dual_svid(torch.from_numpy(W).cuda(), ranks))
    torch.cuda.synchronize()
    ref = oracle.dual_svid.init_paths(W.astype(np.float64), ranks)
    nW = np.linalg.norm(W)
    for p in range(len(ranks)):
        # the scales: equal up to one fp16 rounding step where the fp64 values straddle a rounding point
        for k in ("h", "g", "l"):
            a, b = oracle.decode_fp16(got[p][k]), oracle.decode_fp16(ref[p][k])
            assert np.all(np.abs(a - b) <= 2.0 ** -10 * np.maximum(np.abs(b), 2.0 ** -14)), f"path {p} {k}"
            assert np.mean(a == b) > 0.98, f"path {p} {k}: too many fp16 values differ"
    Wg = oracle.reconstruct_w(got, m, n)
    Wr = oracle.reconstruct_w(ref, m, n)
    assert np.linalg.norm(Wg - Wr) <= 2e-3 * nW
    # the residual path lowers the error, as the oracle's does
    if len(ranks) == 2:
        e1 = np.linalg.norm(W - oracle.reconstruct_w(got[:1], m, n))
        assert np.linalg.norm(W - Wg) < e1


def test_dual_svid_exact_on_rank_one_magnitudes():
    # W = Hm[:, :r] diag(s) Hn[:, :r]^T: |U'| and |V'| are exactly rank 1, so
    # the only error left is the fp16 rounding of the three scales
    from scipy.linalg import hadamard
    m, n, s = 128, 64, np.array([7.0, 4.0, 3.0, 2.0, 1.25, 1.0])
    W = (hadamard(m)[:, :6] / np.sqrt(m)) @ np.diag(s) @ (hadamard(n)[:, :6] / np.sqrt(n)).T
    W32 = W.astype(np.float32)
    got = host_paths(lb.init_dual_svid(torch.from_numpy(W32).cuda(), [6]))
    Wg = oracle.reconstruct_w(got, m, n)
    assert np.abs(Wg - W32).max() <= 3 * 2.0 ** -11 * np.abs(W32).max()


def test_initialised_layer_runs_the_forward():
    m, n, ranks, T = 512, 384, [40, 40], 8
    W = fp32_weight(77, m, n)
    dev = lb.init_dual_svid(torch.from_numpy(W).cuda(), ranks)
    lin = lb.Linear(m, n, dev)
    x = synth.activations((77, 1, T), T, n)
    y = lin.forward(x_tensor(x), regime=lb.REGIME_DECODE)
    torch.cuda.synchronize()
    assert_bf16_close(to_f64(y), oracle.forward(x_f64(x), host_paths(dev), m, n), "initialised layer")
