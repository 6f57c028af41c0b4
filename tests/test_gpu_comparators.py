"""The benchmark's decompress-then-compute comparator computes the same layer:
W rebuilt from the layer's own packed signs and fp16 scales, then x W^T,
against the oracle (pages: kongchang.com/en "Sub-1-Bit LLM Compression ...",
section "Issues That Warrant Caution", on unpacking the factors before the
matrix product)."""
import numpy as np
import pytest

import bench
import oracle
import synth
from lbtest import assert_bf16_close, log, to_f64, x_f64, x_tensor

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu(gpu):
    return gpu


@pytest.mark.parametrize("m,n,ranks,T", [(300, 520, [37, 45], 3), (1024, 4096, [102, 102], 1), (96, 200, [33], 5)])
def test_decompress_then_compute_matches_oracle(m, n, ranks, T):
    paths = synth.layer_tensors(61, m, n, m, n, ranks)
    x = synth.activations((61, T, n), T, n)
    dev = bench.upload_paths(paths, torch)
    W = bench.decompress_weight(dev, torch)
    torch.cuda.synchronize()
    assert W.shape == (m, n) and W.dtype == torch.bfloat16
    # the rebuilt weight itself, element by element (bf16 products of fp16
    # scales and a bf16 rounding of the sum: relative to the weight's rms)
    Wref = oracle.reconstruct_w(paths, m, n)
    werr = np.abs(to_f64(W) - Wref)
    assert np.max(werr) <= 2e-2 * np.sqrt(np.mean(Wref ** 2)) + 2.0 ** -7 * np.max(np.abs(Wref))
    y = bench.decompress_then_compute(dev, x_tensor(x), torch)
    torch.cuda.synchronize()
    s = assert_bf16_close(to_f64(y), oracle.forward(x_f64(x), paths, m, n), "decompress-then-compute")
    log(f"decompress-then-compute {m}x{n} r={ranks} T={T}: E_rms {s['erms']:.2e}")


def test_unpack_signs_torch_matches_oracle():
    words = synth.sign_words((62, 1), 37, 70)
    got = bench.unpack_signs_torch(torch.from_numpy(words.view(np.int32)).cuda(), 70, torch)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().astype(np.int8), oracle.unpack_signs(words, 37, 70))
