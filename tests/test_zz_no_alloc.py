"""lb_linear_forward_noalloc through the C ABI: the same results as
lb_linear_forward_ex with the regime it runs (decode for bf16 x, exact for
fp32 I/O), bit for bit, on calls in a row that reuse the fixed scratch, the
second with a smaller input; against the oracle; sizes beyond the scratch are
refused with the output untouched."""
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


def noalloc(lin, x, y):
    """The entry point itself, called through ctypes."""
    st = torch.cuda.current_stream().cuda_stream
    return lb.lib().lb_linear_forward_noalloc(lin.handle, x.data_ptr(), y.data_ptr(), x.shape[0],
                                             lb._binding._io_of(x, y), st)


def layer(key, m, n, ranks):
    paths = synth.layer_tensors(key, m, n, m, n, ranks)
    return paths, lb.Linear.from_numpy(m, n, paths)


# (m, n, ranks, T) per call: the second call of each case is smaller
CASES = {
    "bf16": [(1000, 1200, [149, 102], 9), (300, 520, [37, 45], 3), (1000, 1200, [149, 102], 1)],
    "bf16_fp32": [(1024, 4096, [246, 246], 16), (640, 384, [20], 5)],
    "fp32": [(1000, 1200, [149, 102], 40), (777, 2100, [319, 5], 6), (300, 700, [37, 45], 2)],
    "long": [(4096, 1024, [46, 46], 40), (513, 257, [33, 31], 17)],   # several 16-token launches
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_noalloc_matches_forward_ex(case):
    for m, n, ranks, T in CASES[case]:
        log(f"noalloc {case}: m={m} n={n} ranks={ranks} T={T}")
        paths, lin = layer(71, m, n, ranks)
        io_x = "fp32" if case == "fp32" else "bf16"
        x_np = synth.activations((71, m, T), T, n, io=io_x)
        x = x_tensor(x_np)
        ydt = torch.bfloat16 if case in ("bf16", "long") else torch.float32
        regime = lb.REGIME_EXACT if case == "fp32" else lb.REGIME_DECODE
        y_ref_lib = lin.forward(x, regime=regime, out_dtype=ydt)
        y = torch.full((T, m), 7.0, dtype=ydt, device="cuda")
        assert noalloc(lin, x, y) == lb._binding.OK, lb.lib().lb_last_error().decode()
        torch.cuda.synchronize()
        bits = torch.int16 if ydt == torch.bfloat16 else torch.int32
        assert torch.equal(y.view(bits), y_ref_lib.view(bits)), "no-allocation forward differs from lb_linear_forward_ex"
        ref = oracle.forward(x_f64(x_np), paths, m, n)
        if case == "fp32":
            assert_fp32_close(to_f64(y), ref, "noalloc fp32")
        else:
            assert_bf16_close(to_f64(y), ref, f"noalloc {case}")
        lin.close()


def test_noalloc_refuses_sizes_beyond_the_scratch():
    """fp32 tokens whose latent sums need more than the 8 MiB scratch are
    refused before any launch; y keeps its contents; a smaller call on the
    same linear then runs."""
    m, n, ranks = 512, 512, [1024, 1024]
    paths, lin = layer(72, m, n, ranks)
    T = 1100   # 2 paths x 1100 tokens x 1024 latents x 4 bytes > 8 MiB
    x = torch.zeros((T, n), dtype=torch.float32, device="cuda")
    y = torch.full((T, m), 3.0, dtype=torch.float32, device="cuda")
    assert noalloc(lin, x, y) == lb._binding.UNSUPPORTED
    assert b"scratch" in lb.lib().lb_last_error()
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)
    T = 4
    x_np = synth.activations((72, T), T, n, io="fp32")
    y = torch.empty((T, m), dtype=torch.float32, device="cuda")
    assert noalloc(lin, x_tensor(x_np), y) == lb._binding.OK
    torch.cuda.synchronize()
    assert_fp32_close(to_f64(y), oracle.forward(x_f64(x_np), paths, m, n), "noalloc after refusal")
    lin.close()


def test_noalloc_argument_errors():
    m, n = 64, 128
    _, lin = layer(73, m, n, [8, 8])
    x = torch.zeros((4, n), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((4, m), dtype=torch.bfloat16, device="cuda")
    L = lb.lib()
    st = torch.cuda.current_stream().cuda_stream
    assert L.lb_linear_forward_noalloc(lin.handle, x.data_ptr() + 2, y.data_ptr(), 4, lb.BF16, st) == \
        lb._binding.ALIGNMENT
    assert L.lb_linear_forward_noalloc(lin.handle, x.data_ptr(), y.data_ptr(), 0, lb.BF16, st) == \
        lb._binding.INVALID_ARGUMENT
    assert L.lb_linear_forward_noalloc(None, x.data_ptr(), y.data_ptr(), 4, lb.BF16, st) == \
        lb._binding.INVALID_ARGUMENT
    assert L.lb_linear_forward_noalloc(lin.handle, x.data_ptr(), y.data_ptr(), 4, 7, st) == \
        lb._binding.INVALID_ARGUMENT
    lin.close()
