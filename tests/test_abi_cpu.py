"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and its host logic (rank rule, host packer, argument
validation) agrees with the oracle bit for bit."""
import ctypes as C
import os
import re
from fractions import Fraction

import numpy as np
import pytest

import binary_rank_gemm_amd as lb
import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "littlebit.h")


def header_functions(path=HEADER):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lb_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    declared = header_functions()
    assert len(declared) >= 16
    assert sorted(lb.EXPORTS) == declared
    import binary_rank_gemm_amd.probe as probe
    assert header_functions(os.path.join(ROOT, "include", "littlebit_probe.h")) == sorted(probe.EXPORTS)
    L = lb.lib()
    headers = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    assert "littlebit.h" in headers
    for h in headers:
        for name in header_functions(os.path.join(ROOT, "include", h)):
            assert hasattr(L, name), f"{h}: {name}"


def test_status_strings():
    L = lb.lib()
    for s in range(7):
        assert L.lb_status_string(s)
    assert L.lb_status_string(99) == b"unknown status"


def test_rank_rule_matches_oracle():
    for wl in synth.WORKLOADS.values():
        if wl.bpw is None:
            continue
        for s in wl.mats:
            want = oracle.rank_for_bpw(s.m, s.n, wl.bpw)
            assert lb.rank_for_bpw(s.m, s.n, wl.bpw.numerator, wl.bpw.denominator) == want
    rng = np.random.default_rng(0)
    for _ in range(300):
        m, n = (int(v) for v in rng.integers(1, 1 << 20, 2))
        num, den = int(rng.integers(1, 100)), int(rng.integers(1, 1000))
        assert lb.rank_for_bpw(m, n, num, den) == oracle.rank_for_bpw(m, n, Fraction(num, den))
    assert lb.rank_for_bpw(10, 10, 1, 1) == 3          # exact tie rounds up
    assert lb.rank_for_bpw(0, 10, 1, 1) == -1
    assert lb.rank_for_bpw(10, 10, 1, 0) == -1


@pytest.mark.parametrize("rows,rank", [(1, 1), (3, 3), (5, 31), (7, 32), (9, 33), (4, 64), (2, 65), (11, 319), (3, 1027)])
def test_host_packer_bit_exact_vs_oracle(rows, rank):
    s = synth.int8_signs((90, rows, rank), rows, rank)
    got = lb.pack_signs_host(s)
    assert got.dtype == np.uint32 and got.shape == (rows, lb.packed_words_per_row(rank))
    assert np.array_equal(got, oracle.pack_signs(s))


def test_host_packer_golden_and_errors():
    assert lb.pack_signs_host(np.array([[-1, 1, 1]], np.int8)).tolist() == [[1]]
    assert lb.pack_signs_host(np.array([[-1] * 40], np.int8)).tolist() == [[0xFFFFFFFF, 0xFF]]
    out = np.full((1, 1), 0xDEADBEEF, np.uint32)
    L = lb.lib()
    bad = np.array([[1, 0, -1]], np.int8)
    assert L.lb_pack_signs_host(bad.ctypes.data, 1, 3, out.ctypes.data) == lb._binding.INVALID_SIGN
    assert out[0, 0] == 0xDEADBEEF, "outputs must be untouched on error"
    assert b"value 0" in L.lb_last_error()
    assert L.lb_pack_signs_host(None, 1, 3, out.ctypes.data) == lb._binding.INVALID_ARGUMENT
    assert L.lb_pack_signs_host(bad.ctypes.data, 0, 3, out.ctypes.data) == lb._binding.INVALID_ARGUMENT
    assert L.lb_pack_signs_host(bad.ctypes.data, 1, -2, out.ctypes.data) == lb._binding.INVALID_ARGUMENT


def test_argument_validation_before_any_device_work():
    """Validation errors are returned before the library touches the GPU."""
    L = lb.lib()
    h = C.c_void_p()
    dummy = C.c_void_p(16)
    path = lb.LbPath(8, dummy, dummy, dummy, dummy, dummy)
    arr = (lb.LbPath * 2)(path, path)
    assert L.lb_linear_create(16, 16, arr, 3, None, C.byref(h)) == lb._binding.INVALID_ARGUMENT
    assert L.lb_linear_create(16, 16, arr, 0, None, C.byref(h)) == lb._binding.INVALID_ARGUMENT
    assert L.lb_linear_create(0, 16, arr, 1, None, C.byref(h)) == lb._binding.INVALID_ARGUMENT
    assert L.lb_linear_create(16, (1 << 20) + 1, arr, 1, None, C.byref(h)) == lb._binding.UNSUPPORTED
    assert L.lb_linear_create(16, 16, None, 1, None, C.byref(h)) == lb._binding.INVALID_ARGUMENT
    assert L.lb_linear_create(16, 16, arr, 1, None, None) == lb._binding.INVALID_ARGUMENT
    zero_rank = (lb.LbPath * 1)(lb.LbPath(0, dummy, dummy, dummy, dummy, dummy))
    assert L.lb_linear_create(16, 16, zero_rank, 1, None, C.byref(h)) == lb._binding.INVALID_ARGUMENT
    big_rank = (lb.LbPath * 1)(lb.LbPath(4097, dummy, dummy, dummy, dummy, dummy))
    assert L.lb_linear_create(16, 16, big_rank, 1, None, C.byref(h)) == lb._binding.UNSUPPORTED
    null_u = (lb.LbPath * 1)(lb.LbPath(8, None, dummy, dummy, dummy, dummy))
    assert L.lb_linear_create(16, 16, null_u, 1, None, C.byref(h)) == lb._binding.INVALID_ARGUMENT
    assert h.value is None, "no handle on error"
    # forward / stack on null handles
    assert L.lb_linear_forward(None, dummy, dummy, 1, 0, None) == lb._binding.INVALID_ARGUMENT
    assert L.lb_stack_forward(None, None, None, 1, 0, None) == lb._binding.INVALID_ARGUMENT
    assert L.lb_stack_create(None, 1, C.byref(h)) == lb._binding.INVALID_ARGUMENT
    one = (C.c_void_p * 1)(None)
    assert L.lb_stack_create(one, 0, C.byref(h)) == lb._binding.INVALID_ARGUMENT
    assert L.lb_stack_create(one, 1, C.byref(h)) == lb._binding.INVALID_ARGUMENT
    assert L.lb_linear_destroy(None) == lb._binding.OK
    assert L.lb_stack_destroy(None) == lb._binding.OK
    assert L.lb_stack_set_persistent(None, 1) == lb._binding.INVALID_ARGUMENT
    assert L.lb_stack_persistent_status(None, None, None) == lb._binding.INVALID_ARGUMENT
    assert L.lb_pack_signs(None, 1, 1, dummy, None) == lb._binding.INVALID_ARGUMENT
    assert L.lb_unpack_signs(dummy, 0, 1, dummy, None) == lb._binding.INVALID_ARGUMENT
    assert L.lb_packed_words_per_row(0) == 0 and L.lb_packed_words_per_row(32) == 1
    import binary_rank_gemm_amd.probe as probe
    assert probe._fn()(None, 16, None) == lb._binding.INVALID_ARGUMENT
    assert probe._fn()(dummy, 0, None) == lb._binding.INVALID_ARGUMENT
    assert probe._fn()(dummy, 24, None) == lb._binding.INVALID_ARGUMENT
    outs = (lb._binding.LbPathInit * 1)(lb._binding.LbPathInit(4, dummy, dummy, dummy, dummy, dummy))
    assert L.lb_init_dual_svid(None, 8, 8, outs, 1, None) == lb._binding.INVALID_ARGUMENT
    assert L.lb_init_dual_svid(dummy, 8, 8, None, 1, None) == lb._binding.INVALID_ARGUMENT
    assert L.lb_init_dual_svid(dummy, 8, 8, outs, 3, None) == lb._binding.INVALID_ARGUMENT
    bad = (lb._binding.LbPathInit * 1)(lb._binding.LbPathInit(9, dummy, dummy, dummy, dummy, dummy))
    assert L.lb_init_dual_svid(dummy, 8, 8, bad, 1, None) == lb._binding.INVALID_ARGUMENT   # rank > min(m, n)
    nul = (lb._binding.LbPathInit * 1)(lb._binding.LbPathInit(4, dummy, None, dummy, dummy, dummy))
    assert L.lb_init_dual_svid(dummy, 8, 8, nul, 1, None) == lb._binding.INVALID_ARGUMENT


def test_binding_constants_match_header():
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "littlebit.h")).read()
    regimes = dict(re.findall(r"LB_REGIME_(\w+) = (\d+)", hdr))
    assert {k: int(v) for k, v in regimes.items()} == {"AUTO": lb.REGIME_AUTO, "EXACT": lb.REGIME_EXACT,
                                                      "DECODE": lb.REGIME_DECODE, "PREFILL": lb.REGIME_PREFILL}
    dtypes = dict(re.findall(r"LB_(BF16|FP32|BF16_FP32) = (\d+)", hdr))
    assert {k: int(v) for k, v in dtypes.items()} == {"BF16": lb.BF16, "FP32": lb.FP32, "BF16_FP32": lb.BF16_FP32}
    L = lb.lib()
    out = C.c_int(-1)
    assert L.lb_auto_regime(None, 1, 4, 0, C.byref(out)) == lb._binding.INVALID_ARGUMENT
    one = (C.c_void_p * 1)(None)
    assert L.lb_auto_regime(one, 1, 4, 0, C.byref(out)) == lb._binding.INVALID_ARGUMENT
    assert L.lb_auto_regime(one, 0, 4, 0, C.byref(out)) == lb._binding.INVALID_ARGUMENT
    assert out.value == -1


def test_binding_io_types():
    """The binding's lb_dtype of an (x, y) pair; other pairs are refused."""
    torch = pytest.importorskip("torch")
    b, f = torch.zeros(1, dtype=torch.bfloat16), torch.zeros(1, dtype=torch.float32)
    io = lb._binding._io_of
    assert (io(b, b), io(f, f), io(b, f)) == (lb.BF16, lb.FP32, lb.BF16_FP32) == (0, 1, 2)
    with pytest.raises(TypeError):
        io(f, b)
    with pytest.raises(TypeError):
        io(b, torch.zeros(1, dtype=torch.float16))


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import importlib
    b = importlib.import_module("binary_rank_gemm_amd._binding")
    monkeypatch.setattr(b, "_lib", None)
    monkeypatch.setattr(b, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        b.lib()


def test_bound_stack_checks_every_entry():
    """BoundStack refuses entries whose shapes do not match their linear, or
    that are not contiguous device tensors, before any pointer reaches the
    library (which cannot see shapes)."""
    torch = pytest.importorskip("torch")
    from types import SimpleNamespace
    fake = SimpleNamespace(linears=[SimpleNamespace(d_in=8, d_out=4), SimpleNamespace(d_in=4, d_out=6)])
    bf = torch.bfloat16
    good_x = [torch.zeros(3, 8, dtype=bf), torch.zeros(3, 4, dtype=bf)]
    good_y = [torch.zeros(3, 4, dtype=bf), torch.zeros(3, 6, dtype=bf)]
    B = lb._binding.BoundStack
    with pytest.raises(ValueError, match="entry 1: x"):
        B(fake, [good_x[0], torch.zeros(3, 5, dtype=bf)], good_y, 0, None, 0)
    with pytest.raises(ValueError, match="entry 0: y"):
        B(fake, good_x, [torch.zeros(3, 5, dtype=bf), good_y[1]], 0, None, 0)
    with pytest.raises(ValueError, match="entry 1: x"):
        B(fake, [good_x[0], torch.zeros(2, 4, dtype=bf)], good_y, 0, None, 0)   # token counts differ
    with pytest.raises(ValueError, match="contiguous"):
        B(fake, [good_x[0], torch.zeros(4, 3, dtype=bf).t()], good_y, 0, None, 0)
    with pytest.raises(ValueError, match="device"):
        B(fake, good_x, good_y, 0, None, 0)   # host tensors
    with pytest.raises(ValueError, match="one x and one y"):
        B(fake, good_x[:1], good_y, 0, None, 0)
