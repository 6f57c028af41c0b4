"""Parity of the HIP library (through its C ABI) with the CPU oracle.

Exact probes use inputs for which every intermediate is exactly representable
(small integers, one-hot activations, unit or power-of-two scales), so the GPU
must match the oracle bit for bit; float parity uses seeded synthetic layers
and the acceptance criteria in lbtest.py.
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


def f16bits(v):
    return np.asarray(v, np.float16).view(np.uint16)


def build(m, n, paths):
    return lb.Linear.from_numpy(m, n, paths)


def seeded_paths(key, m, n, ranks):
    return synth.layer_tensors(key[0], key[1], key[2], m, n, ranks)


# ----------------------------------------------------------------------------
# packing
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("rows,rank", [(1, 1), (17, 31), (100, 32), (33, 33), (1000, 319), (64, 1027)])
def test_pack_signs_device_bit_exact(rows, rank):
    log(f"pack rows={rows} rank={rank}")
    s = synth.int8_signs((11, rows, rank), rows, rank)
    d = torch.from_numpy(s).cuda()
    w = lb.pack_signs(d)
    torch.cuda.synchronize()
    got = w.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, oracle.pack_signs(s))
    assert np.array_equal(got, lb.pack_signs_host(s))
    back = lb.unpack_signs(w, rank)
    torch.cuda.synchronize()
    assert np.array_equal(back.cpu().numpy(), s)


def test_pack_signs_device_rejects_bad_values_untouched():
    s = np.ones((4, 40), np.int8)
    s[2, 17] = 0
    d = torch.from_numpy(s).cuda()
    out = torch.full((4, 2), 12345, dtype=torch.int32, device="cuda")
    with pytest.raises(lb.LittleBitError) as ei:
        lb.lib()
        st = lb._binding._check(lb.lib().lb_pack_signs(d.data_ptr(), 4, 40, out.data_ptr(),
                                                         torch.cuda.current_stream().cuda_stream))
    assert ei.value.status == lb._binding.INVALID_SIGN
    torch.cuda.synchronize()
    assert torch.all(out == 12345)


# ----------------------------------------------------------------------------
# fp32 exact path
# ----------------------------------------------------------------------------

def test_exact_fp32_single_512_workload():
    wl = synth.WORKLOADS["single-512"]
    m, n, r, T = 512, 512, wl.fixed_rank, wl.tokens[0]
    log(f"exact fp32 single-512 T={T}")
    paths = seeded_paths((wl.wid, 0, 0), m, n, [r, r])
    x = synth.layer_activations(wl, 0, 0, n, T)
    lin = build(m, n, paths)
    y = lin.forward(x_tensor(x))
    torch.cuda.synchronize()
    s = assert_fp32_close(to_f64(y), oracle.forward(x_f64(x), paths, m, n), "single-512 fp32")
    log(f"  E_max/rms = {s['emax_rel_rms']:.2e}")


def test_exact_fp32_integer_probe_bit_exact():
    """x in {-2..2}, scales in {1, 2}: every partial sum is an integer < 2^22, exact in fp32."""
    rng = np.random.default_rng(21)
    m, n, ranks, T = 300, 2048, [64, 40], 3
    paths = []
    for p, r in enumerate(ranks):
        paths.append(dict(rank=r, u_words=synth.sign_words((21, p, 0), m, r), v_words=synth.sign_words((21, p, 1), n, r),
                          h=f16bits(rng.choice([1.0, 2.0], m)), g=f16bits(rng.choice([1.0, 2.0], n)),
                          l=f16bits(rng.choice([1.0, 2.0], r))))
    x = rng.integers(-2, 3, size=(T, n)).astype(np.float32)
    y_ref = oracle.forward(x.astype(np.float64), paths, m, n)
    assert np.max(np.abs(y_ref)) < 2 ** 22
    lin = build(m, n, paths)
    y = lin.forward(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(y), y_ref)


@pytest.mark.parametrize("m,n,ranks,T", [(300, 700, [37, 45], 5), (1000, 64, [1], 1), (33, 4100, [130, 7], 2)])
def test_exact_fp32_ragged(m, n, ranks, T):
    log(f"exact fp32 m={m} n={n} ranks={ranks} T={T}")
    paths = seeded_paths((22, m, n), m, n, ranks)
    x = synth.activations((22, T, n), T, n, io="fp32")
    y = build(m, n, paths).forward(x_tensor(x))
    torch.cuda.synchronize()
    assert_fp32_close(to_f64(y), oracle.forward(x_f64(x), paths, m, n), "ragged fp32")


@pytest.mark.parametrize("m,n,ranks,T", [(300, 700, [37, 45], 40), (1000, 1200, [149, 102], 130),
                                         (513, 257, [33, 31], 200), (96, 4100, [1], 16), (4096, 1024, [246, 246], 300)])
def test_exact_fp32_tiled_form(m, n, ranks, T):
    """fp32 I/O with 16 tokens or more runs the tiled fp32 matrix-core form:
    ragged tokens (128-row tiles), ragged n (n % 4 != 0: element-wise loads),
    ranks not a multiple of 32, one path."""
    log(f"exact fp32 tiled m={m} n={n} ranks={ranks} T={T}")
    paths = seeded_paths((36, m, n), m, n, ranks)
    x = synth.activations((36, T, n), T, n, io="fp32")
    y = build(m, n, paths).forward(x_tensor(x))
    torch.cuda.synchronize()
    s = assert_fp32_close(to_f64(y), oracle.forward(x_f64(x), paths, m, n), "tiled fp32")
    log(f"  E_max/rms = {s['emax_rel_rms']:.2e}")


def test_exact_fp32_tiled_integer_probe_bit_exact():
    """The tiled form with integer inputs whose every partial sum stays below
    2^22: exact in fp32 whatever the order, so equal to the oracle bit for bit."""
    rng = np.random.default_rng(37)
    m, n, ranks, T = 300, 2048, [64, 40], 150
    paths = []
    for p, r in enumerate(ranks):
        paths.append(dict(rank=r, u_words=synth.sign_words((37, p, 0), m, r), v_words=synth.sign_words((37, p, 1), n, r),
                          h=f16bits(rng.choice([1.0, -2.0], m)), g=f16bits(rng.choice([-1.0, 2.0], n)),
                          l=f16bits(rng.choice([1.0, 2.0], r))))
    x = rng.integers(-2, 3, size=(T, n)).astype(np.float32)
    y_ref = oracle.forward(x.astype(np.float64), paths, m, n)
    assert np.max(np.abs(y_ref)) < 2 ** 22
    y = build(m, n, paths).forward(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(y), y_ref)


# ----------------------------------------------------------------------------
# decode path (bf16)
# ----------------------------------------------------------------------------

def onehot_x(n, ks, vals=None):
    x = np.zeros((len(ks), n), np.float32)
    for t, k in enumerate(ks):
        x[t, k] = 1.0 if vals is None else vals[t]
    return synth.bf16_bits_from_f32(x)


@pytest.mark.parametrize("regime", [lb.REGIME_DECODE, lb.REGIME_EXACT, lb.REGIME_PREFILL])
def test_identity_probe_bit_exact(regime):
    """Unit scales, x = e_k: y = row k of V_p contracted with U_p, summed over
    paths -- integers of magnitude <= r1 + r2 <= 256, exact in bf16."""
    m, n, ranks = 333, 1000, [100, 80]
    ones = lambda k: f16bits(np.ones(k))
    paths = [dict(rank=r, u_words=synth.sign_words((23, p, 0), m, r), v_words=synth.sign_words((23, p, 1), n, r),
                  h=ones(m), g=ones(n), l=ones(r)) for p, r in enumerate(ranks)]
    ks = [0, 1, 127, 128, 500, 998, 999, 640]
    x = onehot_x(n, ks)
    log(f"identity probe regime={regime}")
    y = build(m, n, paths).forward(x_tensor(x), regime=regime)
    torch.cuda.synchronize()
    y_ref = oracle.forward(x_f64(x), paths, m, n)
    assert np.array_equal(to_f64(y), y_ref)


@pytest.mark.parametrize("regime", [lb.REGIME_DECODE, lb.REGIME_PREFILL])
def test_power_of_two_scales_bit_exact(regime):
    """Scales in {1, 2} and x in {+-1, +-2} one-hot: |y| <= 256, every step exact."""
    rng = np.random.default_rng(24)
    m, n, ranks = 70, 4000, [10, 6]
    paths = []
    for p, r in enumerate(ranks):
        paths.append(dict(rank=r, u_words=synth.sign_words((24, p, 0), m, r), v_words=synth.sign_words((24, p, 1), n, r),
                          h=f16bits(rng.choice([1.0, 2.0], m)), g=f16bits(rng.choice([1.0, 2.0], n)),
                          l=f16bits(rng.choice([1.0, 2.0], r))))
    ks = [5, 3999, 2048, 77, 1000, 129, 130, 3000, 12, 13, 14]
    x = onehot_x(n, ks, vals=[1, -1, 2, -2, 1, 1, -1, 2, -2, 1, 2])
    y_ref = oracle.forward(x_f64(x), paths, m, n)
    assert np.max(np.abs(y_ref)) <= 256
    y = build(m, n, paths).forward(x_tensor(x), regime=regime)
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(y), y_ref)


def test_prefill_identity_probe_many_tokens_bit_exact():
    """x = I_n (T = n = 640 tokens, spans three 256-row tiles): y = sum_p U_p V_p^T, exact."""
    m, n, ranks = 700, 640, [90, 70]
    ones = lambda k: f16bits(np.ones(k))
    paths = [dict(rank=r, u_words=synth.sign_words((29, p, 0), m, r), v_words=synth.sign_words((29, p, 1), n, r),
                  h=ones(m), g=ones(n), l=ones(r)) for p, r in enumerate(ranks)]
    x = synth.bf16_bits_from_f32(np.eye(n, dtype=np.float32))
    y = build(m, n, paths).forward(x_tensor(x), regime=lb.REGIME_PREFILL)
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(y), oracle.forward(x_f64(x), paths, m, n))


def test_prefill_k_parts_probe_bit_exact():
    """48 tokens, K = 9000 (141 K blocks: GEMM1 in two K parts).  Each token
    row holds two ones, one in each part's K range; with unit scales every sum
    is a small integer, so the parts' fp32 sums and the bf16 results are exact."""
    m, n, ranks, T = 300, 9000, [40, 30], 48
    ones = lambda k: f16bits(np.ones(k))
    paths = [dict(rank=r, u_words=synth.sign_words((35, p, 0), m, r), v_words=synth.sign_words((35, p, 1), n, r),
                  h=ones(m), g=ones(n), l=ones(r)) for p, r in enumerate(ranks)]
    xf = np.zeros((T, n), np.float32)
    split = 71 * 64                                   # first K element of the second part
    for t in range(T):
        xf[t, (t * 97) % split] = 1.0
        xf[t, split + (t * 131) % (n - split)] = 1.0
    x = synth.bf16_bits_from_f32(xf)
    y = build(m, n, paths).forward(x_tensor(x), regime=lb.REGIME_PREFILL)
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(y), oracle.forward(x_f64(x), paths, m, n))


@pytest.mark.parametrize("m,n,ranks", [(300, 320, [20, 40]), (640, 384, [270, 20]), (1000, 320, [149, 102]),
                                       (300, 100, [20, 40]), (640, 128, [149, 102])])
def test_prefill_identity_probe_narrow_tiles_bit_exact(m, n, ranks):
    """x = I_n with unit scales through the prefill GEMMs at shapes whose last
    column tiles are 128 or 64 wide (GEMM1 N = the concatenated padded rank,
    GEMM2 N = m), some with a wave's columns in both paths: y = sum_p U_p V_p^T
    exactly."""
    ones = lambda k: f16bits(np.ones(k))
    paths = [dict(rank=r, u_words=synth.sign_words((35, p, 0), m, r), v_words=synth.sign_words((35, p, 1), n, r),
                  h=ones(m), g=ones(n), l=ones(r)) for p, r in enumerate(ranks)]
    x = synth.bf16_bits_from_f32(np.eye(n, dtype=np.float32))
    y = build(m, n, paths).forward(x_tensor(x), regime=lb.REGIME_PREFILL)
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(y), oracle.forward(x_f64(x), paths, m, n))


DECODE_SHAPES = [
    # m, n, ranks, T, outliers
    (512, 512, [16, 16], 4, 0.0),        # the single-512 shape in bf16
    (300, 700, [37, 45], 1, 0.0),        # ragged everything
    (1000, 1200, [149, 102], 3, 0.0),
    (4096, 4096, [102, 102], 1, 0.01),   # Llama-2-7B q/k/v/o at 0.1 BPW with outlier channels
    (1024, 8192, [46, 46], 8, 0.0),      # Llama-2-70B k/v at 0.1 BPW
    (777, 2100, [319, 5], 9, 0.0),       # two token blocks, unequal ranks
    (640, 384, [1, 1], 16, 0.0),
    (513, 257, [33, 31], 17, 0.0),       # 17 tokens: two launches of the decode kernel
    (2000, 300, [600], 2, 0.0),          # single path, rank above one column group
    (1536, 2048, [77, 51], 2, 0.01),     # two tokens with 16-byte x rows (the streamed V form's four-row A image)
    (456, 440, [400, 300], 13, 0.0),     # 7 units at 16-token launches: the wide U launch, ragged quads
    (520, 512, [500, 480], 16, 0.0),     # 8 units: the wide U launch
    (600, 560, [520, 480], 12, 0.0),     # 9 units: the plain U form
]


@pytest.mark.parametrize("m,n,ranks,T,outl", DECODE_SHAPES)
def test_decode_parity(m, n, ranks, T, outl):
    log(f"decode m={m} n={n} ranks={ranks} T={T}")
    paths = seeded_paths((25, m, n), m, n, ranks)
    x = synth.activations((25, T, n), T, n, outlier_frac=outl)
    lin = build(m, n, paths)
    y = lin.forward(x_tensor(x), regime=lb.REGIME_DECODE)
    torch.cuda.synchronize()
    s = assert_bf16_close(to_f64(y), oracle.forward(x_f64(x), paths, m, n), f"decode {m}x{n}")
    log(f"  E_rms={s['erms']:.2e} E_max/rms={s['emax_rel_rms']:.2e}")
    # deterministic: a second run is bit-identical
    y2 = lin.forward(x_tensor(x), regime=lb.REGIME_DECODE)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_forward_errors():
    m, n = 64, 128
    lin = build(m, n, seeded_paths((26, 0, 0), m, n, [8, 8]))
    x = torch.zeros((4, n), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((4, m), dtype=torch.bfloat16, device="cuda")
    L = lb.lib()
    st = torch.cuda.current_stream().cuda_stream
    assert L.lb_linear_forward(lin.handle, x.data_ptr() + 2, y.data_ptr(), 3, lb.BF16, st) == lb._binding.ALIGNMENT
    assert L.lb_linear_forward(lin.handle, x.data_ptr(), y.data_ptr(), 0, lb.BF16, st) == lb._binding.INVALID_ARGUMENT
    assert L.lb_linear_forward_ex(lin.handle, x.data_ptr(), y.data_ptr(), 4, lb.FP32, lb.REGIME_DECODE, st) == \
        lb._binding.UNSUPPORTED
    assert L.lb_linear_forward_ex(lin.handle, x.data_ptr(), y.data_ptr(), 4, lb.BF16, 9, st) == \
        lb._binding.INVALID_ARGUMENT
    info = lin.info()
    assert info["d_out"] == m and info["d_in"] == n and info["ranks"] == [8, 8] and info["device_bytes"] > 0


def test_bound_stack_matches_forward():
    """Stack.bind fixes the pointer arrays once; its forward() runs the same
    launches as Stack.forward."""
    shapes = [(256, 512, [16, 16]), (1024, 300, [33, 20])]
    lins, paths, xs = make_stack(34, shapes, 3)
    xt = [x_tensor(x) for x in xs]
    ya = [torch.empty((3, m), dtype=torch.bfloat16, device="cuda") for (m, _, _) in shapes]
    yb = [torch.empty_like(y) for y in ya]
    S = lb.Stack(lins)
    S.forward(xt, ya, regime=lb.REGIME_DECODE, use_graph=False)
    bound = S.bind(xt, yb, regime=lb.REGIME_DECODE, use_graph=False)
    for _ in range(2):
        bound.forward()
    torch.cuda.synchronize()
    for a, b in zip(ya, yb):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    with pytest.raises(TypeError):
        S.bind(xt, [ya[0].float(), ya[1]])
    del bound
    S.close()


# ----------------------------------------------------------------------------
# bf16 x, fp32 y (LB_BF16_FP32)
# ----------------------------------------------------------------------------

MIXED_CASES = [  # (regime, m, n, ranks, T)
    (lb.REGIME_DECODE, 777, 2100, [319, 5], 1),
    (lb.REGIME_DECODE, 513, 257, [33, 31], 9),
    (lb.REGIME_DECODE, 1024, 640, [102, 90], 16),
    (lb.REGIME_DECODE, 130, 200, [40], 17),        # two decode launches; rows not whole quads
    (lb.REGIME_PREFILL, 600, 520, [70, 50], 200),
    (lb.REGIME_PREFILL, 258, 300, [33], 130),      # ragged rows of y (not a multiple of 4 columns)
    (lb.REGIME_EXACT, 300, 257, [31, 9], 3),
]


@pytest.mark.parametrize("regime,m,n,ranks,T", MIXED_CASES)
def test_bf16_in_fp32_out(regime, m, n, ranks, T):
    """fp32 y from bf16 x: against the oracle, and rounding the fp32 result to
    bf16 (nearest even) gives the bf16-output forward bit for bit (the same
    sums, stored before the last rounding)."""
    log(f"bf16->fp32 regime={regime} m={m} n={n} ranks={ranks} T={T}")
    paths = seeded_paths((31, m, n), m, n, ranks)
    x = x_tensor(synth.activations((31, T, n), T, n))
    lin = build(m, n, paths)
    yf = lin.forward(x, regime=regime, out_dtype=torch.float32)
    yb = lin.forward(x, regime=regime)
    torch.cuda.synchronize()
    assert yf.dtype == torch.float32 and yb.dtype == torch.bfloat16
    ref = oracle.forward(to_f64(x), paths, m, n)
    if regime == lb.REGIME_EXACT:
        assert_fp32_close(to_f64(yf), ref, "exact bf16->fp32")
    else:
        s = assert_bf16_close(to_f64(yf), ref, "bf16->fp32")
        log(f"  E_rms={s['erms']:.2e} E_max/rms={s['emax_rel_rms']:.2e}")
    assert torch.equal(yf.to(torch.bfloat16).view(torch.int16), yb.view(torch.int16))


@pytest.mark.parametrize("regime,T", [(lb.REGIME_DECODE, 4), (lb.REGIME_PREFILL, 256), (lb.REGIME_PREFILL, 72)])
def test_stack_bf16_in_fp32_out(regime, T):
    shapes = [(256, 512, [16, 16]), (1024, 300, [33, 20]), (96, 96, [5])]
    lins, paths, xs = make_stack(32, shapes, T)
    xt = [x_tensor(x) for x in xs]
    ys = [torch.empty((T, m), dtype=torch.float32, device="cuda") for (m, _, _) in shapes]
    S = lb.Stack(lins)
    S.forward(xt, ys, regime=regime, use_graph=False)
    torch.cuda.synchronize()
    for (m, n, _), p, x, y in zip(shapes, paths, xs, ys):
        assert_bf16_close(to_f64(y), oracle.forward(x_f64(x), p, m, n), f"stack bf16->fp32 {m}x{n}")
    with pytest.raises(TypeError):
        S.forward(xt, [y.to(torch.bfloat16) if i == 0 else y for i, y in enumerate(ys)], regime=regime)
    S.close()


# ----------------------------------------------------------------------------
# stacks
# ----------------------------------------------------------------------------

STACK_SHAPES = [(256, 512, [16, 16]), (1024, 300, [33, 20]), (200, 2000, [102, 90]), (4096, 1024, [46, 46]),
                (96, 96, [5]), (700, 700, [149, 149])]


def make_stack(key, shapes, T, io="bf16"):
    lins, paths, xs = [], [], []
    for i, (m, n, ranks) in enumerate(shapes):
        p = seeded_paths((key, i, 0), m, n, ranks)
        paths.append(p)
        lins.append(build(m, n, p))
        xs.append(synth.activations((key, i, T), T, n, io=io))
    return lins, paths, xs


@pytest.mark.parametrize("T", [1, 8, 16])
def test_stack_decode_graph_eager_single_agree(T):
    log(f"stack decode T={T}")
    lins, paths, xs = make_stack(27, STACK_SHAPES, T)
    S = lb.Stack(lins)
    xd = [x_tensor(x) for x in xs]
    ys_g = [torch.empty((T, m), dtype=torch.bfloat16, device="cuda") for m, _, _ in STACK_SHAPES]
    ys_e = [torch.empty_like(y) for y in ys_g]
    S.forward(xd, ys_e, regime=lb.REGIME_DECODE, use_graph=False)
    S.forward(xd, ys_g, regime=lb.REGIME_DECODE, use_graph=True)
    torch.cuda.synchronize()
    for i, (m, n, _) in enumerate(STACK_SHAPES):
        single = lins[i].forward(xd[i], regime=lb.REGIME_DECODE)
        torch.cuda.synchronize()
        assert torch.equal(ys_g[i].view(torch.int16), ys_e[i].view(torch.int16)), f"graph != eager, entry {i}"
        # a single forward is a smaller launch, cut into smaller items: its
        # partial sums are grouped differently, so it is held to the oracle
        ref = oracle.forward(x_f64(xs[i]), paths[i], m, n)
        assert_bf16_close(to_f64(ys_g[i]), ref, f"stack entry {i}")
        assert_bf16_close(to_f64(single), ref, f"single entry {i}")
    # replay the captured graph several times with eager work in between
    ref = [y.clone() for y in ys_g]
    for rep in range(3):
        for y in ys_g:
            y.zero_()
        junk = torch.randn(1000, 1000, device="cuda") @ torch.randn(1000, 1000, device="cuda")
        S.forward(xd, ys_g, regime=lb.REGIME_DECODE, use_graph=True)
        torch.cuda.synchronize()
        del junk
        for i in range(len(ys_g)):
            assert torch.equal(ys_g[i].view(torch.int16), ref[i].view(torch.int16)), f"replay {rep} entry {i}"


# Stack shapes in whole 64-row quads of y, rows of x read with 16-byte loads
FLOW_SHAPES = [(256, 512, [16, 16]), (1024, 320, [33, 20]), (192, 2048, [102, 90]), (4096, 1024, [46, 46]),
               (64, 64, [5]), (704, 704, [149, 149])]


@pytest.mark.parametrize("T", [1, 5, 16])
def test_stack_decode_repeated_steps_and_token_change(T):
    """Decode steps of one stack: every entry against the oracle, direct
    launches and a captured graph equal bit for bit over repeated steps, and a
    token-count change (the plan is rebuilt) and back gives the same outputs."""
    log(f"decode stack repeated steps T={T}")
    lins, paths, xs = make_stack(39, FLOW_SHAPES, T)
    S = lb.Stack(lins)
    xd = [x_tensor(x) for x in xs]
    runs = []
    for g in (False, True, False):
        ys = [torch.full((T, m), 9.0, dtype=torch.bfloat16, device="cuda") for m, _, _ in FLOW_SHAPES]
        for _ in range(3):
            S.forward(xd, ys, regime=lb.REGIME_DECODE, use_graph=g)
        torch.cuda.synchronize()
        runs.append(ys)
    for i, (m, n, _) in enumerate(FLOW_SHAPES):
        assert_bf16_close(to_f64(runs[0][i]), oracle.forward(x_f64(xs[i]), paths[i], m, n), f"dataflow entry {i}")
        for r in runs[1:]:
            assert torch.equal(runs[0][i].view(torch.int16), r[i].view(torch.int16)), f"entry {i} differs between runs"
    # another token count on the same stack, then back
    T2 = 2 if T != 2 else 3
    x2 = [x_tensor(synth.activations((39, i, T2), T2, n)) for i, (_, n, _) in enumerate(FLOW_SHAPES)]
    y2 = [torch.empty((T2, m), dtype=torch.bfloat16, device="cuda") for m, _, _ in FLOW_SHAPES]
    S.forward(x2, y2, regime=lb.REGIME_DECODE)
    ys = [torch.empty((T, m), dtype=torch.bfloat16, device="cuda") for m, _, _ in FLOW_SHAPES]
    S.forward(xd, ys, regime=lb.REGIME_DECODE)
    torch.cuda.synchronize()
    for i, (m, n, _) in enumerate(FLOW_SHAPES):
        assert torch.equal(ys[i].view(torch.int16), runs[0][i].view(torch.int16)), f"entry {i} after T change"
        assert_bf16_close(to_f64(y2[i]), oracle.forward(to_f64(x2[i]), paths[i], m, n), f"T={T2} entry {i}")
    S.close()


# A model's linears in their real order, chained through their buffers: per
# layer q, k, v read the layer input; o reads q's output; gate and up read o's
# output; down reads gate's output; the next layer's q, k, v read down's
# output.  (m, n) per linear at model width D and MLP width F.
CHAIN_D, CHAIN_F = 256, 704
CHAIN_LAYER = [(CHAIN_D, CHAIN_D, [16, 12]), (CHAIN_D // 4, CHAIN_D, [9, 9]), (CHAIN_D // 4, CHAIN_D, [9, 9]),
               (CHAIN_D, CHAIN_D, [16, 12]), (CHAIN_F, CHAIN_D, [33, 20]), (CHAIN_F, CHAIN_D, [33, 20]),
               (CHAIN_D, CHAIN_F, [33, 20])]


def chained_stack(key, layers, T, io):
    shapes = CHAIN_LAYER * layers
    lins, paths = [], []
    for i, (m, n, ranks) in enumerate(shapes):
        p = seeded_paths((key, i, 0), m, n, ranks)
        paths.append(p)
        lins.append(build(m, n, p))
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    x0 = x_tensor(synth.activations((key, 99, T), T, CHAIN_D, io=io))
    ys = [torch.empty((T, m), dtype=dt, device="cuda") for m, _, _ in shapes]
    xs = []
    for l in range(layers):
        b = 7 * l
        inp = x0 if l == 0 else ys[b - 1]
        xs += [inp, inp, inp, ys[b], ys[b + 3], ys[b + 3], ys[b + 4]]
    return shapes, lins, paths, xs, ys


@pytest.mark.parametrize("regime,T,io", [(lb.REGIME_DECODE, 1, "bf16"), (lb.REGIME_DECODE, 16, "bf16"),
                                         (lb.REGIME_DECODE, 40, "bf16"), (lb.REGIME_PREFILL, 200, "bf16"),
                                         (lb.REGIME_EXACT, 3, "fp32"), (lb.REGIME_EXACT, 24, "fp32")])
def test_stack_chained_in_model_order(regime, T, io):
    """Each entry sees its producer's finished output: every link matches the
    oracle applied to the input the entry actually read, graph and direct
    launches agree bit for bit, and single forwards run one after another
    match the oracle link by link too (bit for bit with the stack where the
    plan does not depend on the launch's size: prefill and exact)."""
    log(f"chained stack regime={regime} T={T} io={io}")
    layers = 2
    shapes, lins, paths, xs, ys = chained_stack(31, layers, T, io)
    S = lb.Stack(lins)
    close = assert_bf16_close if io == "bf16" else assert_fp32_close
    bits = torch.int16 if io == "bf16" else torch.int32
    runs = []
    for use_graph in (False, True):
        for y in ys:
            y.zero_()
        S.forward(xs, ys, regime=regime, use_graph=use_graph)
        torch.cuda.synchronize()
        for i, (m, n, _) in enumerate(shapes):
            close(to_f64(ys[i]), oracle.forward(to_f64(xs[i]), paths[i], m, n), f"chained entry {i} graph={use_graph}")
        runs.append([y.clone() for y in ys])
    for i in range(len(shapes)):
        assert torch.equal(runs[0][i].view(bits), runs[1][i].view(bits)), f"graph != direct, entry {i}"
    for y in ys:
        y.zero_()
    for i, (m, n, _) in enumerate(shapes):
        lins[i].forward(xs[i], ys[i], regime=regime)
        torch.cuda.synchronize()
        close(to_f64(ys[i]), oracle.forward(to_f64(xs[i]), paths[i], m, n), f"single link {i}")
        if regime != lb.REGIME_DECODE:
            assert torch.equal(runs[0][i].view(bits), ys[i].view(bits)), f"stack != singles, entry {i}"


@pytest.mark.parametrize("T", [1, 16, 40, 100, 300])
def test_stack_auto_runs_the_regime_it_reports(T):
    """lb_auto_regime names the regime a stack forward in AUTO runs: the AUTO
    outputs equal the forced regime's bit for bit, and match the oracle; few
    tokens run the decode kernels, many the prefill GEMMs."""
    lins, paths, xs = make_stack(38, STACK_SHAPES, T)
    rg = lb.auto_regime(lins, T)
    log(f"stack AUTO T={T}: regime {rg}")
    assert rg in (lb.REGIME_DECODE, lb.REGIME_PREFILL)
    if T == 1:
        assert rg == lb.REGIME_DECODE
    if T == 300:
        assert rg == lb.REGIME_PREFILL
    xd = [x_tensor(x) for x in xs]
    ya = [torch.empty((T, m), dtype=torch.bfloat16, device="cuda") for m, _, _ in STACK_SHAPES]
    yb = [torch.empty_like(y) for y in ya]
    S = lb.Stack(lins)
    S.forward(xd, ya)
    S.forward(xd, yb, regime=rg, use_graph=False)
    torch.cuda.synchronize()
    for i, (m, n, _) in enumerate(STACK_SHAPES):
        assert torch.equal(ya[i].view(torch.int16), yb[i].view(torch.int16)), f"entry {i}"
        assert_bf16_close(to_f64(ya[i]), oracle.forward(x_f64(xs[i]), paths[i], m, n), f"AUTO entry {i}")
    S.close()


@pytest.mark.parametrize("regime", [lb.REGIME_DECODE, lb.REGIME_PREFILL])
def test_stack_refuses_output_over_own_input(regime):
    """An entry whose y overlaps its own x is refused, also when the same bad
    call is repeated (a failed call must not leave the stack looking prepared
    for those pointers); a valid call at the same token count afterwards runs
    and matches the oracle, and a retry of the bad call is refused again."""
    m = n = 256
    T = 4 if regime == lb.REGIME_DECODE else 200
    p = seeded_paths((32, 0, 0), m, n, [16])
    S = lb.Stack([build(m, n, p)])
    xn = synth.activations((32, 1, T), T, n, io="bf16")
    x = x_tensor(xn)
    y = torch.empty((T, m), dtype=torch.bfloat16, device="cuda")
    S.forward([x], [y], regime=regime)        # a valid call first: the stack holds a plan
    torch.cuda.synchronize()
    for _ in range(2):
        with pytest.raises(lb.LittleBitError, match="overlaps its own x"):
            S.forward([x], [x], regime=regime)
    y.zero_()
    S.forward([x], [y], regime=regime)
    torch.cuda.synchronize()
    assert_bf16_close(to_f64(y), oracle.forward(x_f64(xn), p, m, n), "after refused calls")
    with pytest.raises(lb.LittleBitError, match="overlaps its own x"):
        S.forward([x], [x], regime=regime)
    S.close()


@pytest.mark.parametrize("T", [3, 40])
def test_stack_exact_fp32_matches_single(T):
    lins, paths, xs = make_stack(28, STACK_SHAPES[:4], T, io="fp32")
    S = lb.Stack(lins)
    xd = [x_tensor(x) for x in xs]
    ys = [torch.empty((T, m), dtype=torch.float32, device="cuda") for m, _, _ in STACK_SHAPES[:4]]
    S.forward(xd, ys)
    torch.cuda.synchronize()
    for i, (m, n, _) in enumerate(STACK_SHAPES[:4]):
        single = lins[i].forward(xd[i])
        torch.cuda.synchronize()
        assert torch.equal(ys[i], single)
        assert_fp32_close(to_f64(ys[i]), oracle.forward(x_f64(xs[i]), paths[i], m, n), f"fp32 stack {i}")


# ----------------------------------------------------------------------------
# prefill path (bf16 MFMA GEMMs)
# ----------------------------------------------------------------------------

PREFILL_SHAPES = [
    # m, n, ranks, T
    (300, 700, [37, 45], 130),           # ragged everything, one row tile
    (1000, 1200, [149, 102], 300),       # two row tiles, ragged
    (513, 257, [33, 31], 600),           # n not a multiple of 8: element-wise A loads
    (4096, 1024, [46, 46], 256),
    (2000, 300, [600], 129),             # single path
    (1024, 2048, [704, 704], 512),       # Llama-2-13B-like rank at 0.55 BPW
    (4096, 14336, [478, 478], 256),      # long K: many blocks through the LDS pipeline
    (700, 520, [20, 40], 300),           # GEMM1: one 128-wide tile whose first wave spans both paths
    (640, 384, [270, 20], 260),          # GEMM1: a 64-wide last tile spanning both paths; GEMM2: 128-wide last tile
    # at most 64 tokens: 64-row tiles
    (1000, 1200, [149, 102], 16),        # one partial 64-row stripe
    (4096, 1024, [46, 46], 64),          # one full stripe
    # 65 to 128 tokens: 128-row tiles
    (700, 520, [20, 40], 100),           # a partial stripe; a wave's columns in both paths
    (4096, 1024, [46, 46], 128),         # one full 128-row stripe
    (300, 700, [37, 45], 65),            # one 128-row stripe with a single live row
    (513, 257, [33, 31], 128),           # a full stripe, element-wise A loads (n % 8 != 0)
    # one row stripe and more than 128 K blocks: GEMM1 runs in K parts, added by a second launch
    (300, 9000, [37, 45], 40),           # 141 blocks: 2 parts, ragged last block
    (256, 20000, [20, 20], 64),          # 313 blocks: 3 parts, full 64-row stripe
    (513, 8300, [33, 31], 16),           # 2 parts, partial-stripe kernel, element-wise A loads
    (700, 17000, [20, 40], 100),         # 128-row tiles, 3 parts, a wave's columns in both paths
    (300, 16500, [37, 45], 200),         # 256-row tiles, 3 parts
]


@pytest.mark.parametrize("m,n,ranks,T", PREFILL_SHAPES)
def test_prefill_parity(m, n, ranks, T):
    log(f"prefill m={m} n={n} ranks={ranks} T={T}")
    paths = seeded_paths((30, m, n), m, n, ranks)
    x = synth.activations((30, T, n), T, n)
    lin = build(m, n, paths)
    y = lin.forward(x_tensor(x), regime=lb.REGIME_PREFILL)
    torch.cuda.synchronize()
    s = assert_bf16_close(to_f64(y), oracle.forward(x_f64(x), paths, m, n), f"prefill {m}x{n}")
    log(f"  E_rms={s['erms']:.2e} E_max/rms={s['emax_rel_rms']:.2e}")
    for _ in range(4):   # deterministic: repeated runs are bit-identical
        y2 = lin.forward(x_tensor(x), regime=lb.REGIME_PREFILL)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    # where AUTO picks prefill at this token count, it runs the same kernels
    if lb.auto_regime([lin], T) == lb.REGIME_PREFILL:
        y3 = lin.forward(x_tensor(x))
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y3.view(torch.int16))


def test_prefill_token_count_changes():
    m, n = 400, 520
    paths = seeded_paths((31, 0, 0), m, n, [40, 24])
    lin = build(m, n, paths)
    for T in (200, 513, 128, 1):
        x = synth.activations((31, T, n), T, n)
        y = lin.forward(x_tensor(x), regime=lb.REGIME_PREFILL)
        torch.cuda.synchronize()
        assert_bf16_close(to_f64(y), oracle.forward(x_f64(x), paths, m, n), f"prefill T={T}")


@pytest.mark.parametrize("T", [40, 7])
def test_stack_prefill_k_parts(T):
    """A stack whose long-K entries (141 and 313 K blocks) have their GEMM1 cut
    into K parts, beside whole ones: every entry against the oracle, and
    against the same linear run alone (cut the same way), bit for bit."""
    shapes = [(300, 9000, [37, 45]), (256, 512, [16, 16]), (256, 20000, [20, 20]), (200, 2000, [102, 90])]
    lins, paths, xs = make_stack(36, shapes, T)
    S = lb.Stack(lins)
    xd = [x_tensor(x) for x in xs]
    ys = [torch.empty((T, m), dtype=torch.bfloat16, device="cuda") for m, _, _ in shapes]
    S.forward(xd, ys, regime=lb.REGIME_PREFILL, use_graph=False)
    torch.cuda.synchronize()
    for i, (m, n, _) in enumerate(shapes):
        single = lins[i].forward(xd[i], regime=lb.REGIME_PREFILL)
        torch.cuda.synchronize()
        assert torch.equal(ys[i].view(torch.int16), single.view(torch.int16)), f"stack != single, entry {i}"
        assert_bf16_close(to_f64(ys[i]), oracle.forward(x_f64(xs[i]), paths[i], m, n), f"K-part stack {i}")
    S.close()


@pytest.mark.parametrize("T", [300, 90])
def test_stack_prefill_graph_eager_single_agree(T):
    log(f"stack prefill T={T}")
    lins, paths, xs = make_stack(32, STACK_SHAPES, T)
    S = lb.Stack(lins)
    xd = [x_tensor(x) for x in xs]
    ys_g = [torch.empty((T, m), dtype=torch.bfloat16, device="cuda") for m, _, _ in STACK_SHAPES]
    ys_e = [torch.empty_like(y) for y in ys_g]
    S.forward(xd, ys_e, regime=lb.REGIME_PREFILL, use_graph=False)
    S.forward(xd, ys_g, regime=lb.REGIME_PREFILL, use_graph=True)
    torch.cuda.synchronize()
    for i, (m, n, _) in enumerate(STACK_SHAPES):
        single = lins[i].forward(xd[i], regime=lb.REGIME_PREFILL)
        torch.cuda.synchronize()
        assert torch.equal(ys_g[i].view(torch.int16), ys_e[i].view(torch.int16)), f"graph != eager, entry {i}"
        assert torch.equal(ys_g[i].view(torch.int16), single.view(torch.int16)), f"stack != single, entry {i}"
        assert_bf16_close(to_f64(ys_g[i]), oracle.forward(x_f64(xs[i]), paths[i], m, n), f"prefill stack {i}")
    ref = [y.clone() for y in ys_g]
    for rep in range(3):
        for y in ys_g:
            y.zero_()
        junk = torch.randn(1000, 1000, device="cuda") @ torch.randn(1000, 1000, device="cuda")
        S.forward(xd, ys_g, regime=lb.REGIME_PREFILL, use_graph=True)
        torch.cuda.synchronize()
        del junk
        for i in range(len(ys_g)):
            assert torch.equal(ys_g[i].view(torch.int16), ref[i].view(torch.int16)), f"replay {rep} entry {i}"
