"""Pins of the CPU oracle against things other than itself: the worked example
printed on the SmoothQuant tutorial page, closed forms of the smoothing
factor, invariants of the equivalent transform, textbook rounding, library
routines (numpy/torch conversions and integer matmul) and error bounds.

Each test names the passage it pins.  All run on the CPU in seconds.
"""
import json
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def ulp_dist(a, b):
    """Distance in units in the last place between float32 arrays."""
    ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


def sig3(v):
    """Round to three significant figures, as the page prints."""
    return float(f"{v:.3g}")


# ---------------------------------------------------------------- worked example

def test_tutorial_worked_example(orc):
    """[SQ-tutorial] section 缩放的效果: x = (100, 0.5), w = (0.01, 0.01),
    alpha = 0.5; a 0.4 activation in channel B goes from ~100 % to ~2.5 %
    relative error."""
    g = json.load(open(os.path.join(GOLDEN, "smoothquant_tutorial_worked_example.json")))
    v = g["probe_value_channel_B"]
    # Activations whose channel maxima are exactly (100, 0.5); the probe 0.4 sits in channel B.
    X = np.array([[100.0, v], [-3.0, 0.5]], np.float32)
    W = np.array([[0.01, -0.01], [0.005, 0.002], [-0.003, 0.01]], np.float32)
    x_amax = orc.absmax_cols(X)
    w_amax = orc.absmax_cols(W)
    assert list(x_amax) == g["channel_amax_x"]
    assert np.array_equal(w_amax, np.asarray(g["channel_amax_w"], np.float32))  # fl(0.01)

    # Before smoothing: per-tensor step = 100 / 127 from the tensor's max.
    q_row, step = orc.quantize_rows_f32(np.array([[100.0, v]], np.float32))
    u = g["unsmoothed"]
    assert sig3(step[0]) == u["step"]
    assert int(q_row[0, 1]) == u["q"]
    deq = float(q_row[0, 1]) * float(step[0])
    assert sig3(deq) == u["dequant"]
    assert sig3(abs(deq - v)) == u["abs_error"]
    assert abs(abs(deq - v) / v - u["rel_error_approx"]) < 0.05

    # After smoothing with alpha = 0.5.
    s, inv_s, st = orc.compute_scales(x_amax, w_amax, g["alpha"], static=True)
    sm = g["smoothed"]
    assert sig3(s[0]) == sm["s_A"] and sig3(s[1]) == sm["s_B"]
    assert sig3(st[0]) == sm["step"]
    xq, xs = orc.quantize_act(X, inv_s, orc.PER_TENSOR_STATIC, st)
    assert sig3(np.float32(v) * inv_s[1]) == sm["x_over_s"]
    assert int(xq[0, 1]) == sm["q"]
    deq_s = float(xq[0, 1]) * float(xs[0])
    assert sig3(deq_s) == sm["dequant_scaled"]
    back = deq_s * float(s[1])
    assert sig3(back) == sm["dequant"]
    assert float(f"{abs(back - v):.2g}") == sm["abs_error"]  # printed as 0.010
    assert abs(abs(back - v) / v - sm["rel_error_approx"]) < 0.005
    # Balance after smoothing: both channels' activation and weight maxima agree.
    assert abs(x_amax[0] * inv_s[0] - s[0] * w_amax[0]) < 1e-5


# ---------------------------------------------------------------- smoothing factors

def _amax_pair(syn, K, seed=11):
    x = np.abs(syn.normal(seed, 1, (K,))) * 10 + 1e-3
    w = np.abs(syn.normal(seed, 2, (K,))) * 0.05 + 1e-4
    return x.astype(np.float32), w.astype(np.float32)


def test_alpha_zero_is_inverse_weight_max(orc, syn):
    """[SQ-tutorial] 缩放因子, case alpha = 0: s_j = 1 / w_j."""
    x, w = _amax_pair(syn, 4096)
    s, inv = orc.compute_scales(x, w, 0.0)
    expect = (1.0 / w.astype(np.float64)).astype(np.float32)
    assert ulp_dist(s, expect).max() <= 1


def test_alpha_one_is_activation_max(orc, syn):
    """[SQ-tutorial] 缩放因子, case alpha = 1: s_j = x_j."""
    x, w = _amax_pair(syn, 4096)
    s, inv = orc.compute_scales(x, w, 1.0)
    assert np.array_equal(s, x)
    assert ulp_dist(inv, (1.0 / x.astype(np.float64)).astype(np.float32)).max() <= 1


def test_alpha_half_balances_both_sides(orc, syn):
    """[SQ-tutorial] 缩放因子: with alpha = 0.5, x_j / s_j = s_j * w_j."""
    x, w = _amax_pair(syn, 4096)
    s, inv = orc.compute_scales(x, w, 0.5)
    lhs = x.astype(np.float64) / s
    rhs = s.astype(np.float64) * w
    assert np.max(np.abs(lhs - rhs) / rhs) < 2e-7


def test_clamps(orc):
    """[SQ-practice] §3.2: maxima and s clamped below at 1e-5."""
    x = np.array([0.0, 1e-9, 4.0, 1e12], np.float32)
    w = np.array([0.0, 1e-9, 0.0, 1e-9], np.float32)
    s, inv = orc.compute_scales(x, w, 0.5)
    assert s[0] == np.float32(1.0)           # 1e-5^.5 / 1e-5^.5
    assert s[2] == np.float32(math.sqrt(4.0 / 1e-5).__float__()) or ulp_dist(
        s[2:3], np.float32(math.sqrt(4.0 / np.float64(np.float32(1e-5))))).max() <= 1
    s2, _ = orc.compute_scales(np.array([1e-5], np.float32), np.array([1e6], np.float32), 0.9)
    assert s2[0] == np.float32(1e-5)         # floor on s itself


def test_smoothed_max_shrinks_single_layer(orc, syn):
    """[SQ-ondevice] §3 example (1024x1024 layer, channel 0 x50): the smoothed
    input's max is smaller, and equals max_j x_j^(1-a) w_j^(1-a) (a = 0.5)."""
    cfg = syn.single_1024()
    X, W = cfg["X"], cfg["W"]
    x = orc.absmax_cols(X)
    w = orc.absmax_cols(W)
    s, inv = orc.compute_scales(x, w, 0.5)
    smoothed_max = float(np.max(np.abs(X.astype(np.float64) / s.astype(np.float64))))
    closed = float(np.max(np.sqrt(x.astype(np.float64) * w.astype(np.float64))))
    orig = float(np.max(np.abs(X)))
    print(f"\noriginal max {orig:.2f}, smoothed max {smoothed_max:.4f}")
    assert smoothed_max < orig / 10
    assert abs(smoothed_max - closed) / closed < 1e-6


def test_smoothing_axis_is_input_channel(orc, syn):
    """[SQ-tutorial] SmoothQuant 的原理 and 缩放因子: scaling weight channel j by
    s_j makes its max s_j * w_j; with alpha = 0.5 it matches x_j / s_j."""
    X, W, _ = syn.linear_layer(7, 64, 96, 256, 3, 20.0, 100.0, 0.03)
    x = orc.absmax_cols(X)
    w = orc.absmax_cols(W)
    s, inv = orc.compute_scales(x, w, 0.5)
    Wp = orc.smooth_weights_f32(W, s)
    col_max = orc.absmax_cols(Wp)
    assert np.array_equal(col_max, (w * s).astype(np.float32))
    xs_max = x.astype(np.float64) / s
    assert np.max(np.abs(col_max - xs_max) / xs_max) < 1e-6


def test_equivalence_fp64(orc, syn):
    """[SQ-tutorial] SmoothQuant 的原理: (X S^-1)(S W) = X W in the reals;
    in fp64 to 1e-9 relative (Frobenius)."""
    for X, W in ((syn.single_1024()["X"], syn.single_1024()["W"]),
                 syn.linear_layer(2, 48, 80, 512, 6, 20.0, 100.0, 0.025)[:2]):
        x = orc.absmax_cols(X)
        w = orc.absmax_cols(W)
        s, _ = orc.compute_scales(x, w, 0.5)
        y64 = orc.matmul_f64(X, W)
        ys64 = orc.smoothed_matmul_f64(X, W, s)
        ref = X.astype(np.float64) @ W.astype(np.float64).T
        assert np.linalg.norm(y64 - ref) / np.linalg.norm(ref) < 1e-12
        assert np.linalg.norm(ys64 - y64) / np.linalg.norm(y64) < 1e-9


# ---------------------------------------------------------------- quantizer

def test_round_half_even(orc):
    """Round half to even (Python's round() is the textbook reference)."""
    vals = [k + 0.5 for k in range(-12, 12)] + [0.49999997, 2.5000002, -7.5, 1e7 + 0.5, 3e8]
    for v in vals:
        f = float(np.float32(v))
        assert orc.round_half_even(f) == float(round(f)), v


def test_quantizer_ties_and_exact_unit_step(orc):
    """[INT8-expl] §2.1 quantizer with a row whose max is 127: step = 1, so
    q = round_half_even(v) exactly."""
    row = np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.49, -126.5, 126.5]], np.float32)
    q, step = orc.quantize_rows_f32(row)
    assert step[0] == 1.0
    assert list(q[0]) == [round(float(v)) for v in row[0]]


def test_quantizer_clamp_never_minus_128(orc):
    """[INT8-expl] §2.1: clip to [-127, 127]; static steps too small clamp."""
    x = np.array([[1000.0, -1000.0, 0.3, -0.3]], np.float32)
    xq, xs = orc.quantize_act(x, None, orc.PER_TENSOR_STATIC, np.array([0.01, 100.0], np.float32))
    assert list(xq[0]) == [127, -127, 30, -30]
    assert xs[0] == np.float32(0.01)
    big = np.full((1, 16), -5.0, np.float32)
    q, _ = orc.quantize_rows_f32(big)
    assert q.min() == -127


def test_quantizer_zero_row(orc):
    """[INT8-expl] §2.1 guard max(max_abs, 1e-8): an all-zero row gives q = 0."""
    q, step = orc.quantize_rows_f32(np.zeros((2, 8), np.float32))
    assert not q.any()
    assert step[0] == np.float32(np.float32(1e-8) / np.float32(127.0))


def test_quantizer_error_bound(orc, syn):
    """Abs-max quantization error is at most half a step (plus rounding of
    the step itself) for every element."""
    v = syn.normal(5, 1, (64, 1000)) * np.linspace(0.01, 100, 64, dtype=np.float32)[:, None]
    q, step = orc.quantize_rows_f32(v)
    err = np.abs(q.astype(np.float64) * step[:, None] - v)
    assert np.all(err <= step[:, None] * (0.5 + 1e-5))
    assert np.all(np.abs(q).max(axis=1) == 127)


def test_per_token_vs_static_modes(orc, syn):
    """Per-token steps are row maxima / 127; the static mode takes the step
    it is given for every row ([SQ-tutorial] 为什么激活不能用逐通道量化)."""
    X = syn.normal(9, 1, (8, 128))
    xq, xs = orc.quantize_act(X, None, orc.PER_TOKEN_DYNAMIC)
    rowmax = np.abs(X).max(axis=1)
    assert np.array_equal(xs, (rowmax / np.float32(127)).astype(np.float32))
    st = np.array([rowmax.max() / 127, 127 / rowmax.max()], np.float32)
    xq2, xs2 = orc.quantize_act(X, None, orc.PER_TENSOR_STATIC, st)
    assert xs2.shape == (1,) and xs2[0] == st[0]
    assert np.abs(xq2).max() == 127


# ---------------------------------------------------------------- abs-max

def test_absmax_matches_numpy_and_accumulates(orc, syn):
    """[SQ-practice] §3.2 / [SQ-ondevice] §3: per-channel max over tokens; a
    running max across calibration batches."""
    a = syn.normal(1, 1, (37, 301)).astype(np.float16)
    b = syn.normal(1, 2, (5, 301)).astype(np.float16) * np.float16(3)
    m1 = orc.absmax_cols(a)
    assert np.array_equal(m1, np.abs(a.astype(np.float32)).max(axis=0))
    m2 = orc.absmax_cols(b, m1.copy())
    assert np.array_equal(m2, np.maximum(m1, np.abs(b.astype(np.float32)).max(axis=0)))
    bf = (syn.normal(1, 3, (7, 33)).view(np.uint32) >> 16).astype(np.uint16)
    ref = np.abs((bf.astype(np.uint32) << 16).view(np.float32)).max(axis=0)
    assert np.array_equal(orc.absmax_cols(bf), ref)


# ---------------------------------------------------------------- GEMM

def test_int32_gemm_bruteforce(orc):
    """[INT8-expl] §2.1: int8 x int8 summed in int32 (toy 4x8 @ 8x16 and random
    tiny shapes, extremal +-127 included) against numpy's int64 matmul."""
    rng = np.random.default_rng(123)
    shapes = [(4, 16, 8), (1, 1, 1), (3, 5, 7), (17, 33, 64), (64, 64, 64)]
    for M, N, K in shapes:
        for extremal in (False, True):
            if extremal:
                xq = rng.choice(np.array([-127, 127], np.int8), size=(M, K))
                wq = rng.choice(np.array([-127, 127], np.int8), size=(N, K))
            else:
                xq = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
                wq = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
            _, acc = orc.gemm_i8_dequant(xq, wq, np.ones(M, np.float32), np.ones(N, np.float32))
            ref = xq.astype(np.int64) @ wq.astype(np.int64).T
            assert np.array_equal(acc, ref)
    K = 8192
    xq = np.full((2, K), -127, np.int8)
    wq = np.full((3, K), -127, np.int8)
    _, acc = orc.gemm_i8_dequant(xq, wq, np.ones(2, np.float32), np.ones(3, np.float32))
    assert acc[0, 0] == 127 * 127 * K


def test_dequant_unit_and_power_of_two_scales(orc):
    """[SQ-tutorial] Y = diag(dX) Xq Wq diag(dW): unit scales give the integer
    sum itself; power-of-two scales are exact."""
    rng = np.random.default_rng(5)
    xq = rng.integers(-127, 128, size=(6, 64), dtype=np.int8)
    wq = rng.integers(-127, 128, size=(9, 64), dtype=np.int8)
    y, acc = orc.gemm_i8_dequant(xq, wq, np.ones(6, np.float32), np.ones(9, np.float32))
    assert np.array_equal(y, acc.astype(np.float32))
    dx = np.float32(2.0) ** -rng.integers(0, 10, 6).astype(np.float32)
    dw = np.float32(2.0) ** -rng.integers(0, 10, 9).astype(np.float32)
    y2, _ = orc.gemm_i8_dequant(xq, wq, dx, dw)
    assert np.array_equal(y2, acc.astype(np.float64) * dx[:, None] * dw[None, :])


def test_dequant_outer_product_and_rounding_bound(orc, syn):
    """[INT8-expl] §2.1 outer-product c_x (x) c_w: row m scales by dx_m and
    column n by dw_n; fp32 y within 3 roundings of the exact product."""
    rng = np.random.default_rng(8)
    xq = rng.integers(-127, 128, size=(16, 512), dtype=np.int8)
    wq = rng.integers(-127, 128, size=(24, 512), dtype=np.int8)
    dx = (np.abs(syn.normal(3, 1, (16,))) * 0.01 + 1e-4).astype(np.float32)
    dw = (np.abs(syn.normal(3, 2, (24,))) * 0.001 + 1e-5).astype(np.float32)
    y, acc = orc.gemm_i8_dequant(xq, wq, dx, dw)
    exact = acc.astype(np.float64) * dx[:, None].astype(np.float64) * dw[None, :]
    rel = np.abs(y - exact) / np.maximum(np.abs(exact), 1e-300)
    assert rel.max() <= 3 * 2.0 ** -24 * 1.0001
    # per-tensor: one step for every row
    y1, _ = orc.gemm_i8_dequant(xq, wq, dx[:1], dw)
    y1r, _ = orc.gemm_i8_dequant(xq, wq, np.full(16, dx[0], np.float32), dw)
    assert np.array_equal(y1, y1r)


def test_sampled_gemm_matches_full(orc):
    rng = np.random.default_rng(2)
    xq = rng.integers(-127, 128, size=(20, 96), dtype=np.int8)
    wq = rng.integers(-127, 128, size=(30, 96), dtype=np.int8)
    dx = rng.random(20).astype(np.float32)
    dw = rng.random(30).astype(np.float32)
    y, acc = orc.gemm_i8_dequant(xq, wq, dx, dw, y_dt=orc.BF16)
    r = rng.integers(0, 20, 50)
    c = rng.integers(0, 30, 50)
    ys, accs = orc.gemm_i8_dequant_at(xq, wq, dx, dw, r, c, y_dt=orc.BF16)
    assert np.array_equal(ys, y[r, c]) and np.array_equal(accs, acc[r, c])


# ---------------------------------------------------------------- narrowing

def test_fp16_narrowing_matches_numpy(orc, syn):
    """Output narrowing is IEEE round-to-nearest-even (numpy's float16 cast)."""
    v = np.concatenate([
        syn.normal(4, 1, (20000,)) * 1000,
        syn.normal(4, 2, (20000,)) * 1e-5,            # subnormal range
        np.array([65504, 65519.99, 65520, 1e6, 2.0 ** -25, 2.0 ** -24 * 1.5, -0.0,
                  1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11], np.float32),
    ]).astype(np.float32)
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    got = np.array([orc.f32_to_f16_bits(float(t)) for t in v], np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_narrowing_matches_torch(orc, syn):
    torch = pytest.importorskip("torch")
    v = np.concatenate([syn.normal(4, 3, (20000,)) * 50,
                        np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -1 - 2.0 ** -8], np.float32)])
    v = v.astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.f32_to_bf16_bits(float(t)) for t in v], np.uint16)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- LLM.int8()

def test_outlier_columns_bruteforce(orc, syn):
    """[INT8-expl] §2.2/§4.1: a column is an outlier dim when any |x| >= 6."""
    cfg = syn.llm_int8_2048(M=256, N=64, K=512)
    X = cfg["X"]
    idx = orc.outlier_columns(X, 6.0)
    ref = np.nonzero((np.abs(X.astype(np.float32)) >= 6.0).any(axis=0))[0]
    assert np.array_equal(idx, ref)
    assert np.array_equal(idx, np.asarray(cfg["dims"]))


def test_mixed_with_no_outliers_is_vectorwise(orc, syn):
    """[INT8-expl] §2.2 code branch: with O empty the whole product goes the
    int8 vector-wise way (rows of X, output channels of W)."""
    cfg = syn.llm_int8_2048(M=64, N=48, K=256)
    X, W = cfg["X"], cfg["W"]
    wq, ws = orc.smooth_weights(W, None)
    r = orc.int8_mixed_matmul(X, wq, ws, W, float("inf"))
    assert r["idx"].size == 0
    xq, xs = orc.quantize_act(X, None, orc.PER_TOKEN_DYNAMIC)
    y, acc = orc.gemm_i8_dequant(xq, wq, xs, ws, y_dt=orc.F16)
    assert np.array_equal(r["acc"], acc)
    assert np.array_equal(r["y"].view(np.uint16), y.view(np.uint16))


def test_mixed_with_every_column_is_fp16_product(orc, syn):
    """[INT8-expl] §2.2: the 16-bit side product, accumulated in fp32, is
    within the classical summation bound of the exact product when every
    column is an outlier dim."""
    X, W, _ = syn.linear_layer(12, 32, 40, 128, 0, 1, 1, 0.02)
    wq, ws = orc.smooth_weights(W, None)
    r = orc.int8_mixed_matmul(X, wq, ws, W, 1e-30, y_dt=orc.F32)
    nz = (np.abs(X.astype(np.float32)) > 0).any(axis=0)
    assert r["idx"].size == int(nz.sum())
    assert not r["acc"].any()
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    bound = 128 * 2.0 ** -24 * (np.abs(X.astype(np.float64)) @ np.abs(W.astype(np.float64)).T)
    assert np.all(np.abs(r["y"] - exact) <= bound + 1e-30)


def test_mixed_single_outlier_side_is_exact(orc):
    """One outlier dim: the side term is one exact fp16 x fp16 product."""
    X = np.zeros((3, 64), np.float16)
    X[:, 5] = np.array([7.0, -9.5, 0.25], np.float16)
    X[:, 9] = np.array([1.0, 2.0, -3.0], np.float16)
    W = np.zeros((4, 64), np.float16)
    W[:, 5] = np.array([0.5, -0.125, 3.0, 0.0], np.float16)
    W[:, 9] = np.array([1.0, 1.0, 1.0, 1.0], np.float16)
    wq, ws = orc.smooth_weights(W, None)
    r = orc.int8_mixed_matmul(X, wq, ws, W, 6.0, y_dt=orc.F32)
    assert list(r["idx"]) == [5]
    side = np.outer(X[:, 5].astype(np.float64), W[:, 5].astype(np.float64))
    int8_part = r["acc"].astype(np.float64) * r["x_scale"][:, None] * ws[None, :]
    assert np.allclose(r["y"], side + int8_part, rtol=1e-6, atol=1e-6)
    assert np.array_equal(r["acc"], r["xq"].astype(np.int64) @ wq.astype(np.int64).T)


def test_mixed_row_step_excludes_outlier_columns(orc):
    """[INT8-expl] §2.2 decomposition: the int8 path quantizes x[:, mask], the
    columns that are not outlier dims, so a row's step comes from those
    columns only and the outlier columns contribute no codes.  Worked by
    hand: column 5 (7, -9.5, 0.25) reaches 6 and is an outlier dim; column 9
    (1, 2, -3) does not.  Row 0's non-outlier maximum is 1 (not 7): step
    1/127 and code 127 at column 9; rows 1 and 2 have maxima 2 and 3.  The
    weights are quantized per output channel over all K: row 0 (0.5 and 1)
    has step 1/127 and codes 64 (127 * 0.5 = 63.5, half to even) and 127;
    row 1 (-0.125, 1) codes -16 (-15.875) and 127; row 2 (3, 1) step 3/127,
    codes 127 and 42 (127 / 3 = 42.33); row 3 (0, 1) code 127."""
    X = np.zeros((3, 64), np.float16)
    X[:, 5] = np.array([7.0, -9.5, 0.25], np.float16)
    X[:, 9] = np.array([1.0, 2.0, -3.0], np.float16)
    W = np.zeros((4, 64), np.float16)
    W[:, 5] = np.array([0.5, -0.125, 3.0, 0.0], np.float16)
    W[:, 9] = np.array([1.0, 1.0, 1.0, 1.0], np.float16)
    wq, ws = orc.smooth_weights(W, None)
    assert list(wq[:, 5]) == [64, -16, 127, 0] and list(wq[:, 9]) == [127, 127, 42, 127]
    f = np.float32
    assert list(ws) == [f(1) / f(127), f(1) / f(127), f(3) / f(127), f(1) / f(127)]
    r = orc.int8_mixed_matmul(X, wq, ws, W, 6.0, y_dt=orc.F32)
    assert list(r["idx"]) == [5]
    assert list(r["x_scale"]) == [f(1) / f(127), f(2) / f(127), f(3) / f(127)]
    want_xq = np.zeros((3, 64), np.int8)
    want_xq[:, 9] = [127, 127, -127]
    assert np.array_equal(r["xq"], want_xq)          # column 5 carries no code
    assert r["acc"].tolist() == [[16129, 16129, 5334, 16129], [16129, 16129, 5334, 16129],
                                 [-16129, -16129, -5334, -16129]]


def test_mixed_merge_rounds_once(orc):
    """[INT8-expl] §2.2 adds the 16-bit side result and the int8 result into
    one 16-bit output; the reading here forms fl(dequant + side) in fp32 and
    rounds to fp16 once.  Worked by hand: non-outlier row maximum 127/64
    gives step 2^-6 and codes x * 64; weight row maximum 127/32 gives step
    2^-5 and codes w * 32; the int8 sum 127 * 16 + 17 * 1 = 2049 dequantizes
    exactly to 2049 * 2^-11 = 1 + 2^-11; the outlier dim (x = 8) times
    w = 2^-14 gives side = 2^-11.  One rounding: 1 + 2^-10 exactly.  Rounding
    the dequantized value to fp16 first (1 + 2^-11 is a tie: 1.0) and then
    adding gives 1.0."""
    K = 64
    X = np.zeros((1, K), np.float16)
    X[0, 0] = 127 / 64          # q = 127
    X[0, 1] = 17 / 64           # q = 17
    X[0, 3] = 8.0               # the outlier dim
    W = np.zeros((1, K), np.float16)
    W[0, 0] = 0.5               # q = 16
    W[0, 1] = 1 / 32            # q = 1
    W[0, 2] = 127 / 32          # the row maximum, q = 127 (X is 0 there)
    W[0, 3] = 2.0 ** -14
    wq, ws = orc.smooth_weights(W, None)
    assert ws[0] == 2.0 ** -5 and list(wq[0, :3]) == [16, 1, 127]
    r = orc.int8_mixed_matmul(X, wq, ws, W, 6.0, y_dt=orc.F16)
    assert list(r["idx"]) == [3]
    assert r["x_scale"][0] == 2.0 ** -6
    assert r["acc"][0, 0] == 2049
    assert r["y"][0, 0] == np.float16(1 + 2.0 ** -10)
    assert np.float16(np.float16(1 + 2.0 ** -11) + np.float16(2.0 ** -11)) == 1.0  # the other order


def test_mixed_side_sums_in_ascending_column_order(orc):
    """The side term accumulates the outlier dims in ascending column order
    from 0 in fp32.  Worked by hand with a zero int8 part: products 2^10
    (column 2), 2^-14 (column 5), 2^-14 (column 7).  Ascending:
    2^10 + 2^-14 is a tie at fp32's 2^-13 spacing and rounds to 2^10, twice:
    the sum is 2^10.  Any order that adds the two small products first gives
    2^10 + 2^-13."""
    K = 16
    X = np.zeros((1, K), np.float16)
    W = np.zeros((2, K), np.float16)
    X[0, [2, 5, 7]] = 8.0
    W[0, 2], W[0, 5], W[0, 7] = 128.0, 2.0 ** -17, 2.0 ** -17
    W[1, 2], W[1, 5], W[1, 7] = 2.0 ** -17, 2.0 ** -17, 128.0   # the big product last
    wq, ws = orc.smooth_weights(W, None)
    r = orc.int8_mixed_matmul(X, wq, ws, W, 6.0, y_dt=orc.F32)
    assert list(r["idx"]) == [2, 5, 7]
    assert not r["xq"].any() and not r["acc"].any()
    assert r["y"][0, 0] == np.float32(2.0 ** 10)
    assert r["y"][0, 1] == np.float32(2.0 ** 10 + 2.0 ** -13)


def test_mixed_threshold_is_inclusive(orc):
    """[INT8-expl] §4.1: a value reaching the threshold marks its dimension:
    |x| = 6.0 is an outlier, 5.99609375 (the fp16 value just below) is not."""
    X = np.zeros((2, 16), np.float16)
    X[0, 4] = -6.0
    X[1, 11] = 5.99609375
    X[1, 12] = 6.0
    assert list(orc.outlier_columns(X, 6.0)) == [4, 12]


def test_mixed_prep_and_sampled(orc, syn):
    cfg = syn.llm_int8_2048(M=128, N=96, K=256)
    X, W = cfg["X"], cfg["W"]
    wq, ws = orc.smooth_weights(W, None)
    r = orc.int8_mixed_matmul(X, wq, ws, W, 6.0)
    idx, xq, xs = orc.int8_mixed_prep(X, 6.0)
    assert np.array_equal(idx, r["idx"]) and np.array_equal(xq, r["xq"])
    rows = np.arange(0, 128, 7)
    cols = (rows * 5) % 96
    ys, accs = orc.int8_mixed_at(X, xq, xs, wq, ws, W, idx, rows, cols)
    assert np.array_equal(ys.view(np.uint16), r["y"].view(np.uint16)[rows, cols])
    assert np.array_equal(accs, r["acc"][rows, cols])


def test_vectorwise_toy_error(orc, syn):
    """[INT8-expl] §2.1 toy: X (4x8) with one value x40, W (8x16), rows of X
    and columns of W quantized separately; the dequantized product is close
    to the fp32 product (the page reports errors of order 1e-3..1e-2)."""
    X = syn.normal(0, 1, (4, 8)).astype(np.float16)
    X[0, 3] = 40.0
    Wt = syn.normal(0, 2, (16, 8)).astype(np.float16)   # W^T: [out, in]
    wq, ws = orc.smooth_weights(Wt, None)
    xq, xs = orc.quantize_act(X, None, orc.PER_TOKEN_DYNAMIC)
    y, _ = orc.gemm_i8_dequant(xq, wq, xs, ws)
    ref = X.astype(np.float32) @ Wt.astype(np.float32).T
    rel = np.abs(y - ref).max() / np.abs(ref).max()
    assert rel < 3e-2


# ---------------------------------------------------------------- generator

def test_generator_splitmix64_published_sequence(syn):
    """SplitMix64's first outputs from state 1234567, as listed with the
    published reference implementation."""
    got = syn.raw_u64(1234567, 5)
    assert list(map(int, got)) == [6457827717110365317, 3203168211198807973,
                                   9817491932198370423, 4593380528125082431,
                                   16408922859458223821]


def test_generator_is_deterministic_and_normal(syn):
    a = syn.normal(3, 2, (1000, 100))
    b = syn.normal(3, 2, (1000, 100))
    assert np.array_equal(a, b)
    assert abs(a.mean()) < 0.01 and abs(a.std() - 1) < 0.01
    assert not np.array_equal(a, syn.normal(3, 1, (1000, 100)))
