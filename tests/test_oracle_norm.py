"""Pins of the oracle's norm folding and fused norm -> int8 quantizer
against exact rational arithmetic, the fp64 norm, closed forms and the
already pinned row quantizer (CPU only).

The norm is the one of the SmoothQuant tutorial page, section on folding
the smoothing into LayerNorm: y_j = (x_j - mu) / sigma * gamma_j + beta_j,
with gamma'_j = gamma_j / s_j and beta'_j = beta_j / s_j.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _rows(seed, M, K, scale=2.0, outliers=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)) * scale
    if outliers:
        x[:, rng.choice(K, size=max(1, K // 100), replace=False)] *= 40.0
    return x.astype(np.float16)


def _ulp32(a, b):
    ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


def test_fold_norm_division():
    rng = np.random.default_rng(1)
    g = rng.standard_normal(512).astype(np.float32)
    b = rng.standard_normal(512).astype(np.float32)
    s = (np.abs(rng.standard_normal(512)) * 5 + 0.01).astype(np.float32)
    g2, b2 = oracle.fold_norm(g, s, b)
    # IEEE division is correctly rounded: the exact quotient rounded once
    for i in range(0, 512, 37):
        assert g2[i] == np.float32(Fraction(float(g[i])) / Fraction(float(s[i])))
        assert b2[i] == np.float32(Fraction(float(b[i])) / Fraction(float(s[i])))
    # power-of-two s divides exactly
    p2 = np.float32(2.0) ** rng.integers(-6, 7, 512).astype(np.float32)
    g3, b3 = oracle.fold_norm(g, p2, b)
    assert np.array_equal(g3, g / p2) and np.array_equal(b3, b / p2)
    g4, b4 = oracle.fold_norm(g, s)
    assert b4 is None and np.array_equal(g4, g2)


@pytest.mark.parametrize("K", [8, 96, 1024])
def test_norm_stats_exact_mean_and_variance(K):
    x = _rows(K, 5, K)
    mu, rstd = oracle.norm_stats(x, oracle.NORM_LAYER, 1e-5)
    mu_r, rstd_r = oracle.norm_stats(x, oracle.NORM_RMS, 1e-6)
    for m in range(x.shape[0]):
        xs = [Fraction(float(v)) for v in x[m]]
        mean = sum(xs) / K
        var = sum((v - mean) ** 2 for v in xs) / K
        ms = sum(v * v for v in xs) / K
        # the mean is the exact rational rounded to double, then to fp32
        assert mu[m] == np.float32(float(mean))
        assert mu_r[m] == 0.0
        want = np.float32(1.0 / np.sqrt(float(var) + np.float64(np.float32(1e-5))))
        assert _ulp32(rstd[m], want) <= 1
        want_r = np.float32(1.0 / np.sqrt(float(ms) + np.float64(np.float32(1e-6))))
        assert _ulp32(rstd_r[m], want_r) <= 1


def test_norm_stats_extremes_stay_exact():
    # the largest fp16 magnitudes and subnormals in one row: the integer sums
    # must not overflow or lose the small terms
    K = 4096
    x = np.full((2, K), np.float16(6e-8), dtype=np.float16)  # fp16 subnormals
    x[0, ::2] = np.float16(65504.0)
    x[1, ::3] = np.float16(-65504.0)
    mu, rstd = oracle.norm_stats(x, oracle.NORM_LAYER, 0.0)
    for m in range(2):
        xs = [Fraction(float(v)) for v in x[m]]
        mean = sum(xs) / K
        var = sum((v - mean) ** 2 for v in xs) / K
        assert mu[m] == np.float32(float(mean))
        assert _ulp32(rstd[m], np.float32(1.0 / np.sqrt(float(var)))) <= 1


def test_layer_norm_matches_fp64():
    M, K = 6, 2048
    x = _rows(3, M, K)
    rng = np.random.default_rng(4)
    g = (rng.standard_normal(K) * 0.5 + 1.0).astype(np.float32)
    b = (rng.standard_normal(K) * 0.1).astype(np.float32)
    for norm, eps in ((oracle.NORM_LAYER, 1e-5), (oracle.NORM_RMS, 1e-6)):
        _, _, y = oracle.norm_quantize(x, g, b, norm, eps, want_y=True)
        x64 = x.astype(np.float64)
        mu = x64.mean(1, keepdims=True) if norm == oracle.NORM_LAYER else 0.0
        var = ((x64 - mu) ** 2).mean(1, keepdims=True)
        y64 = (x64 - mu) / np.sqrt(var + np.float32(eps)) * g + b
        err = np.abs(y - y64).max() / np.abs(y64).max()
        assert err < 2e-6, (norm, err)
        # gamma multiplies column j: a transposed or shifted gamma fails this
        assert np.abs(y - y64).max() < 1e-5 * np.abs(y64).max()


def test_layer_norm_scale_invariance():
    # x -> 2x scales mu and sigma by exactly 2 (eps = 0): the output is the
    # same bit pattern
    x = _rows(5, 4, 1024, scale=1.0)
    g = np.linspace(0.5, 1.5, 1024, dtype=np.float32)
    b = np.linspace(-0.1, 0.1, 1024, dtype=np.float32)
    _, _, y1 = oracle.norm_quantize(x, g, b, oracle.NORM_LAYER, 0.0, want_y=True)
    _, _, y2 = oracle.norm_quantize((x.astype(np.float32) * 2).astype(np.float16), g, b,
                                    oracle.NORM_LAYER, 0.0, want_y=True)
    assert np.array_equal(y1, y2)


def test_constant_row_gives_beta():
    K = 512
    x = np.full((3, K), np.float16(1.375), dtype=np.float16)
    x[1] = np.float16(-7.0)
    x[2] = np.float16(0.0)
    g = np.linspace(0.5, 2.0, K, dtype=np.float32)
    b = np.linspace(-1.0, 1.0, K, dtype=np.float32)
    _, _, y = oracle.norm_quantize(x, g, b, oracle.NORM_LAYER, 1e-5, want_y=True)
    assert np.array_equal(y, np.broadcast_to(b, y.shape))


def test_folded_norm_equals_norm_over_s():
    # the page's identity: the norm with gamma/s, beta/s emits y/s
    M, K = 4, 1024
    x = _rows(6, M, K)
    rng = np.random.default_rng(7)
    g = (rng.standard_normal(K) * 0.3 + 1.0).astype(np.float32)
    b = (rng.standard_normal(K) * 0.2).astype(np.float32)
    s = (np.abs(rng.standard_normal(K)) * 4 + 0.05).astype(np.float32)
    g2, b2 = oracle.fold_norm(g, s, b)
    _, _, y = oracle.norm_quantize(x, g, b, oracle.NORM_LAYER, 1e-5, want_y=True)
    _, _, yf = oracle.norm_quantize(x, g2, b2, oracle.NORM_LAYER, 1e-5, want_y=True)
    ref = y.astype(np.float64) / s
    assert np.abs(yf - ref).max() <= 4e-7 * np.abs(ref).max() + 1e-30
    assert np.allclose(yf, ref, rtol=1e-6, atol=1e-6 * np.abs(ref).max())


@pytest.mark.parametrize("norm", [0, 1])
def test_norm_quantize_uses_the_row_quantizer(norm):
    M, K = 5, 768
    x = _rows(8 + norm, M, K)
    g = np.linspace(0.2, 1.8, K, dtype=np.float32)
    xq, xs, y = oracle.norm_quantize(x, g, None, norm, 1e-5, want_y=True)
    q2, s2 = oracle.quantize_rows_f32(y)
    assert np.array_equal(xq, q2) and np.array_equal(xs, s2)
    # per-tensor static: clamp(round(y * inv)) with the given step
    st = np.array([0.02, 50.0], np.float32)
    xq3, xs3 = oracle.norm_quantize(x, g, None, norm, 1e-5, mode=oracle.PER_TENSOR_STATIC,
                                    static_scale=st)
    want = np.clip(np.round(y * np.float32(50.0)), -127, 127).astype(np.int8)
    assert np.array_equal(xq3, want) and xs3[0] == np.float32(0.02)
    assert (np.abs(xq3) == 127).any()  # the step is tight enough to clamp
