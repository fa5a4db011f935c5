"""GPU parity of the norm folding and the fused norm -> int8 quantizer
against the CPU oracle, on the same seeded inputs.

Bars: folded parameters bit-exact (one correctly rounded division each);
int8 codes and row steps bit-exact given the same folded parameters (the
row statistics are exact sums on both sides, then the same sequence of
correctly rounded double operations).
"""
import numpy as np
import pytest

import oracle
import synth
import w8a8_post_quantization_amd as sq
from tests.gpu_util import assert_bits_equal, dev, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t

    if not _t.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    sq.lib()
    return _t


def _x(seed, M, K, scale=2.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)) * scale
    if K >= 100:
        x[:, rng.choice(K, size=K // 100, replace=False)] *= 30.0
    return x.astype(np.float16)


def test_fold_norm_parity(torch):
    K = 7168
    g, b = synth.norm_params(K)
    s = (np.abs(synth.normal(3, 4, (K,))) * 6 + 0.02).astype(np.float32)
    log("fold_norm")
    g2, b2 = sq.fold_norm(dev(g, torch), dev(s, torch), dev(b, torch))
    g_o, b_o = oracle.fold_norm(g, s, b)
    assert_bits_equal(host(g2, torch), g_o, "gamma'")
    assert_bits_equal(host(b2, torch), b_o, "beta'")
    g3, b3 = sq.fold_norm(dev(g, torch), dev(s, torch))
    assert b3 is None
    assert_bits_equal(host(g3, torch), g_o, "gamma' (no beta)")


@pytest.mark.parametrize("M,K,norm,with_beta,mode", [
    (1, 16, 0, True, 1), (3, 48, 1, False, 1), (7, 1024, 0, True, 1), (33, 2048, 1, True, 1),
    (256, 7168, 0, True, 1), (256, 7168, 1, False, 1), (5, 16384, 0, False, 1),
    (64, 4096, 1, True, 0), (40, 2064, 0, True, 0), (2, 8208, 0, True, 1), (0, 64, 0, True, 0),
    (0, 64, 1, False, 1), (300, 512, 0, False, 1),
    # many rows: blocks walk several rows (beta staged in LDS up to K = 8192)
    (2048, 1024, 0, True, 1), (2100, 4096, 1, False, 1), (2051, 48, 1, True, 1),
    (4096, 8192, 0, True, 0), (2304, 7168, 0, True, 1), (2049, 2064, 1, True, 0),
    (2050, 8208, 0, True, 1)])
def test_norm_quantize_parity(torch, M, K, norm, with_beta, mode):
    x = _x(M * 31 + K, M, K)
    g, b = synth.norm_params(K, seed=M + K)
    b = b if with_beta else None
    st = None
    if mode == 0:
        st = np.array([0.01, 100.0], np.float32)  # tight: some codes clamp
    eps = 1e-5 if norm == 0 else 1e-6
    log(f"norm_quantize M={M} K={K} norm={norm} beta={with_beta} mode={mode}")
    xq, xs = sq.norm_quantize_act(dev(x, torch), dev(g, torch),
                                  None if b is None else dev(b, torch), norm, eps, mode,
                                  None if st is None else dev(st, torch))
    xq_o, xs_o = oracle.norm_quantize(x, g, b, norm, eps, mode, st)
    assert_bits_equal(host(xs, torch), xs_o, "x_scale")
    assert_bits_equal(host(xq, torch), xq_o, "xq")


@pytest.mark.parametrize("M,K,norm,with_beta,mode", [
    # the wave-per-row kernel forced, at every row length it is built for
    # (K = 2048, 3072, ..., 8192), with rows fewer than, equal to and more
    # than its waves, ragged over them
    (1, 2048, 0, True, 1), (9, 3072, 1, False, 1), (37, 4096, 0, True, 0),
    (300, 5120, 1, True, 1), (2049, 6144, 0, True, 1), (100, 7168, 0, False, 0),
    (513, 8192, 1, True, 1), (4099, 7168, 0, True, 1), (2053, 7168, 1, False, 0),
    (77, 2048, 0, True, 1), (3001, 8192, 1, True, 1), (2048, 4096, 0, False, 0)])
def test_norm_quantize_wave_kernel(torch, M, K, norm, with_beta, mode):
    x = _x(M * 17 + K, M, K)
    g, b = synth.norm_params(K, seed=M + 2 * K)
    b = b if with_beta else None
    st = np.array([0.01, 100.0], np.float32) if mode == 0 else None
    eps = 1e-5 if norm == 0 else 1e-6
    log(f"norm_quantize wave kernel M={M} K={K} norm={norm} beta={with_beta} mode={mode}")
    xq, xs = sq.norm_quantize_act(dev(x, torch), dev(g, torch),
                                  None if b is None else dev(b, torch), norm, eps, mode,
                                  None if st is None else dev(st, torch), kernel=1)
    xq_o, xs_o = oracle.norm_quantize(x, g, b, norm, eps, mode, st)
    assert_bits_equal(host(xs, torch), xs_o, "x_scale")
    assert_bits_equal(host(xq, torch), xq_o, "xq")


def test_norm_quantize_kernels_agree_many_rows(torch):
    """At 8200 rows x 7168 the library picks the wave-per-row kernel; the
    block-per-row kernel forced on the same rows gives the same bits, and
    both match the oracle on every row."""
    M, K = 8200, 7168
    x = _x(5, M, K)
    g, b = synth.norm_params(K, seed=3)
    xd, gd, bd = dev(x, torch), dev(g, torch), dev(b, torch)
    xq_o, xs_o = oracle.norm_quantize(x, g, b, 0, 1e-5)
    for kernel in (None, 0, 1):
        log(f"norm_quantize {M}x{K} kernel={kernel}")
        xq, xs = sq.norm_quantize_act(xd, gd, bd, 0, 1e-5, kernel=kernel)
        assert_bits_equal(host(xs, torch), xs_o, f"x_scale kernel={kernel}")
        assert_bits_equal(host(xq, torch), xq_o, f"xq kernel={kernel}")


@pytest.mark.parametrize("norm,with_beta,mode", [(1, False, 0), (0, True, 0), (1, True, 1)])
def test_norm_quantize_wave_kernel_streamed_codes(torch, norm, with_beta, mode):
    """Codes beyond the 256 MB last-level cache are stored nontemporally:
    33000 rows x 8192 (270 MB of codes) through that store path."""
    M, K = 33000, 8192
    x = _x(101 + norm, M, K)
    g, b = synth.norm_params(K, seed=13)
    b = b if with_beta else None
    st = np.array([0.02, 50.0], np.float32) if mode == 0 else None
    log(f"norm_quantize streamed codes M={M} K={K} norm={norm} beta={with_beta} mode={mode}")
    xq, xs = sq.norm_quantize_act(dev(x, torch), dev(g, torch),
                                  None if b is None else dev(b, torch), norm, 1e-5, mode,
                                  None if st is None else dev(st, torch))
    xq_o, xs_o = oracle.norm_quantize(x, g, b, norm, 1e-5, mode, st)
    assert_bits_equal(host(xs, torch), xs_o, "x_scale")
    assert_bits_equal(host(xq, torch), xq_o, "xq")


def test_norm_quantize_extreme_rows(torch):
    """Largest fp16 magnitudes, subnormals, constant and zero rows."""
    K = 4096
    x = np.full((6, K), np.float16(6e-8), dtype=np.float16)
    x[0, ::2] = np.float16(65504.0)
    x[1, ::3] = np.float16(-65504.0)
    x[2] = np.float16(1.375)                    # constant row: y = beta
    x[3] = np.float16(0.0)                      # zero row
    x[4] = _x(9, 1, K)[0]
    x[5, :] = np.float16(-2.0)
    x[5, 7] = np.float16(3.0)
    g, b = synth.norm_params(K, seed=11)
    for norm in (0, 1):
        xq_o, xs_o = oracle.norm_quantize(x, g, b, norm, 1e-5)
        for kernel in (0, 1):
            log(f"norm_quantize extremes norm={norm} kernel={kernel}")
            xq, xs = sq.norm_quantize_act(dev(x, torch), dev(g, torch), dev(b, torch), norm,
                                          1e-5, kernel=kernel)
            assert_bits_equal(host(xs, torch), xs_o, "x_scale")
            assert_bits_equal(host(xq, torch), xq_o, "xq")


def test_folded_norm_prefill_full_size(torch):
    """The prefill layer's input path at full size: smoothing factors from
    the layer's statistics, folded into the norm, then the fused norm ->
    per-token int8 of X fp16 [256, 7168]."""
    cfg = synth.prefill_30b()
    X, W = cfg["X"], cfg["W"]
    g, b = synth.norm_params(X.shape[1])
    log("folded norm prefill stats")
    xa = oracle.absmax_cols(X)
    wa = oracle.absmax_cols(W)
    s, _ = oracle.compute_scales(xa, wa, 0.5)
    g2, b2 = sq.fold_norm(dev(g, torch), dev(s, torch), dev(b, torch))
    g_o, b_o = oracle.fold_norm(g, s, b)
    assert_bits_equal(host(g2, torch), g_o, "gamma'")
    assert_bits_equal(host(b2, torch), b_o, "beta'")
    log("folded norm prefill quantize")
    xq, xs = sq.norm_quantize_act(dev(X, torch), g2, b2, sq.SQ_NORM_LAYER, 1e-5)
    xq_o, xs_o = oracle.norm_quantize(X, g_o, b_o, oracle.NORM_LAYER, 1e-5)
    assert_bits_equal(host(xs, torch), xs_o, "x_scale")
    assert_bits_equal(host(xq, torch), xq_o, "xq")
