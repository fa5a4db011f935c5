"""The alpha sweep (a report of quantization error against alpha) run on the
CPU oracle: closed forms of its outlier ratios and the pages' central claim
on a small outlier layer.  The same sweep on the GPU kernels is compared with
this one in a GPU test below.

x_j / s_j = (x_j w_j)^(1 - alpha) and s_j w_j = (x_j w_j)^alpha (the
SmoothQuant tutorial page, section 缩放因子), so the max/median ratios are
R^(1 - alpha) and R^alpha for R the ratio of x_j w_j: 1 at the two ends and
equal at alpha = 0.5.
"""
import numpy as np
import pytest

import alpha_sweep
import oracle
import synth


class OracleBackend:
    def absmax(self, a):
        return oracle.absmax_cols(a)

    def scales(self, x_amax, w_amax, alpha, static):
        r = oracle.compute_scales(x_amax, w_amax, alpha, static=static)
        return r[0], r[1], (r[2] if static else None)

    def smooth_weights(self, w, s):
        return oracle.smooth_weights(w, s)

    def quantize_act(self, x, inv_s, st):
        mode = oracle.PER_TENSOR_STATIC if st is not None else oracle.PER_TOKEN_DYNAMIC
        return oracle.quantize_act(x, inv_s, mode, st)

    def gemm(self, xq, wq, xs, ws):
        return oracle.gemm_i8_dequant(xq, wq, xs, ws, y_dt=oracle.F32,
                                      per_row=int(xs.size > 1))[0]

    def rows(self, t, idx):
        return t[idx]

    def host(self, t):
        return t


def _layer(M=64, K=256, N=192):
    # X with two outlier channels (x25 .. x40), W ~ N(0, 0.03)
    X, W, _ = synth.linear_layer(11, M, N, K, 2, 25.0, 40.0, 0.03)
    return {"X": X, "W": W}


ALPHAS = [None, 0.0, 0.25, 0.5, 0.75, 1.0]


@pytest.fixture(scope="module")
def rows_static():
    cfg = _layer()
    return alpha_sweep.sweep(cfg["X"], cfg["W"], ALPHAS, alpha_sweep.STATIC, OracleBackend(),
                             sample_rows=64)


def test_ratio_closed_forms(rows_static):
    by = {r["alpha"]: r for r in rows_static}
    assert by[0.0]["w_ratio"] == pytest.approx(1.0, rel=1e-5)
    assert by[1.0]["x_ratio"] == pytest.approx(1.0, rel=1e-5)
    assert by[0.5]["x_ratio"] == pytest.approx(by[0.5]["w_ratio"], rel=1e-4)
    # R^(1 - a) and R^a from the alpha = 0 / alpha = 1 ends
    R = by[0.0]["x_ratio"]
    assert by[1.0]["w_ratio"] == pytest.approx(R, rel=1e-4)
    for a in (0.25, 0.5, 0.75):
        assert by[a]["x_ratio"] == pytest.approx(R ** (1 - a), rel=1e-3)
        assert by[a]["w_ratio"] == pytest.approx(R ** a, rel=1e-3)


def test_smoothing_helps_static_per_tensor(rows_static):
    # the pages' claim: with outlier channels and one activation step per
    # tensor, migrating difficulty into the weights cuts the output error
    by = {r["alpha"]: r for r in rows_static}
    assert by[0.5]["y_err"] < 0.5 * by["none"]["y_err"]
    # the trade-off: activation error falls and weight error rises with alpha
    assert by[1.0]["x_err"] < by[0.25]["x_err"]
    assert by[1.0]["w_err"] > by[0.25]["w_err"]
    assert by["none"]["x_zero"] > by[0.5]["x_zero"]


def test_sweep_shape_and_token_mode():
    cfg = _layer(M=32)
    rows = alpha_sweep.sweep(cfg["X"], cfg["W"], [None, 0.5], alpha_sweep.TOKEN,
                             OracleBackend(), sample_rows=16)
    assert [r["alpha"] for r in rows] == ["none", 0.5]
    for r in rows:
        assert 0 < r["y_err"] < 0.2 and 0 <= r["x_zero"] <= 1
    md = alpha_sweep.markdown(rows, "t")
    assert md.count("\n| ") == 3


@pytest.mark.gpu
def test_gpu_sweep_matches_oracle_sweep():
    cfg = _layer(M=128, K=1024, N=512)
    want = alpha_sweep.sweep(cfg["X"], cfg["W"], ALPHAS, alpha_sweep.STATIC, OracleBackend(),
                             sample_rows=64)
    got = alpha_sweep.sweep(cfg["X"], cfg["W"], ALPHAS, alpha_sweep.STATIC,
                            alpha_sweep.GpuBackend(), sample_rows=64)
    for g, w in zip(got, want):
        assert g["alpha"] == w["alpha"]
        for k in ("y_err", "x_err", "w_err", "x_zero", "w_zero", "x_ratio", "w_ratio"):
            assert g[k] == pytest.approx(w[k], rel=1e-3, abs=1e-6), (g["alpha"], k)


@pytest.mark.gpu
def test_llm_int8_error_report_on_gpu():
    """The LLM.int8() rows of the report on a reduced workload: threshold inf
    keeps no outlier column, 6.0 finds the six planted dimensions, and
    keeping them in 16-bit lowers the error."""
    import alpha_sweep
    import synth

    backend = alpha_sweep.GpuBackend()
    cfg = synth.llm_int8_2048(M=256, N=512, K=1024)
    rows = alpha_sweep.mixed_errors(cfg["X"], cfg["W"], [float("inf"), 6.0], backend, 128)
    assert [r["n_outliers"] for r in rows[:2]] == [0, 6]
    assert rows[1]["y_err"] < rows[0]["y_err"]
    assert rows[2]["method"].startswith("SmoothQuant") and 0 < rows[2]["y_err"] < rows[0]["y_err"]
