"""Pins of the oracle's output-channel folding (CPU only).

The SmoothQuant tutorial page, section 融入前序线性层的权重 and the table of
fold positions: the 1/s_j that down_proj's input needs is applied by
multiplying up_proj's output channel j by 1/s_j (o_proj's by v_proj's), and
down_proj's input channel j is multiplied by s_j as usual.  The oracle's
fold_smooth_weights applies a per-output-row factor before the per-column
smoothing and the per-row int8 quantizer.
"""
import numpy as np
import pytest

import oracle


def _w(seed, N, K, std=0.03, dt=np.float16):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((N, K)) * std).astype(dt)


@pytest.mark.parametrize("dt", [np.float16, np.float32])
def test_unit_row_factor_is_plain_smoothing(dt):
    w = _w(1, 96, 256, dt=dt)
    s = (np.abs(np.random.default_rng(2).standard_normal(256)) + 0.1).astype(np.float32)
    q0, d0 = oracle.smooth_weights(w, s)
    q1, d1 = oracle.fold_smooth_weights(w, np.ones(96, np.float32), s)
    q2, d2 = oracle.fold_smooth_weights(w, None, s)
    assert np.array_equal(q0, q1) and np.array_equal(d0, d1)
    assert np.array_equal(q0, q2) and np.array_equal(d0, d2)


def test_power_of_two_row_factor_scales_steps_exactly():
    # fl(fl(w r) s) = fl(w s) r for r = 2^e, so the row maximum, 127 / max and
    # the step all scale by r exactly and the codes do not change.
    N, K = 128, 512
    w = _w(3, N, K)
    rng = np.random.default_rng(4)
    s = (np.abs(rng.standard_normal(K)) * 3 + 0.05).astype(np.float32)
    r = (2.0 ** rng.integers(-5, 6, N)).astype(np.float32)
    q0, d0 = oracle.smooth_weights(w, s)
    q1, d1 = oracle.fold_smooth_weights(w, r, s)
    assert np.array_equal(q0, q1)
    assert np.array_equal(d1, d0 * r)


def test_dequantized_weights_follow_rows_and_columns():
    # W''_q[n, k] * step_n lies within half a step (plus fp32 rounding) of
    # r_n W[n, k] s_k: a row factor applied along K, or s along N, fails.
    N, K = 64, 256
    w = _w(5, N, K)
    rng = np.random.default_rng(6)
    r = (np.abs(rng.standard_normal(N)) * 2 + 0.1).astype(np.float32)
    s = (np.abs(rng.standard_normal(K)) * 2 + 0.1).astype(np.float32)
    q, d = oracle.fold_smooth_weights(w, r, s)
    want = r[:, None].astype(np.float64) * w.astype(np.float64) * s[None, :].astype(np.float64)
    got = q.astype(np.float64) * d[:, None].astype(np.float64)
    bound = 0.5 * d[:, None].astype(np.float64) * (1 + 1e-6) + np.abs(want) * 2.0 ** -21
    assert (np.abs(got - want) <= bound).all()
    # the row maxima of r W s hit +-127 exactly once per row at least
    assert (np.abs(q).max(axis=1) == 127).all()


def test_folded_mlp_matches_unfolded():
    # down(act(gate x) * up(x)) with up's rows times 1/s and down's columns
    # times s is the same function; with int8 weights it stays within the
    # quantization error of the unfolded int8 MLP, and the intermediate
    # activation arrives divided by s.
    rng = np.random.default_rng(7)
    M, H, F = 32, 256, 512
    x = rng.standard_normal((M, H))
    wg = (rng.standard_normal((F, H)) * 0.05).astype(np.float32)
    wu = (rng.standard_normal((F, H)) * 0.05).astype(np.float32)
    wd = (rng.standard_normal((H, F)) * 0.05).astype(np.float32)
    wu[[3, 77, 301], :] *= 40.0  # outlier channels of down_proj's input
    silu = lambda t: t / (1.0 + np.exp(-t))
    g = silu(x @ wg.T.astype(np.float64))
    h = g * (x @ wu.T.astype(np.float64))
    y_ref = h @ wd.T.astype(np.float64)

    act_amax = np.abs(h).max(axis=0).astype(np.float32)
    w_amax = oracle.absmax_cols(wd)
    s, inv_s = oracle.compute_scales(act_amax, w_amax, 0.5)
    uq, ud = oracle.fold_smooth_weights(wu, inv_s, None)
    dq, dd = oracle.smooth_weights(wd, s)
    up_f = uq.astype(np.float64) * ud[:, None]
    h_f = g * (x @ up_f.T)
    # the intermediate activation is h / s up to the int8 error of up
    rel_h = np.abs(h_f * s - h).max() / np.abs(h).max()
    assert rel_h < 0.02, rel_h
    # smoothing shrank the outlier channels of down_proj's input
    assert np.abs(h_f).max(axis=0)[[3, 77, 301]].max() < 0.5 * np.abs(h).max(axis=0)[[3, 77, 301]].min()
    y = h_f @ (dq.astype(np.float64) * dd[:, None]).T
    rel_y = np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref)
    assert rel_y < 0.02, rel_y
    # folding the wrong way round (rows times s) breaks the identity
    uq2, ud2 = oracle.fold_smooth_weights(wu, s, None)
    h_bad = g * (x @ (uq2.astype(np.float64) * ud2[:, None]).T)
    y_bad = h_bad @ (dq.astype(np.float64) * dd[:, None]).T
    assert np.linalg.norm(y_bad - y_ref) / np.linalg.norm(y_ref) > 0.5
