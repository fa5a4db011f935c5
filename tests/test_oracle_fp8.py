"""Pins of the oracle's FP8 (e4m3) variant (CPU only).

The SmoothQuant encyclopedia page (newton.com.tw), section 技術原理與特性:
the quantized model can run on INT8 or FP8 units.  The e4m3 format (OCP
e4m3fn) is pinned against torch's own float8_e4m3fn conversion, a library
routine independent of the oracle; the quantizers and the GEMM against
closed forms and numpy.
"""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")


def _torch_enc(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.fp8_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert ours[0x7E] == 448.0 and ours[0x38] == 1.0 and ours[0x01] == 2.0 ** -9


def test_encode_round_trip_and_torch():
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle.fp8_decode(finite)
    assert np.array_equal(oracle.fp8_encode(vals), finite)
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.uniform(-448, 448, 4000), rng.uniform(-0.03, 0.03, 4000),
                        rng.uniform(-2.0 ** -8, 2.0 ** -8, 1000)]).astype(np.float32)
    assert np.array_equal(oracle.fp8_encode(v), _torch_enc(v))


def test_encode_ties_to_even():
    pos = oracle.fp8_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)  # exact in fp32
    got = oracle.fp8_encode(mids).astype(np.int64)
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, want)
    assert np.array_equal(got, _torch_enc(mids))
    # just off the midpoints the nearest code wins
    up = np.nextafter(mids, np.float32(np.inf))
    assert np.array_equal(oracle.fp8_encode(up).astype(np.int64), lo + 1)


def test_row_quantizer_fp8():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal((6, 512)) * np.array([1, 10, 1e-3, 100, 1, 1])[:, None]).astype(
        np.float32)
    v[5] = 0.0
    q, step = oracle.quantize_rows_fp8(v)
    deq = oracle.fp8_decode(q).astype(np.float64) * step[:, None]
    for r in range(5):
        a = np.abs(v[r]).max()
        assert step[r] == np.float32(a) / np.float32(448)
        assert (np.abs(oracle.fp8_decode(q[r])) == 448).sum() >= 1   # the max hits 448
        # relative error of normal values (|z| >= 2^-6) at most half a step of
        # the 3-bit mantissa; subnormals within 2^-10 of the code grid
        z = np.abs(v[r].astype(np.float64) / step[r])
        normal = z >= 2.0 ** -6
        err = np.abs(deq[r] - v[r])
        assert (err[normal] <= np.abs(v[r][normal]) * 2.0 ** -4 * (1 + 1e-6)).all()
        assert (err[~normal] <= 2.0 ** -10 * step[r] * (1 + 1e-6)).all()
    assert (q[5] == 0).all() and step[5] == np.float32(1e-8) / np.float32(448)


def test_act_and_weights_fp8_static_and_smoothing():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((8, 256)) * 3).astype(np.float16)
    inv_s = (rng.uniform(0.2, 2.0, 256)).astype(np.float32)
    xa = oracle.absmax_cols(x)
    st = oracle.static_scale(xa, inv_s, 448.0)
    a = (xa * inv_s).max()
    assert st[0] == np.float32(a) / np.float32(448) and st[1] == np.float32(448) / np.float32(a)
    q, xs = oracle.quantize_act_fp8(x, inv_s, oracle.PER_TENSOR_STATIC, st)
    xs_f = (x.astype(np.float32) * inv_s)
    want = oracle.fp8_encode(np.clip(xs_f * st[1], -448, 448))
    assert np.array_equal(q, want) and xs[0] == st[0]
    # per-token equals the row quantizer on the smoothed rows
    qd, xsd = oracle.quantize_act_fp8(x, inv_s)
    q2, s2 = oracle.quantize_rows_fp8(xs_f)
    assert np.array_equal(qd, q2) and np.array_equal(xsd, s2)
    # weights: columns smoothed, rows quantized
    w = (rng.standard_normal((16, 256)) * 0.03).astype(np.float16)
    s = (1.0 / inv_s).astype(np.float32)
    wq, ws = oracle.smooth_weights_fp8(w, s)
    q3, s3 = oracle.quantize_rows_fp8(w.astype(np.float32) * s)
    assert np.array_equal(wq, q3) and np.array_equal(ws, s3)
    # int8 static step from the same routine equals a2's
    s_o, inv_o, st8 = oracle.compute_scales(xa, oracle.absmax_cols(w), 0.5, static=True)
    assert np.array_equal(oracle.static_scale(xa, inv_o, 127.0), st8)


def test_gemm_fp8_exact_sum():
    rng = np.random.default_rng(3)
    M, N, K = 7, 9, 320
    xi = rng.integers(-16, 17, (M, K)).astype(np.float32)
    wi = rng.integers(-16, 17, (N, K)).astype(np.float32)
    xq, wq = oracle.fp8_encode(xi), oracle.fp8_encode(wi)
    assert np.array_equal(oracle.fp8_decode(xq), xi)
    xs = rng.uniform(0.01, 0.1, M).astype(np.float32)
    ws = rng.uniform(0.01, 0.1, N).astype(np.float32)
    y, acc = oracle.gemm_fp8_dequant(xq, wq, xs, ws)
    ref = xi.astype(np.float64) @ wi.astype(np.float64).T
    assert np.array_equal(acc, ref)
    c = xs[:, None] * ws[None, :]
    assert np.array_equal(y, acc.astype(np.float32) * c)
    # the sampled form gives the same values
    rows, cols = np.array([0, 3, 6]), np.array([8, 0, 4])
    y2, acc2 = oracle.gemm_fp8_dequant_at(xq, wq, xs, ws, rows, cols)
    assert np.array_equal(acc2, acc[rows, cols]) and np.array_equal(y2, y[rows, cols])
    # the largest and the smallest products together stay exact
    xq2 = np.array([[0x7E, 0x01, 0xFE, 0x01]], np.uint8)    # 448, 2^-9, -448, 2^-9
    wq2 = np.array([[0x7E, 0x01, 0x7E, 0x81]], np.uint8)    # 448, 2^-9, 448, -2^-9
    one = np.ones(1, np.float32)
    _, acc3 = oracle.gemm_fp8_dequant(xq2[:, :2], wq2[:, :2], one, one)
    assert acc3[0, 0] == 448.0 ** 2 + 2.0 ** -18 and acc3[0, 0] != 448.0 ** 2
    _, acc4 = oracle.gemm_fp8_dequant(xq2, wq2, one, one)
    assert acc4[0, 0] == 0.0
