"""The whole a1 -> a5 chain, and the e4m3 quantizers, on seeded random
shapes against the oracle.

The shapes are drawn from one generator seed per case so a failure names a
reproducible case. They span the decode kernel (M <= 32) and the tiled one,
K with and without a whole number of 128-byte stages, ragged M and N, and
every input type, activation mode and output type. Bars as everywhere: the
abs-max bit-exact; s, 1/s and the static step within 4 ulp; given the
oracle's scale tensors, the int8 codes, steps, int32 sums and narrowed
outputs bit-exact, and the e4m3 codes and steps bit-exact.
"""
import numpy as np
import pytest

import oracle
import synth
import w8a8_post_quantization_amd as sq
from tests.gpu_util import assert_bits_equal, dev, host, log, to_bf16_bits, ulp_dist

pytestmark = pytest.mark.gpu

N_CASES = 36


@pytest.fixture(scope="module")
def torch():
    import torch as _t

    if not _t.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    sq.lib()
    return _t


def _case(i):
    r = np.random.default_rng(9000 + i)
    M = int(r.integers(1, 33)) if i % 3 == 0 else int(r.integers(33, 700))
    N = int(r.integers(1, 800))
    K = 128 * int(r.integers(1, 24)) if i % 2 == 0 else 16 * int(r.integers(1, 190))
    return dict(M=M, N=N, K=K, dt=("f16", "bf16", "f32")[i % 3],
                static=bool(r.integers(0, 2)), ydt=("f32", "f16", "bf16")[int(r.integers(0, 3))],
                alpha=float(r.choice([0.3, 0.5, 0.6, 0.8])), n_out=int(r.integers(0, 5)),
                factor=float(r.uniform(5.0, 80.0)), seed=100 + i)


def _inputs(c):
    K = c["K"]
    n = min(c["n_out"], K)
    ch = synth.choose(c["seed"], 3, K, n) if n else np.zeros(0, np.int64)
    X = synth.activations(c["seed"], 1, c["M"], K, ch, np.full(n, c["factor"]), np.float32)
    W = synth.weights(c["seed"], 2, c["N"], K, 0.03, np.float32)
    if c["dt"] == "f16":
        return X.astype(np.float16), W.astype(np.float16)
    if c["dt"] == "bf16":
        return to_bf16_bits(X), to_bf16_bits(W)
    return X, W


@pytest.mark.parametrize("i", range(N_CASES))
def test_chain_random_shape(torch, i):
    c = _case(i)
    X, W = _inputs(c)
    log(f"random case {i}: {c}")
    xa = host(sq.absmax_reduce(dev(X, torch)), torch)
    wa = host(sq.absmax_reduce(dev(W, torch)), torch)
    xa_o, wa_o = oracle.absmax_cols(X), oracle.absmax_cols(W)
    assert_bits_equal(xa, xa_o, "x amax")
    assert_bits_equal(wa, wa_o, "w amax")
    got = sq.compute_scales(dev(xa_o, torch), dev(wa_o, torch), c["alpha"], static=c["static"])
    want = oracle.compute_scales(xa_o, wa_o, c["alpha"], static=c["static"])
    for g, w, name in zip(got, want, ("s", "inv_s", "static step")):
        assert ulp_dist(host(g, torch), w).max() <= 4, name
    s_o, inv_o = want[0], want[1]
    st_o = want[2] if c["static"] else None

    wq, ws = sq.smooth_weights(dev(W, torch), dev(s_o, torch))
    wq_o, ws_o = oracle.smooth_weights(W, s_o)
    assert_bits_equal(host(ws, torch), ws_o, "w_scale")
    assert_bits_equal(host(wq, torch), wq_o, "wq")

    mode = sq.SQ_PER_TENSOR_STATIC if c["static"] else sq.SQ_PER_TOKEN_DYNAMIC
    xq, xs = sq.quantize_act(dev(X, torch), dev(inv_o, torch), mode,
                             None if st_o is None else dev(st_o, torch))
    xq_o, xs_o = oracle.quantize_act(X, inv_o, mode, st_o)
    assert_bits_equal(host(xs, torch), xs_o, "x_scale")
    assert_bits_equal(host(xq, torch), xq_o, "xq")

    ydt = {"f32": oracle.F32, "f16": oracle.F16, "bf16": oracle.BF16}[c["ydt"]]
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[c["ydt"]]
    y, acc = sq.gemm_i8_dequant(xq, wq, xs, ws, out_dtype=tdt, with_acc=True)
    y_o, acc_o = oracle.gemm_i8_dequant(xq_o, wq_o, xs_o, ws_o, y_dt=ydt,
                                        per_row=int(xs_o.size > 1))
    assert_bits_equal(host(acc, torch), acc_o, "acc")
    assert_bits_equal(host(y, torch), y_o, "y")

    # the e4m3 quantizers on the same inputs and scales
    wq8, ws8 = sq.smooth_weights_fp8(dev(W, torch), dev(s_o, torch))
    wq8_o, ws8_o = oracle.smooth_weights_fp8(W, s_o)
    assert_bits_equal(host(ws8, torch), ws8_o, "w_scale e4m3")
    assert_bits_equal(host(wq8, torch), wq8_o, "wq e4m3")
    st8_o = oracle.static_scale(xa_o, inv_o, 448.0) if c["static"] else None
    xq8, xs8 = sq.quantize_act_fp8(dev(X, torch), dev(inv_o, torch), mode,
                                   None if st8_o is None else dev(st8_o, torch))
    xq8_o, xs8_o = oracle.quantize_act_fp8(X, inv_o, mode, st8_o)
    assert_bits_equal(host(xs8, torch), xs8_o, "x_scale e4m3")
    assert_bits_equal(host(xq8, torch), xq8_o, "xq e4m3")


N_MIXED = 16


def _mixed_case(i):
    r = np.random.default_rng(9500 + i)
    M = int(r.integers(1, 40)) if i % 4 == 0 else int(r.integers(40, 600))
    N = int(r.integers(1, 500))
    K = 128 * int(r.integers(1, 12)) if i % 2 == 0 else 16 * int(r.integers(1, 100))
    n_dims = int(r.choice([0, 1, 3, 6, 31, 32, 33, 40]))
    return dict(M=M, N=N, K=K, n_dims=min(n_dims, K), thr=float(r.choice([6.0, 6.0, 10.0])),
                ydt=("f16", "f32", "bf16")[i % 3], seed=200 + i)


@pytest.mark.parametrize("i", range(N_MIXED))
def test_mixed_random_shape(torch, i):
    """LLM.int8() (a6) on seeded random shapes: |O| from 0 to 40 planted
    dimensions (across the 32-column staging chunks), ragged M and N, K with
    and without whole 128-byte stages, every output type; |O| and y
    bit-exact against the oracle given the oracle's weight quantization."""
    c = _mixed_case(i)
    log(f"mixed random case {i}: {c}")
    cfg = synth.llm_int8_2048(M=c["M"], N=c["N"], K=c["K"], seed=c["seed"], n_dims=c["n_dims"])
    X, W = cfg["X"], cfg["W"]
    wq_o, ws_o = oracle.smooth_weights(W, None)
    ydt = {"f32": oracle.F32, "f16": oracle.F16, "bf16": oracle.BF16}[c["ydt"]]
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[c["ydt"]]
    y, cnt = sq.int8_mixed_matmul(dev(X, torch), dev(wq_o, torch), dev(ws_o, torch),
                                  dev(W, torch), c["thr"], out_dtype=tdt, with_count=True)
    r = oracle.int8_mixed_matmul(X, wq_o, ws_o, W, c["thr"], y_dt=ydt)
    assert int(host(cnt, torch)[0]) == r["idx"].size
    assert_bits_equal(host(y, torch), r["y"], "y")


N_TILED = 24


def _tiled_case(i):
    r = np.random.default_rng(9800 + i)
    M = int(r.integers(33, 700))
    N = int(r.integers(1, 800))
    K = 128 * int(r.integers(1, 28)) if i % 3 else 16 * int(r.integers(1, 200))
    return dict(M=M, N=N, K=K, tile=i % 4, ydt=("f32", "f16", "bf16")[int(r.integers(0, 3))],
                per_row=bool(r.integers(0, 4)), seed=300 + i)


@pytest.mark.parametrize("i", range(N_TILED))
def test_gemm_random_shape_every_tile(torch, i):
    """a5 on seeded random shapes with each tiled block shape forced in turn
    (256 x 256, 256 x 128, 128 x 128 and the 128 x 128 K-split pairs), K with
    and without whole 128-byte stages and with fewer stages than a ring holds:
    int32 sums and narrowed outputs bit-exact against the oracle."""
    c = _tiled_case(i)
    log(f"tiled random case {i}: {c}")
    r = np.random.default_rng(c["seed"])
    M, N, K = c["M"], c["N"], c["K"]
    xq = r.integers(-127, 128, (M, K), dtype=np.int8)
    wq = r.integers(-127, 128, (N, K), dtype=np.int8)
    xs = (r.random(M if c["per_row"] else 1) * 0.01 + 1e-3).astype(np.float32)
    ws = (r.random(N) * 0.001 + 1e-5).astype(np.float32)
    ydt = {"f32": oracle.F32, "f16": oracle.F16, "bf16": oracle.BF16}[c["ydt"]]
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[c["ydt"]]
    y, acc = sq.gemm_i8_dequant(dev(xq, torch), dev(wq, torch), dev(xs, torch), dev(ws, torch),
                                out_dtype=tdt, with_acc=True, tile=c["tile"])
    y_o, acc_o = oracle.gemm_i8_dequant(xq, wq, xs, ws, y_dt=ydt, per_row=int(c["per_row"]))
    assert_bits_equal(host(acc, torch), acc_o, "acc")
    assert_bits_equal(host(y, torch), y_o, "y")
