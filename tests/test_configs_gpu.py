"""GPU parity at the full sizes of the five workloads (and the 940 MB
activation stream the benchmark times), in the launch configurations the
benchmark uses, against the CPU oracle on the same seeded inputs.

Protocol: a1 outputs bit-exact; a2 within 4 ulp; a3..a6 are then fed the
oracle's s / 1/s / static step and must match bit for bit (int8 tensors,
per-row steps, int32 sums and the narrowed outputs).  The quantization error
against the fp64 product is printed, not gated.
"""
import numpy as np
import pytest

import oracle
import synth
import w8a8_post_quantization_amd as sq
from tests.gpu_util import assert_bits_equal, dev, host, log, ulp_dist

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t

    if not _t.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    sq.lib()
    return _t


def _stats(torch, X, W, alpha, static=False):
    """a1 on X and W and a2, checked; returns the oracle's scale tensors."""
    xa = host(sq.absmax_reduce(dev(X, torch)), torch)
    wa = host(sq.absmax_reduce(dev(W, torch)), torch)
    xa_o, wa_o = oracle.absmax_cols(X), oracle.absmax_cols(W)
    assert_bits_equal(xa, xa_o, "x amax")
    assert_bits_equal(wa, wa_o, "w amax")
    got = sq.compute_scales(dev(xa_o, torch), dev(wa_o, torch), alpha, static=static)
    want = oracle.compute_scales(xa_o, wa_o, alpha, static=static)
    for g, w, name in zip(got, want, ("s", "inv_s", "static")):
        assert ulp_dist(host(g, torch), w).max() <= 4, name
    return want


def _weights(torch, W, s):
    wq, ws = sq.smooth_weights(dev(W, torch), None if s is None else dev(s, torch))
    wq_o, ws_o = oracle.smooth_weights(W, s)
    assert_bits_equal(host(ws, torch), ws_o, "w_scale")
    assert_bits_equal(host(wq, torch), wq_o, "wq")
    return wq, ws, wq_o, ws_o


def _act(torch, X, inv, mode=sq.SQ_PER_TOKEN_DYNAMIC, st=None):
    xq, xs = sq.quantize_act(dev(X, torch), dev(inv, torch), mode,
                             None if st is None else dev(st, torch))
    xq_o, xs_o = oracle.quantize_act(X, inv, mode, st)
    assert_bits_equal(host(xs, torch), xs_o, "x_scale")
    assert_bits_equal(host(xq, torch), xq_o, "xq")
    return xq, xs, xq_o, xs_o


def _gemm(torch, xq, wq, xs, ws, xq_o, wq_o, xs_o, ws_o, ydt):
    tdt = {oracle.F32: torch.float32, oracle.F16: torch.float16, oracle.BF16: torch.bfloat16}[ydt]
    y, acc = sq.gemm_i8_dequant(xq, wq, xs, ws, out_dtype=tdt, with_acc=True)
    y_o, acc_o = oracle.gemm_i8_dequant(xq_o, wq_o, xs_o, ws_o, y_dt=ydt,
                                        per_row=int(xs_o.size > 1))
    assert_bits_equal(host(acc, torch), acc_o, "acc")
    assert_bits_equal(host(y, torch), y_o, "y")
    return y_o


def _rel_err(y, X, W):
    y = y.astype(np.float32) if y.dtype != np.uint16 else (
        y.astype(np.uint32) << 16).view(np.float32)
    ref = oracle.matmul_f64(X, W)
    return float(np.linalg.norm(y - ref) / np.linalg.norm(ref))


def test_single_1024(torch):
    """X fp32 [16,1024] (channel 0 x50), W fp32 [1024,1024], alpha 0.5,
    per-tensor static X, per-channel W, fp32 out."""
    cfg = synth.single_1024()
    X, W = cfg["X"], cfg["W"]
    log("single_1024")
    s_o, inv_o, st_o = _stats(torch, X, W, 0.5, static=True)
    wq, ws, wq_o, ws_o = _weights(torch, W, s_o)
    xq, xs, xq_o, xs_o = _act(torch, X, inv_o, sq.SQ_PER_TENSOR_STATIC, st_o)
    y_o = _gemm(torch, xq, wq, xs, ws, xq_o, wq_o, xs_o, ws_o, oracle.F32)
    # unsmoothed reference for the error report
    xq_u, xs_u = oracle.quantize_act(X, None, oracle.PER_TENSOR_STATIC,
                                     np.array([np.abs(X).max() / 127, 127 / np.abs(X).max()],
                                              np.float32))
    wq_u, ws_u = oracle.smooth_weights(W, None)
    y_u, _ = oracle.gemm_i8_dequant(xq_u, wq_u, xs_u, ws_u)
    print(f"\nsingle_1024 rel. error vs fp64: smoothed {_rel_err(y_o, X, W):.4f}, "
          f"unsmoothed {_rel_err(y_u, X, W):.4f}")


def test_prefill_30b(torch):
    """X fp16 [256,7168] (6 channels x U(20,100)), W fp16 [28672,7168],
    alpha 0.5, per-token X, bf16 out - full size, every output compared."""
    cfg = synth.prefill_30b()
    X, W = cfg["X"], cfg["W"]
    log("prefill_30b stats")
    s_o, inv_o = _stats(torch, X, W, 0.5)
    log("prefill_30b weights")
    wq, ws, wq_o, ws_o = _weights(torch, W, s_o)
    log("prefill_30b activations")
    xq, xs, xq_o, xs_o = _act(torch, X, inv_o)
    log("prefill_30b gemm")
    _gemm(torch, xq, wq, xs, ws, xq_o, wq_o, xs_o, ws_o, oracle.BF16)


@pytest.mark.parametrize("alpha", [0.4, 0.5, 0.6])
def test_decoder_1024(torch, alpha):
    """Hidden-1024 decoder GEMM set at M = 4096, fp16 out."""
    cfg = synth.decoder_1024()
    for name, N, K in synth.DECODER_1024_WEIGHTS:
        X = cfg[f"X{K}"]
        W = cfg["W"][name]
        log(f"decoder_1024 alpha={alpha} {name} [{N},{K}]")
        s_o, inv_o = _stats(torch, X, W, alpha)
        wq, ws, wq_o, ws_o = _weights(torch, W, s_o)
        xq, xs, xq_o, xs_o = _act(torch, X, inv_o)
        _gemm(torch, xq, wq, xs, ws, xq_o, wq_o, xs_o, ws_o, oracle.F16)


def test_decode_8192(torch):
    """Calibrate on X_cal [512,8192], quantize W [28672,8192], then decode
    GEMMs at M = 1, 8, 16, 32 with per-token X and fp16 out (decode kernel)."""
    cfg = synth.decode_8192(32)
    W = cfg["W"]
    log("decode_8192 stats")
    s_o, inv_o = _stats(torch, cfg["X_cal"], W, 0.5)
    wq, ws, wq_o, ws_o = _weights(torch, W, s_o)
    for M in (1, 8, 16, 32):
        X = cfg["X"][:M]
        log(f"decode_8192 M={M}")
        xq, xs, xq_o, xs_o = _act(torch, X, inv_o)
        _gemm(torch, xq, wq, xs, ws, xq_o, wq_o, xs_o, ws_o, oracle.F16)


def test_llm_int8_2048(torch):
    """LLM.int8(): X fp16 [2048,4096] with 6 planted dims, W [4096,4096],
    threshold 6, fp16 out."""
    cfg = synth.llm_int8_2048()
    X, W = cfg["X"], cfg["W"]
    log("llm_int8_2048")
    wq, ws, wq_o, ws_o = _weights(torch, W, None)
    M, K = X.shape
    N = W.shape[0]
    work = torch.full((sq.int8_mixed_matmul_workspace(M, N, K),), 0xA5, dtype=torch.uint8,
                      device="cuda")
    y, acc, cnt = sq.int8_mixed_matmul(dev(X, torch), wq, ws, dev(W, torch), 6.0,
                                       workspace=work, with_count=True, with_acc=True)
    r = oracle.int8_mixed_matmul(X, wq_o, ws_o, W, 6.0)
    assert list(r["idx"]) == list(cfg["dims"])
    assert int(host(cnt, torch)[0]) == 6
    # the intermediates of the decomposition ([INT8-expl] §2.2), from the
    # workspace's documented layout: O, X~q, the row steps, the column
    # maxima and mask, the side operands (x and w in the outlier columns,
    # fp32), and the int32 sums of the int8 part
    wb = host(work, torch)
    off = sq.int8_mixed_workspace_parts(M, N, K)
    assert work.numel() == off["total"]
    n_o = int(wb[off["count"]:off["count"] + 4].view(np.int32)[0])
    assert n_o == 6
    assert_bits_equal(wb[off["idx"]:off["idx"] + 4 * n_o].view(np.int32), r["idx"], "O list")
    assert_bits_equal(wb[off["xq"]:off["xq"] + M * K].view(np.int8).reshape(M, K), r["xq"],
                      "X~q")
    assert_bits_equal(wb[off["x_scale"]:off["x_scale"] + 4 * M].view(np.float32), r["x_scale"],
                      "row steps")
    assert_bits_equal(wb[off["colmax"]:off["colmax"] + 4 * K].view(np.float32),
                      oracle.absmax_cols(X), "column maxima")
    mask = np.ones(K, np.float32)
    mask[r["idx"]] = 0.0
    assert_bits_equal(wb[off["mask"]:off["mask"] + 4 * K].view(np.float32), mask, "column mask")
    xs_side = wb[off["x_side"]:off["x_side"] + 4 * n_o * M].view(np.float32).reshape(n_o, M)
    ws_side = wb[off["w_side"]:off["w_side"] + 4 * n_o * N].view(np.float32).reshape(n_o, N)
    assert_bits_equal(xs_side, X[:, r["idx"]].T.astype(np.float32), "side activations")
    assert_bits_equal(ws_side, W[:, r["idx"]].T.astype(np.float32), "side weights")
    assert_bits_equal(host(acc, torch), r["acc"], "acc")
    assert_bits_equal(host(y, torch), r["y"], "y")
    print(f"\nllm_int8_2048 rel. error vs fp64: {_rel_err(r['y'], X, W):.5f}")


def test_activation_stream(torch):
    """The 940 MB activation stream the benchmark times (X fp16
    [65536,7168]): a1, and a4 per-token and static, int8 and e4m3, against
    the oracle."""
    cfg = synth.stream_act()
    X = cfg["X"]
    inv = (1.0 / (oracle.absmax_cols(X[:1024]) + 1.0)).astype(np.float32)
    log("stream a1")
    assert_bits_equal(host(sq.absmax_reduce(dev(X, torch)), torch), oracle.absmax_cols(X),
                      "amax")
    log("stream a4")
    _act(torch, X, inv)
    # codes beyond the last-level cache size are stored nontemporally: the
    # static int8 form and both e4m3 forms of that store path as well
    log("stream a4 static")
    st = oracle.static_scale(oracle.absmax_cols(X), inv, 127.0)
    _act(torch, X, inv, sq.SQ_PER_TENSOR_STATIC, st)
    log("stream a4 e4m3 per-token")
    xq8, xs8 = sq.quantize_act_fp8(dev(X, torch), dev(inv, torch))
    xq8_o, xs8_o = oracle.quantize_act_fp8(X, inv)
    assert_bits_equal(host(xs8, torch), xs8_o, "x_scale e4m3")
    assert_bits_equal(host(xq8, torch), xq8_o, "xq e4m3")
    # the fused LayerNorm -> int8 (beta, per token) the benchmark times on
    # this stream: 65536 rows, one wave per row, gamma and beta in LDS
    log("stream fused norm -> int8")
    g, b = synth.norm_params(X.shape[1])
    xqn, xsn = sq.norm_quantize_act(dev(X, torch), dev(g, torch), dev(b, torch),
                                    sq.SQ_NORM_LAYER, 1e-5, sq.SQ_PER_TOKEN_DYNAMIC)
    xqn_o, xsn_o = oracle.norm_quantize(X, g, b, oracle.NORM_LAYER, 1e-5,
                                        oracle.PER_TOKEN_DYNAMIC, None)
    assert_bits_equal(host(xsn, torch), xsn_o, "x_scale (norm)")
    assert_bits_equal(host(xqn, torch), xqn_o, "xq (norm)")
    del xqn, xsn, xqn_o
    log("stream a4 e4m3 static")
    st8 = oracle.static_scale(oracle.absmax_cols(X), inv, 448.0)
    xq8, xs8 = sq.quantize_act_fp8(dev(X, torch), dev(inv, torch), sq.SQ_PER_TENSOR_STATIC,
                                   dev(st8, torch))
    xq8_o, xs8_o = oracle.quantize_act_fp8(X, inv, oracle.PER_TENSOR_STATIC, st8)
    assert_bits_equal(host(xs8, torch), xs8_o, "x_scale e4m3 static")
    assert_bits_equal(host(xq8, torch), xq8_o, "xq e4m3 static")
