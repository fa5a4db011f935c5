"""The library's calls captured into a HIP graph (through torch.cuda.graph)
replay to the same bits as the eager calls, replay after replay, with other
GPU work and synchronizations in between.  Nothing in the path uses a memset
node (zeroing is done by kernels), so every call is capturable.

Cases: the int8 layer a1 -> a5 (single_1024: per-tensor static step, fp32
out), the fused norm -> int8 with the e4m3 weights and GEMM, and
LLM.int8() with its workspace.
"""
import numpy as np
import pytest

import synth
import w8a8_post_quantization_amd as sq
from tests.gpu_util import dev, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t

    if not _t.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    sq.lib()
    return _t


def _replays_match(torch, run, n_replays=4):
    """run() -> list of output tensors.  Eager once, then captured; every
    replay (with unrelated work between) must equal the eager bits."""
    eager = [host(t, torch).copy() for t in run()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        outs = run()
    scratch = torch.empty(1 << 20, device="cuda")
    for r in range(n_replays):
        scratch.normal_()                     # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            got = host(o, torch)
            assert got.dtype == e.dtype and np.array_equal(got.view(np.uint8), e.view(np.uint8)), \
                f"replay {r}, output {i} differs from the eager run"


def test_graph_int8_layer(torch):
    cfg = synth.single_1024()
    X, W = dev(cfg["X"], torch), dev(cfg["W"], torch)

    def run():
        xa = sq.absmax_reduce(X)
        wa = sq.absmax_reduce(W)
        s, inv, st = sq.compute_scales(xa, wa, 0.5, static=True)
        wq, ws = sq.smooth_weights(W, s)
        xq, xs = sq.quantize_act(X, inv, sq.SQ_PER_TENSOR_STATIC, st)
        y = sq.gemm_i8_dequant(xq, wq, xs, ws, out_dtype=torch.float32)
        return [xa, wa, s, st, wq, ws, xq, xs, y]

    log("graph int8 layer")
    _replays_match(torch, run)


def test_graph_norm_and_fp8(torch):
    M, K, N = 256, 4096, 1024
    X = dev(synth.activations(3, 1, M, K, synth.choose(3, 3, K, 8), np.full(8, 30.0)), torch)
    W = dev(synth.weights(3, 2, N, K, 0.03), torch)
    g, b = synth.norm_params(K)
    g, b = dev(g, torch), dev(b, torch)

    def run():
        xa = sq.absmax_reduce(X)
        wa = sq.absmax_reduce(W)
        s, inv = sq.compute_scales(xa, wa, 0.5)
        g2, b2 = sq.fold_norm(g, s, b)
        xq, xs = sq.norm_quantize_act(X, g2, b2, sq.SQ_NORM_LAYER, 1e-5)
        wq8, ws8 = sq.smooth_weights_fp8(W, s)
        xq8, xs8 = sq.quantize_act_fp8(X, inv)
        y8 = sq.gemm_fp8_dequant(xq8, wq8, xs8, ws8, out_dtype=torch.bfloat16)
        return [g2, b2, xq, xs, wq8, xq8, y8]

    log("graph norm + fp8")
    _replays_match(torch, run)


def test_graph_llm_int8(torch):
    cfg = synth.llm_int8_2048(M=256, N=512, K=1024)
    X, W = dev(cfg["X"], torch), dev(cfg["W"], torch)
    wq, ws = sq.smooth_weights(W)
    ws_buf = torch.empty(sq.int8_mixed_matmul_workspace(256, 512, 1024), dtype=torch.uint8,
                         device="cuda")

    def run():
        y, cnt = sq.int8_mixed_matmul(X, wq, ws, W, 6.0, workspace=ws_buf, with_count=True)
        return [y, cnt]

    log("graph llm.int8")
    _replays_match(torch, run)
