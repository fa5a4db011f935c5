"""Guard bytes around every output: each kernel writes into the middle of a
buffer filled with a sentinel byte, on ragged and tile-edge shapes (every
forced GEMM block shape, decode row counts, K tails); after the call the
bytes before and after the output must still hold the sentinel, and the
output itself must equal the same call's into a plain tensor.  A write past
either end of an output (a missed bound on a ragged edge) fails here even
when it lands in memory the other tests never read."""
import ctypes

import numpy as np
import pytest

import synth
import w8a8_post_quantization_amd as sq
from tests.gpu_util import assert_bits_equal, dev, host, log

pytestmark = pytest.mark.gpu

GUARD = 4096      # bytes on each side
SENT = 0xA5


@pytest.fixture(scope="module")
def torch():
    import torch as _t

    if not _t.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    sq.lib()
    return _t


class Guarded:
    """An output of `nbytes` inside a sentinel-filled buffer."""

    def __init__(self, torch, nbytes):
        self.n = nbytes
        self.buf = torch.full((GUARD + max(nbytes, 1) + GUARD,), SENT, dtype=torch.uint8,
                              device="cuda")
        self.ptr = self.buf.data_ptr() + GUARD

    def check(self, torch, what):
        h = host(self.buf, torch)
        pre, post = h[:GUARD], h[GUARD + self.n:]
        bad_pre = np.nonzero(pre != SENT)[0]
        bad_post = np.nonzero(post != SENT)[0]
        assert bad_pre.size == 0, f"{what}: {bad_pre.size} guard bytes before the output changed"
        assert bad_post.size == 0, (f"{what}: {bad_post.size} guard bytes after the output "
                                    f"changed (first at +{bad_post[0]})")
        return h[GUARD:GUARD + self.n]


def _stream(torch):
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("M,N,K,tile,ydt", [
    (1, 37, 144, None, sq.SQ_F16), (7, 129, 1040, None, sq.SQ_F32), (17, 300, 256, None, sq.SQ_BF16),
    (32, 113, 4096, None, sq.SQ_F16), (33, 127, 128, 0, sq.SQ_F32), (257, 129, 1024, 0, sq.SQ_F16),
    (200, 300, 2048, 1, sq.SQ_BF16), (255, 257, 144, 1, sq.SQ_F32), (129, 131, 512, 2, sq.SQ_F16),
    (300, 70, 1040, 2, sq.SQ_BF16), (129, 131, 512, 3, sq.SQ_F16), (300, 70, 2304, 3, sq.SQ_BF16),
    (257, 255, 1040, 3, sq.SQ_F32)])
def test_gemm_guards(torch, M, N, K, tile, ydt):
    L = sq.lib()
    rng = np.random.default_rng(M * 7 + N + K)
    xq = dev(rng.integers(-127, 128, (M, K), dtype=np.int8), torch)
    wq = dev(rng.integers(-127, 128, (N, K), dtype=np.int8), torch)
    xs = dev((rng.random(M) * 0.01 + 1e-3).astype(np.float32), torch)
    ws = dev((rng.random(N) * 0.001 + 1e-5).astype(np.float32), torch)
    esz = 4 if ydt == sq.SQ_F32 else 2
    gy, ga = Guarded(torch, M * N * esz), Guarded(torch, M * N * 4)
    log(f"guards gemm M={M} N={N} K={K} tile={tile} y={ydt}")
    t = -1 if tile is None else tile
    rc = L.sq_gemm_i8_dequant_tile(xq.data_ptr(), wq.data_ptr(), M, N, K, xs.data_ptr(), 1,
                                   ws.data_ptr(), gy.ptr, ydt, ga.ptr, _stream(torch), t)
    assert rc == 0
    y_bytes, acc_bytes = gy.check(torch, "y"), ga.check(torch, "acc")
    tdt = {sq.SQ_F32: torch.float32, sq.SQ_F16: torch.float16, sq.SQ_BF16: torch.bfloat16}[ydt]
    y, acc = sq.gemm_i8_dequant(xq, wq, xs, ws, out_dtype=tdt, with_acc=True, tile=tile)
    assert_bits_equal(acc_bytes.view(np.int32).reshape(M, N), host(acc, torch), "acc")
    assert np.array_equal(y_bytes, host(y, torch).view(np.uint8).reshape(-1)), "y"


@pytest.mark.parametrize("M,N,K,tile", [(33, 127, 256, 0), (300, 129, 1152, 2), (5, 70, 128, None)])
def test_gemm_fp8_guards(torch, M, N, K, tile):
    L = sq.lib()
    rng = np.random.default_rng(M + N * 3 + K)
    xq = dev((rng.integers(0, 0x7E, (M, K)) | (rng.integers(0, 2, (M, K)) << 7)).astype(np.uint8),
             torch)
    wq = dev((rng.integers(0, 0x7E, (N, K)) | (rng.integers(0, 2, (N, K)) << 7)).astype(np.uint8),
             torch)
    xs = dev((rng.random(M) * 0.01 + 1e-3).astype(np.float32), torch)
    ws = dev((rng.random(N) * 0.001 + 1e-5).astype(np.float32), torch)
    gy = Guarded(torch, M * N * 4)
    log(f"guards gemm fp8 M={M} N={N} K={K} tile={tile}")
    rc = L.sq_gemm_fp8_dequant_tile(xq.data_ptr(), wq.data_ptr(), M, N, K, xs.data_ptr(), 1,
                                    ws.data_ptr(), gy.ptr, sq.SQ_F32, _stream(torch),
                                    -1 if tile is None else tile)
    assert rc == 0
    got = gy.check(torch, "y fp8")
    y = sq.gemm_fp8_dequant(xq, wq, xs, ws, out_dtype=torch.float32, tile=tile)
    assert np.array_equal(got, host(y, torch).view(np.uint8).reshape(-1)), "y fp8"


@pytest.mark.parametrize("rows,K,dt", [(1, 16, "f32"), (37, 1040, "f16"), (2049, 144, "bf16"),
                                       (3, 16400, "f16"), (600, 2064, "f32")])
def test_quantizer_and_absmax_guards(torch, rows, K, dt):
    """a1 (fresh and running max), a3 with and without s, a4 per-token and
    static, and the e4m3 forms."""
    L = sq.lib()
    a = synth.normal(rows + K, 1, (rows, K))
    code = {"f32": sq.SQ_F32, "f16": sq.SQ_F16, "bf16": sq.SQ_BF16}[dt]
    if dt == "f16":
        a = a.astype(np.float16)
    elif dt == "bf16":
        a = ((a.view(np.uint32) + 0x7FFF + ((a.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)
    x = dev(a, torch)
    s = dev((np.abs(synth.normal(rows, 2, (K,))) + 0.1).astype(np.float32), torch)
    st = dev(np.array([0.01, 100.0], np.float32), torch)
    sp = _stream(torch)
    log(f"guards quantizers rows={rows} K={K} {dt}")
    for acc in (0, 1):
        g = Guarded(torch, 4 * K)
        if acc:
            torch.cuda.synchronize()
            g.buf[GUARD:GUARD + 4 * K] = 0   # running max from zero
        assert L.sq_absmax_reduce(x.data_ptr(), code, rows, K, acc, g.ptr, sp) == 0
        g.check(torch, f"amax (accumulate={acc})")
    for sv in (None, s):
        gq, gs = Guarded(torch, rows * K), Guarded(torch, 4 * rows)
        assert L.sq_smooth_weights(x.data_ptr(), code, rows, K, None if sv is None else sv.data_ptr(),
                                   gq.ptr, gs.ptr, sp) == 0
        gq.check(torch, "wq")
        gs.check(torch, "w_scale")
        gq, gs = Guarded(torch, rows * K), Guarded(torch, 4 * rows)
        assert L.sq_smooth_weights_fp8(x.data_ptr(), code, rows, K,
                                       None if sv is None else sv.data_ptr(), gq.ptr, gs.ptr,
                                       sp) == 0
        gq.check(torch, "wq e4m3")
        gs.check(torch, "w_scale e4m3")
    for mode in (sq.SQ_PER_TOKEN_DYNAMIC, sq.SQ_PER_TENSOR_STATIC):
        ns = rows if mode == sq.SQ_PER_TOKEN_DYNAMIC else 1
        for fn in (L.sq_quantize_act, L.sq_quantize_act_fp8):
            gq, gs = Guarded(torch, rows * K), Guarded(torch, 4 * ns)
            assert fn(x.data_ptr(), code, rows, K, s.data_ptr(), mode, st.data_ptr(), gq.ptr,
                      gs.ptr, sp) == 0
            gq.check(torch, f"xq mode={mode}")
            gs.check(torch, f"x_scale mode={mode}")


@pytest.mark.parametrize("M,K,norm,beta", [(1, 16, 0, True), (33, 2064, 1, False),
                                           (2051, 48, 0, True), (2050, 8208, 1, True)])
def test_norm_guards(torch, M, K, norm, beta):
    L = sq.lib()
    x = dev((synth.normal(M, K, (M, K)) * 2).astype(np.float16), torch)
    g, b = synth.norm_params(K)
    gd, bd = dev(g, torch), dev(b, torch) if beta else None
    s = dev((np.abs(synth.normal(K, 3, (K,))) + 0.1).astype(np.float32), torch)
    sp = _stream(torch)
    log(f"guards norm M={M} K={K}")
    gg, gb = Guarded(torch, 4 * K), Guarded(torch, 4 * K)
    assert L.sq_fold_norm(gd.data_ptr(), None if bd is None else bd.data_ptr(), s.data_ptr(), K,
                          gg.ptr, gb.ptr if beta else None, sp) == 0
    gg.check(torch, "gamma'")
    gb.check(torch, "beta'")
    for mode in (sq.SQ_PER_TOKEN_DYNAMIC, sq.SQ_PER_TENSOR_STATIC):
        st = dev(np.array([0.02, 50.0], np.float32), torch)
        ns = M if mode == sq.SQ_PER_TOKEN_DYNAMIC else 1
        gq, gs = Guarded(torch, M * K), Guarded(torch, 4 * ns)
        assert L.sq_norm_quantize_act(x.data_ptr(), sq.SQ_F16, M, K, norm, gd.data_ptr(),
                                      None if bd is None else bd.data_ptr(), 1e-5, mode,
                                      st.data_ptr(), gq.ptr, gs.ptr, sp) == 0
        gq.check(torch, f"norm xq mode={mode}")
        gs.check(torch, f"norm x_scale mode={mode}")


@pytest.mark.parametrize("M,N,K,n_dims,tile", [(33, 70, 144, 3, None), (300, 129, 1040, 33, 2),
                                               (257, 300, 512, 6, 1), (5, 40, 2048, 1, None)])
def test_mixed_guards(torch, M, N, K, n_dims, tile):
    """LLM.int8(): y, the int32 sums, |O| and the workspace itself."""
    L = sq.lib()
    cfg = synth.llm_int8_2048(M=M, N=N, K=K, seed=M + N, n_dims=n_dims)
    X, W = dev(cfg["X"], torch), dev(cfg["W"], torch)
    wq, ws = sq.smooth_weights(W)
    need = L.sq_int8_mixed_matmul_workspace(M, N, K)
    gw = Guarded(torch, need)
    gy, ga, gc = Guarded(torch, M * N * 2), Guarded(torch, M * N * 4), Guarded(torch, 4)
    log(f"guards mixed M={M} N={N} K={K} dims={n_dims} tile={tile}")
    rc = L.sq_int8_mixed_matmul_tile(X.data_ptr(), M, K, wq.data_ptr(), ws.data_ptr(),
                                     W.data_ptr(), N, 6.0, gw.ptr, need, gy.ptr, sq.SQ_F16,
                                     ga.ptr, gc.ptr, _stream(torch), -1 if tile is None else tile)
    assert rc == 0
    gw.check(torch, "workspace")
    y_bytes, acc_bytes = gy.check(torch, "y"), ga.check(torch, "acc")
    assert int(gc.check(torch, "|O|").view(np.int32)[0]) == len(cfg["dims"])
    y, acc = sq.int8_mixed_matmul(X, wq, ws, W, 6.0, with_acc=True, tile=tile)
    assert_bits_equal(acc_bytes.view(np.int32).reshape(M, N), host(acc, torch), "acc")
    assert np.array_equal(y_bytes, host(y, torch).view(np.uint8).reshape(-1)), "y"
