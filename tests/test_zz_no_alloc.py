"""The allocation-free LLM.int8() entry point, sq_int8_mixed_matmul_noalloc
(intermediates in the library's per-GPU device array), against the
workspace form sq_int8_mixed_matmul, both called through the C ABI on the
same inputs: y, the int32 sums and |O| bit-identical, on two calls in a row,
the second with a smaller input (so it runs over the first call's leftovers
in the array).  Outputs are pre-filled with a pattern so unwritten elements
show."""
import ctypes

import numpy as np
import pytest

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


def test_noalloc_matches_workspace_form(torch):
    L = sq.lib()
    P = lambda t: t.data_ptr()  # noqa: E731
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cases = ((2048, 4096, 4096, 6, 5, torch.float16, sq.SQ_F16),
             (300, 520, 1040, 33, 11, torch.float32, sq.SQ_F32))
    for M, N, K, n_dims, seed, tdt, ydt in cases:
        log(f"noalloc LLM.int8() M={M} N={N} K={K} dims={n_dims}")
        cfg = synth.llm_int8_2048(M=M, N=N, K=K, seed=seed, n_dims=n_dims)
        X, W = dev(cfg["X"], torch), dev(cfg["W"], torch)
        wq, ws = sq.smooth_weights(W)
        need = L.sq_int8_mixed_matmul_workspace(M, N, K)
        work = torch.full((need,), 0x5A, dtype=torch.uint8, device="cuda")
        outs = []
        for form in ("workspace", "noalloc"):
            y = torch.full((M, N), float("nan"), dtype=tdt, device="cuda")
            acc = torch.full((M, N), -7, dtype=torch.int32, device="cuda")
            cnt = torch.full((1,), -1, dtype=torch.int32, device="cuda")
            if form == "workspace":
                rc = L.sq_int8_mixed_matmul(P(X), M, K, P(wq), P(ws), P(W), N, 6.0, P(work),
                                            need, P(y), ydt, P(acc), P(cnt), sp)
            else:
                rc = L.sq_int8_mixed_matmul_noalloc(P(X), M, K, P(wq), P(ws), P(W), N, 6.0,
                                                    P(y), ydt, P(acc), P(cnt), sp)
            assert rc == 0, L.sq_status_str(rc).decode()
            torch.cuda.synchronize()
            outs.append((host(y, torch), host(acc, torch), host(cnt, torch)))
        (y1, a1, c1), (y2, a2, c2) = outs
        assert int(c1[0]) == len(cfg["dims"]) and int(c2[0]) == int(c1[0])
        assert not np.isnan(y1.astype(np.float32)).any()
        assert_bits_equal(a2, a1, "int32 sums")
        assert_bits_equal(y2, y1, "y")
