"""The measured-peak probes (include/sq_peaks.h) compute what they claim on
small inputs, so the rates the benchmark derives from them rest on kernels
that did the stated work: the read probe's per-block folds against numpy,
the 2:1 stream's output against numpy, and the MFMA loop's clock samples."""
import ctypes
import os

import numpy as np
import pytest

from tests.gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch

    from w8a8_post_quantization_amd import build as hip_build

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    if not os.path.exists(hip_build.PEAKS_LIB_PATH):
        pytest.fail("libsq_peaks.so is missing: build first")
    L = ctypes.CDLL(hip_build.PEAKS_LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.sqp_mfma_loop.argtypes = [i32, i32, i32, vp, vp, vp]
    L.sqp_read_stream.argtypes = [vp, sz, i32, vp, vp, vp]
    L.sqp_rw_stream.argtypes = [vp, sz, vp, i32, i32, vp, vp]
    return torch, L


def _sp(torch):
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def test_read_stream_folds(env):
    torch, L = env
    rng = np.random.default_rng(0)
    x = rng.integers(0, 2**32, size=(1 << 20) + 12, dtype=np.uint64).astype(np.uint32)  # ragged
    xd = torch.from_numpy(x.view(np.int32)).cuda()
    blocks = 7
    sink = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    log("peaks read stream")
    assert L.sqp_read_stream(xd.data_ptr(), x.nbytes, blocks, sink.data_ptr(), None,
                             _sp(torch)) == 0
    got = sink.cpu().numpy().view(np.uint32)
    # block b folds the 16-byte vectors i with (i // 256) % (4 * blocks) // 4 == b ... i.e.
    # the grid-stride walk: vector i belongs to block (i // 1024) % blocks
    v = x.reshape(-1, 4)
    fold = np.bitwise_xor.reduce(v, axis=1)
    owner = (np.arange(v.shape[0]) // 1024) % blocks
    want = np.array([np.bitwise_xor.reduce(fold[owner == b]) for b in range(blocks)],
                    dtype=np.uint32)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("nt", [0, 1])
def test_rw_stream_output(env, nt):
    torch, L = env
    rng = np.random.default_rng(1 + nt)
    x = rng.integers(0, 2**32, size=(300000 * 4), dtype=np.uint64).astype(np.uint32)
    xd = torch.from_numpy(x.view(np.int32)).cuda()
    y = torch.zeros(x.size // 2, dtype=torch.int32, device="cuda")
    clk = torch.zeros(4, dtype=torch.int64, device="cuda")
    log(f"peaks rw stream nt={nt}")
    assert L.sqp_rw_stream(xd.data_ptr(), x.nbytes, y.data_ptr(), 33, nt, clk.data_ptr(),
                           _sp(torch)) == 0
    v = x.reshape(-1, 4)
    want = np.stack([v[:, 0] ^ v[:, 1], v[:, 2] ^ v[:, 3]], axis=1).reshape(-1)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), want)
    c = clk.cpu().numpy()
    assert c[1] > c[0] and c[3] > c[2]


@pytest.mark.parametrize("fp8", [0, 1])
def test_mfma_loop_clocks(env, fp8):
    torch, L = env
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    clk = torch.zeros(4, dtype=torch.int64, device="cuda")
    log(f"peaks mfma loop fp8={fp8}")
    assert L.sqp_mfma_loop(fp8, 200, 8, sink.data_ptr(), clk.data_ptr(), _sp(torch)) == 0
    torch.cuda.synchronize()
    c = clk.cpu().numpy()
    assert c[1] > c[0] and c[3] > c[2]
    assert int(sink.cpu()[0]) == 0      # the impossible value was not reached
    # bad arguments are refused before any launch
    assert L.sqp_mfma_loop(fp8, 0, 8, sink.data_ptr(), None, _sp(torch)) != 0
