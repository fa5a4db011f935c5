"""The C-ABI library loads on a machine without a GPU, exports every function
include/sq.h declares, and rejects bad arguments on the host before any
launch (so every error path is testable here).  No kernel is launched."""
import ctypes
import os

import pytest

import w8a8_post_quantization_amd as sq

pytestmark = pytest.mark.skipif(not os.path.exists(sq.LIB_PATH),
                                reason="libsq.so not built (run __graft_entry__.build())")

OK, NULL, SHAPE, DTYPE, ALIGN, ARG, WORKSPACE, UNSUP, HIP = range(9)
FAKE = 0x100000  # a 256-aligned non-null address; never dereferenced on these paths


def test_exports_every_declared_symbol():
    L = sq.lib()
    declared = sq.header_functions()
    assert len(declared) == 17
    for name in declared:
        assert hasattr(L, name), name
        assert name in sq.SIGNATURES, name
    assert L.sq_version() == 103
    test_only = sq.header_functions(sq.TEST_HEADER)
    assert test_only == ["sq_gemm_fp8_dequant_tile", "sq_gemm_i8_dequant_tile",
                         "sq_int8_mixed_matmul_tile", "sq_norm_quantize_act_kernel"]
    for name in test_only:
        assert hasattr(L, name) and name in sq.SIGNATURES, name


def test_forced_tile_is_checked():
    L = sq.lib()
    for bad in (-2, 3, 99):
        assert L.sq_gemm_i8_dequant_tile(FAKE, FAKE, 64, 64, 128, FAKE, 1, FAKE, FAKE,
                                         sq.SQ_F32, None, None, bad if bad != 3 else 4) == ARG
        assert L.sq_gemm_fp8_dequant_tile(FAKE, FAKE, 64, 64, 128, FAKE, 1, FAKE, FAKE,
                                          sq.SQ_F32, None, bad) == ARG
        assert L.sq_int8_mixed_matmul_tile(FAKE, 64, 128, FAKE, FAKE, FAKE, 64, 6.0, FAKE, 1 << 20,
                                           FAKE, sq.SQ_F16, None, None, None, bad) == ARG
        assert L.sq_norm_quantize_act_kernel(FAKE, sq.SQ_F16, 64, 512, 0, FAKE, None, 1e-5, 1,
                                             None, FAKE, FAKE, None, bad) == ARG
    assert L.sq_gemm_i8_dequant_tile(FAKE, FAKE, 64, 64, 40, FAKE, 1, FAKE, FAKE, sq.SQ_F32,
                                     None, None, 1) == SHAPE
    assert L.sq_norm_quantize_act_kernel(FAKE, sq.SQ_F16, 64, 40, 0, FAKE, None, 1e-5, 1,
                                         None, FAKE, FAKE, None, 1) == SHAPE


def test_status_strings():
    L = sq.lib()
    for code in range(9):
        assert L.sq_status_str(code).decode().startswith("SQ_")
    assert b"unknown" in L.sq_status_str(42)


def test_absmax_validation():
    L = sq.lib()
    assert L.sq_absmax_reduce(FAKE, 7, 4, 16, 0, FAKE, None) == DTYPE
    assert L.sq_absmax_reduce(FAKE, sq.SQ_F16, -1, 16, 0, FAKE, None) == SHAPE
    assert L.sq_absmax_reduce(FAKE, sq.SQ_F16, 4, 12, 0, FAKE, None) == SHAPE   # 24 B rows
    assert L.sq_absmax_reduce(FAKE, sq.SQ_F32, 4, 6, 0, FAKE, None) == SHAPE
    assert L.sq_absmax_reduce(None, sq.SQ_F16, 4, 16, 0, FAKE, None) == NULL
    assert L.sq_absmax_reduce(FAKE, sq.SQ_F16, 4, 16, 0, None, None) == NULL
    assert L.sq_absmax_reduce(FAKE + 8, sq.SQ_F16, 4, 16, 0, FAKE, None) == ALIGN
    assert L.sq_absmax_reduce(None, sq.SQ_F16, 4, 0, 0, None, None) == OK       # no columns


def test_scales_validation():
    L = sq.lib()
    for bad in (-0.1, 1.5, float("nan")):
        assert L.sq_compute_scales(FAKE, FAKE, 8, bad, FAKE, FAKE, None, None) == ARG
    assert L.sq_compute_scales(FAKE, FAKE, -1, 0.5, FAKE, FAKE, None, None) == SHAPE
    assert L.sq_compute_scales(None, FAKE, 8, 0.5, FAKE, FAKE, None, None) == NULL
    assert L.sq_compute_scales(FAKE, FAKE, 8, 0.5, FAKE + 2, FAKE, None, None) == ALIGN
    assert L.sq_compute_scales(None, None, 0, 0.5, None, None, None, None) == OK


def test_smooth_and_quantize_validation():
    L = sq.lib()
    assert L.sq_smooth_weights(FAKE, sq.SQ_F16, 8, 24, None, FAKE, FAKE, None) == SHAPE
    assert L.sq_smooth_weights(FAKE, 5, 8, 32, None, FAKE, FAKE, None) == DTYPE
    assert L.sq_smooth_weights(None, sq.SQ_F16, 8, 32, None, FAKE, FAKE, None) == NULL
    assert L.sq_smooth_weights(FAKE, sq.SQ_F16, 8, 32, FAKE + 4, FAKE, FAKE, None) == ALIGN
    assert L.sq_smooth_weights(None, sq.SQ_F16, 0, 32, None, None, None, None) == OK
    f = L.sq_smooth_weights_folded
    assert f(FAKE, sq.SQ_F16, 8, 24, FAKE, None, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, 5, 8, 32, FAKE, None, FAKE, FAKE, None) == DTYPE
    assert f(FAKE, sq.SQ_F16, 8, 32, FAKE, None, None, FAKE, None) == NULL
    assert f(FAKE, sq.SQ_F16, 8, 32, FAKE + 2, None, FAKE, FAKE, None) == ALIGN   # row_mul
    assert f(FAKE, sq.SQ_F16, 8, 32, FAKE, FAKE + 4, FAKE, FAKE, None) == ALIGN   # s
    assert f(None, sq.SQ_F16, 0, 32, None, None, None, None, None) == OK
    assert L.sq_quantize_act(FAKE, sq.SQ_F16, 8, 32, None, 3, None, FAKE, FAKE, None) == ARG
    assert L.sq_quantize_act(FAKE, sq.SQ_F16, 8, 32, None, sq.SQ_PER_TENSOR_STATIC, None,
                             FAKE, FAKE, None) == NULL
    assert L.sq_quantize_act(FAKE, sq.SQ_F16, 8, 33, None, 1, None, FAKE, FAKE, None) == SHAPE
    assert L.sq_quantize_act(FAKE, sq.SQ_F16, 8, 32, None, 1, None, FAKE + 1, FAKE, None) == ALIGN
    assert L.sq_quantize_act(None, sq.SQ_F16, 0, 32, None, 1, None, None, FAKE, None) == OK


def test_gemm_validation():
    L = sq.lib()
    args = dict(xq=FAKE, wq=FAKE, M=4, N=4, K=32, xs=FAKE, per_row=1, ws=FAKE, y=FAKE,
                y_dt=sq.SQ_F32, acc=None)

    def call(**kw):
        a = {**args, **kw}
        return L.sq_gemm_i8_dequant(a["xq"], a["wq"], a["M"], a["N"], a["K"], a["xs"],
                                    a["per_row"], a["ws"], a["y"], a["y_dt"], a["acc"], None)

    assert call(y_dt=9) == DTYPE
    assert call(K=40) == SHAPE
    assert call(M=-1) == SHAPE
    assert call(K=133152) == UNSUP
    assert call(xq=None) == NULL
    assert call(y=None) == NULL
    assert call(wq=FAKE + 8) == ALIGN
    assert call(y=FAKE + 2, y_dt=sq.SQ_F32) == ALIGN
    assert call(M=0, xq=None, y=None) == OK
    assert call(N=0) == OK


def test_mixed_validation():
    L = sq.lib()
    need = L.sq_int8_mixed_matmul_workspace(2048, 4096, 4096)
    assert need >= 2048 * 4096 + 2048 * 4 + 3 * 4096 * 4
    assert need % 256 == 0
    # the documented layout: parts back to back, 256-byte rounded, the side
    # operands sized for min(K, SQ_MIXED_SIDE_COLS) columns
    for M, N, K in ((2048, 4096, 4096), (1, 1, 16), (300, 520, 1040), (7, 3, 64)):
        assert L.sq_int8_mixed_matmul_workspace(M, N, K) == \
            sq.int8_mixed_workspace_parts(M, N, K)["total"]
    assert sq.int8_mixed_workspace_parts(7, 3, 64)["side_cols"] == 64
    assert sq.int8_mixed_workspace_parts(7, 3, 4096)["side_cols"] == 128

    def call(thr=6.0, ws=FAKE, wsb=need, K=4096, x=FAKE):
        return L.sq_int8_mixed_matmul(x, 2048, K, FAKE, FAKE, FAKE, 4096, thr, ws, wsb, FAKE,
                                      sq.SQ_F16, None, None, None)

    assert call(thr=0.0) == ARG
    assert call(thr=-1.0) == ARG
    assert call(thr=float("nan")) == ARG
    assert call(ws=None) == WORKSPACE
    assert call(wsb=need - 1) == WORKSPACE
    assert call(ws=FAKE + 16) == ALIGN
    assert call(K=4100) == SHAPE
    assert call(x=None) == NULL


def test_mixed_noalloc_validation():
    """The allocation-free LLM.int8() entry point checks its arguments as the
    workspace form does, and rejects shapes whose intermediates exceed its
    per-GPU array, all on the host (no device call on these paths)."""
    L = sq.lib()
    f = L.sq_int8_mixed_matmul_noalloc
    cap = 32 << 20   # SQ_MIXED_SCRATCH_BYTES

    def call(M=2048, K=4096, N=4096, thr=6.0, x=FAKE, y=FAKE, ydt=sq.SQ_F16, acc=None):
        return f(x, M, K, FAKE, FAKE, FAKE, N, thr, y, ydt, acc, None, None)

    assert call(thr=0.0) == ARG
    assert call(thr=float("nan")) == ARG
    assert call(K=4100) == SHAPE
    assert call(K=0) == SHAPE
    assert call(x=None) == NULL
    assert call(y=FAKE + 1) == ALIGN
    assert call(acc=FAKE + 2) == ALIGN
    assert call(ydt=7) == DTYPE
    assert call(M=0, x=None, y=None) == OK
    assert call(M=8192, K=8192) == WORKSPACE              # 64 MiB of int8 rows alone
    # the largest M for N = K = 4096 that fits, and one row more
    M = 1
    while L.sq_int8_mixed_matmul_workspace(M + 1, 4096, 4096) <= cap:
        M += 1
    assert L.sq_int8_mixed_matmul_workspace(M, 4096, 4096) <= cap < \
        L.sq_int8_mixed_matmul_workspace(M + 1, 4096, 4096)
    assert call(M=M + 1, K=4096) == WORKSPACE
    assert M == 6810   # the 2048-row LLM.int8() workload fits with room


def test_zero_length_rows_are_rejected_before_any_pointer_is_used():
    """K == 0 with at least one row (or output): every entry point returns
    SQ_ERR_SHAPE with NULL operands, so no kernel ever sees a row of no
    elements (whose clamped tail loads would point before the buffer)."""
    L = sq.lib()
    for dt in (sq.SQ_F32, sq.SQ_F16, sq.SQ_BF16):
        assert L.sq_smooth_weights(None, dt, 8, 0, None, None, FAKE, None) == SHAPE
        assert L.sq_smooth_weights(None, dt, 8, 0, None, None, None, None) == SHAPE
        assert L.sq_smooth_weights_folded(None, dt, 8, 0, None, None, None, FAKE, None) == SHAPE
        assert L.sq_smooth_weights_fp8(None, dt, 8, 0, None, None, FAKE, None) == SHAPE
        for mode in (sq.SQ_PER_TENSOR_STATIC, sq.SQ_PER_TOKEN_DYNAMIC):
            assert L.sq_quantize_act(None, dt, 8, 0, None, mode, FAKE, None, FAKE, None) == SHAPE
            assert L.sq_quantize_act_fp8(None, dt, 8, 0, None, mode, FAKE, None, FAKE,
                                         None) == SHAPE
    for ydt in (sq.SQ_F32, sq.SQ_F16, sq.SQ_BF16):
        for M in (1, 8, 33, 300):   # decode and tiled launch shapes alike
            assert L.sq_gemm_i8_dequant(None, None, M, 64, 0, FAKE, 1, FAKE, FAKE, ydt, None,
                                        None) == SHAPE
            assert L.sq_gemm_i8_dequant(None, None, M, 64, 0, None, 1, None, None, ydt, None,
                                        None) == SHAPE
        assert L.sq_gemm_fp8_dequant(None, None, 40, 64, 0, None, 1, None, None, ydt,
                                     None) == SHAPE
        assert L.sq_int8_mixed_matmul(None, 40, 0, None, None, None, 64, 6.0, None, 0, None,
                                      ydt, None, None, None) == SHAPE
    assert L.sq_norm_quantize_act(None, sq.SQ_F16, 8, 0, 0, None, None, 1e-5, 1, None, None,
                                  FAKE, None) == SHAPE
    # no rows or no outputs: nothing to do, any K
    assert L.sq_smooth_weights(None, sq.SQ_F16, 0, 0, None, None, None, None) == OK
    assert L.sq_quantize_act(None, sq.SQ_F16, 0, 0, None, 1, None, None, None, None) == OK
    assert L.sq_gemm_i8_dequant(None, None, 0, 64, 0, None, 1, None, None, sq.SQ_F16, None,
                                None) == OK
    assert L.sq_gemm_i8_dequant(None, None, 8, 0, 0, None, 1, None, None, sq.SQ_F16, None,
                                None) == OK


def test_binding_rejects_zero_width_tensors_on_the_host():
    """Zero-width torch tensors have a null data pointer; the binding passes it
    through and the library's K == 0 check raises before any launch."""
    torch = pytest.importorskip("torch")
    L = sq.lib()
    z = torch.empty((5, 0), dtype=torch.float16)
    assert z.data_ptr() == 0
    assert L.sq_quantize_act(z.data_ptr(), sq.SQ_F16, 5, 0, None, 1, None, z.data_ptr(), FAKE,
                             None) == SHAPE


def test_binding_requires_gpu_tensors():
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError):
        sq.absmax_reduce(torch.zeros(4, 16))


def test_fold_norm_validation():
    L = sq.lib()
    assert L.sq_fold_norm(FAKE, None, FAKE, -1, FAKE, None, None) == SHAPE
    assert L.sq_fold_norm(FAKE, None, FAKE, 0, None, None, None) == OK  # nothing to do
    assert L.sq_fold_norm(None, None, FAKE, 8, FAKE, None, None) == NULL
    assert L.sq_fold_norm(FAKE, FAKE, FAKE, 8, FAKE, None, None) == NULL  # beta without beta_out
    assert L.sq_fold_norm(FAKE + 2, None, FAKE, 8, FAKE, None, None) == ALIGN


def test_norm_quantize_validation():
    L = sq.lib()
    f = L.sq_norm_quantize_act
    # args: x, dt, M, K, norm, gamma, beta, eps, mode, static_scale, xq, x_scale, stream
    assert f(FAKE, sq.SQ_F32, 4, 64, 0, FAKE, None, 1e-5, 1, None, FAKE, FAKE, None) == DTYPE
    assert f(FAKE, sq.SQ_BF16, 4, 64, 0, FAKE, None, 1e-5, 1, None, FAKE, FAKE, None) == DTYPE
    assert f(FAKE, sq.SQ_F16, 4, 64, 2, FAKE, None, 1e-5, 1, None, FAKE, FAKE, None) == ARG
    assert f(FAKE, sq.SQ_F16, 4, 64, 0, FAKE, None, -1.0, 1, None, FAKE, FAKE, None) == ARG
    assert f(FAKE, sq.SQ_F16, 4, 64, 0, FAKE, None, float("inf"), 1, None, FAKE, FAKE, None) == ARG
    assert f(FAKE, sq.SQ_F16, 4, 64, 0, FAKE, None, 1e-5, 3, None, FAKE, FAKE, None) == ARG
    assert f(FAKE, sq.SQ_F16, 4, 40, 0, FAKE, None, 1e-5, 1, None, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, sq.SQ_F16, 4, 0, 0, FAKE, None, 1e-5, 1, None, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, sq.SQ_F16, 4, 16400, 0, FAKE, None, 1e-5, 1, None, FAKE, FAKE, None) == UNSUP
    assert f(FAKE, sq.SQ_F16, 4, 64, 0, None, None, 1e-5, 1, None, FAKE, FAKE, None) == NULL
    assert f(FAKE, sq.SQ_F16, 4, 64, 0, FAKE, None, 1e-5, 0, None, FAKE, FAKE, None) == NULL
    assert f(FAKE, sq.SQ_F16, 4, 64, 1, FAKE, FAKE + 4, 1e-5, 1, None, FAKE, FAKE, None) == ALIGN
    assert f(FAKE, sq.SQ_F16, 0, 64, 0, FAKE, None, 1e-5, 1, None, FAKE, FAKE, None) == OK


def test_fp8_validation():
    L = sq.lib()
    assert L.sq_static_scale(FAKE, None, 8, 0.0, FAKE, None) == ARG
    assert L.sq_static_scale(FAKE, None, 8, float("inf"), FAKE, None) == ARG
    assert L.sq_static_scale(FAKE, None, -1, 448.0, FAKE, None) == SHAPE
    assert L.sq_static_scale(None, None, 8, 448.0, FAKE, None) == NULL
    assert L.sq_static_scale(FAKE + 2, None, 8, 448.0, FAKE, None) == ALIGN
    assert L.sq_smooth_weights_fp8(FAKE, sq.SQ_F16, 8, 24, None, FAKE, FAKE, None) == SHAPE
    assert L.sq_smooth_weights_fp8(FAKE, 9, 8, 32, None, FAKE, FAKE, None) == DTYPE
    assert L.sq_smooth_weights_fp8(FAKE, sq.SQ_F16, 8, 32, None, None, FAKE, None) == NULL
    assert L.sq_smooth_weights_fp8(None, sq.SQ_F16, 0, 32, None, None, None, None) == OK
    assert L.sq_quantize_act_fp8(FAKE, sq.SQ_F16, 8, 32, None, 2, None, FAKE, FAKE, None) == ARG
    assert L.sq_quantize_act_fp8(FAKE, sq.SQ_F16, 8, 32, None, sq.SQ_PER_TENSOR_STATIC, None,
                                 FAKE, FAKE, None) == NULL
    assert L.sq_quantize_act_fp8(FAKE, sq.SQ_F16, 8, 32, None, 1, None, FAKE + 8, FAKE,
                                 None) == ALIGN
    assert L.sq_quantize_act_fp8(None, sq.SQ_F16, 0, 32, None, 1, None, None, None, None) == OK
    g = L.sq_gemm_fp8_dequant
    assert g(FAKE, FAKE, 4, 4, 64, FAKE, 1, FAKE, FAKE, sq.SQ_F16, None) == SHAPE   # K % 128
    assert g(FAKE, FAKE, 4, 4, 0, FAKE, 1, FAKE, FAKE, sq.SQ_F16, None) == SHAPE
    assert g(FAKE, FAKE, 4, 4, 128, FAKE, 1, FAKE, FAKE, 7, None) == DTYPE
    assert g(FAKE, None, 4, 4, 128, FAKE, 1, FAKE, FAKE, sq.SQ_F16, None) == NULL
    assert g(FAKE, FAKE, 4, 4, 128, FAKE, 1, FAKE, FAKE + 1, sq.SQ_F16, None) == ALIGN
    assert g(None, None, 0, 4, 128, None, 1, None, None, sq.SQ_F16, None) == OK


def test_peaks_library_exports_its_header():
    from w8a8_post_quantization_amd import build as hip_build

    if not os.path.exists(hip_build.PEAKS_LIB_PATH):
        pytest.skip("libsq_peaks.so not built")
    P = ctypes.CDLL(hip_build.PEAKS_LIB_PATH)
    declared = sq.header_functions(os.path.join(os.path.dirname(sq.HEADER), "sq_peaks.h"),
                                   prefix="sqp_")
    assert declared == ["sqp_clock_rates", "sqp_mfma_loop", "sqp_read_stream", "sqp_rw_stream"]
    for name in declared:
        assert hasattr(P, name), name
