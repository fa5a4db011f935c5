"""CPU oracle for the W8A8 SmoothQuant path - TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product path (the HIP library and its
binding) never imports, links or runs anything here, and shares no code with
it.  The arithmetic lives in ``sq_oracle.c`` (plain C11, one IEEE binary32
operation per step, see ``sq_oracle.h``); this module only marshals numpy
arrays into it.

Parity status: every function is pinned by CPU tests (``tests/test_oracle_*``)
except the cross-implementation ``pow`` used for the smoothing factors, which
is pinned only through its closed-form special cases (alpha = 0, 0.5, 1) and
the worked example of the SmoothQuant tutorial page.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-fPIC", "-shared", "-Wall", "-Wextra"]

F32, F16, BF16 = 0, 1, 2
PER_TENSOR_STATIC, PER_TOKEN_DYNAMIC = 0, 1
NORM_LAYER, NORM_RMS = 0, 1
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_F = ctypes.c_float


def build() -> str:
    """Compile sq_oracle.c into liboracle.so with gcc."""
    import subprocess

    subprocess.run(["gcc", *CFLAGS, "-o", LIB_PATH + ".tmp",
                    os.path.join(_HERE, "sq_oracle.c"), "-lm"], check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "orc_set_num_threads": (_I, [_I]),
            "orc_f16_to_f32": (_F, [ctypes.c_uint16]),
            "orc_bf16_to_f32": (_F, [ctypes.c_uint16]),
            "orc_f32_to_f16": (ctypes.c_uint16, [_F]),
            "orc_f32_to_bf16": (ctypes.c_uint16, [_F]),
            "orc_round_half_even": (_F, [_F]),
            "orc_absmax_cols": (None, [_P, _I, _I64, _I64, _I, _P]),
            "orc_compute_scales": (None, [_P, _P, _I64, _F, _P, _P, _P]),
            "orc_smooth_weights_f32": (None, [_P, _I, _I64, _I64, _P, _P]),
            "orc_quantize_rows_f32": (None, [_P, _I64, _I64, _P, _P]),
            "orc_smooth_weights": (None, [_P, _I, _I64, _I64, _P, _P, _P]),
            "orc_fold_smooth_weights": (None, [_P, _I, _I64, _I64, _P, _P, _P, _P]),
            "orc_quantize_act": (None, [_P, _I, _I64, _I64, _P, _I, _P, _P, _P]),
            "orc_gemm_i8_dequant": (_I64, [_P, _P, _I64, _I64, _I64, _P, _I, _P, _P, _I, _P]),
            "orc_gemm_i8_dequant_at": (None, [_P, _P, _I64, _P, _I, _P, _I, _P, _P, _I64, _P, _P]),
            "orc_outlier_columns": (_I64, [_P, _I64, _I64, _F, _P]),
            "orc_int8_mixed_matmul": (_I64, [_P, _I64, _I64, _P, _P, _P, _I64, _F, _P, _I,
                                             _P, _P, _P, _P]),
            "orc_int8_mixed_at": (None, [_P, _I64, _P, _P, _P, _P, _P, _P, _I64, _I, _P, _P,
                                         _I64, _P, _P]),
            "orc_matmul_f64": (None, [_P, _I, _P, _I, _I64, _I64, _I64, _P]),
            "orc_smoothed_matmul_f64": (None, [_P, _I, _P, _I, _P, _I64, _I64, _I64, _P]),
            "orc_fold_norm": (None, [_P, _P, _P, _I64, _P, _P]),
            "orc_fp8_decode": (_F, [ctypes.c_uint8]),
            "orc_fp8_encode": (ctypes.c_uint8, [_F]),
            "orc_quantize_rows_fp8": (None, [_P, _I64, _I64, _P, _P]),
            "orc_smooth_weights_fp8": (None, [_P, _I, _I64, _I64, _P, _P, _P]),
            "orc_quantize_act_fp8": (None, [_P, _I, _I64, _I64, _P, _I, _P, _P, _P]),
            "orc_static_scale": (None, [_P, _P, _I64, _F, _P]),
            "orc_gemm_fp8_dequant": (None, [_P, _P, _I64, _I64, _I64, _P, _I, _P, _P, _I, _P]),
            "orc_gemm_fp8_dequant_at": (None, [_P, _P, _I64, _P, _I, _P, _I, _P, _P, _I64, _P,
                                               _P]),
            "orc_norm_stats": (None, [_P, _I64, _I64, _I, _F, _P, _P]),
            "orc_norm_quantize": (None, [_P, _I64, _I64, _I, _P, _P, _F, _I, _P, _P, _P, _P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def set_num_threads(n: int = 0) -> int:
    return lib().orc_set_num_threads(n)


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float16:
        return F16
    if a.dtype == np.uint16:  # raw bfloat16 bits
        return BF16
    raise TypeError(f"unsupported dtype {a.dtype}")


def _c(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _out(shape, y_dt):
    return np.empty(shape, dtype=np.float32 if y_dt == F32 else (np.float16 if y_dt == F16 else np.uint16))


def absmax_cols(x, amax=None):
    x = _c(x)
    rows, cols = x.shape
    out = np.zeros(cols, np.float32) if amax is None else amax
    lib().orc_absmax_cols(x.ctypes.data, _dt(x), rows, cols, 0 if amax is None else 1,
                          out.ctypes.data)
    return out


def compute_scales(act_amax, w_amax, alpha, static=False):
    act_amax = _c(act_amax.astype(np.float32, copy=False))
    w_amax = _c(w_amax.astype(np.float32, copy=False))
    K = act_amax.size
    s = np.empty(K, np.float32)
    inv = np.empty(K, np.float32)
    st = np.empty(2, np.float32) if static else None
    lib().orc_compute_scales(act_amax.ctypes.data, w_amax.ctypes.data, K, float(alpha),
                             s.ctypes.data, inv.ctypes.data, _ptr(st))
    return (s, inv, st) if static else (s, inv)


def smooth_weights_f32(w, s):
    w = _c(w)
    N, K = w.shape
    out = np.empty((N, K), np.float32)
    lib().orc_smooth_weights_f32(w.ctypes.data, _dt(w), N, K, _ptr(s), out.ctypes.data)
    return out


def quantize_rows_f32(v):
    v = _c(v.astype(np.float32, copy=False))
    R, K = v.shape
    q = np.empty((R, K), np.int8)
    step = np.empty(R, np.float32)
    lib().orc_quantize_rows_f32(v.ctypes.data, R, K, q.ctypes.data, step.ctypes.data)
    return q, step


def smooth_weights(w, s=None):
    w = _c(w)
    N, K = w.shape
    wq = np.empty((N, K), np.int8)
    ws = np.empty(N, np.float32)
    if s is not None:
        s = _c(s.astype(np.float32, copy=False))
    lib().orc_smooth_weights(w.ctypes.data, _dt(w), N, K, _ptr(s), wq.ctypes.data, ws.ctypes.data)
    return wq, ws


def fold_smooth_weights(w, row_mul=None, s=None):
    """a3 with the next layer's 1/s folded into the output rows (row_mul)."""
    w = _c(w)
    N, K = w.shape
    wq = np.empty((N, K), np.int8)
    ws = np.empty(N, np.float32)
    if s is not None:
        s = _c(s.astype(np.float32, copy=False))
    if row_mul is not None:
        row_mul = _c(row_mul.astype(np.float32, copy=False))
    lib().orc_fold_smooth_weights(w.ctypes.data, _dt(w), N, K, _ptr(row_mul), _ptr(s),
                                  wq.ctypes.data, ws.ctypes.data)
    return wq, ws


def quantize_act(x, inv_s=None, mode=PER_TOKEN_DYNAMIC, static_scale=None):
    x = _c(x)
    M, K = x.shape
    xq = np.empty((M, K), np.int8)
    xs = np.empty(M if mode == PER_TOKEN_DYNAMIC else 1, np.float32)
    if inv_s is not None:
        inv_s = _c(inv_s.astype(np.float32, copy=False))
    if static_scale is not None:
        static_scale = _c(np.asarray(static_scale, np.float32))
    lib().orc_quantize_act(x.ctypes.data, _dt(x), M, K, _ptr(inv_s), mode, _ptr(static_scale),
                           xq.ctypes.data, xs.ctypes.data)
    return xq, xs


def gemm_i8_dequant(xq, wq, x_scale, w_scale, y_dt=F32, want_acc=True, want_y=True,
                    per_row=None):
    xq, wq = _c(xq), _c(wq)
    M, K = xq.shape
    N = wq.shape[0]
    x_scale = _c(x_scale.astype(np.float32, copy=False))
    w_scale = _c(w_scale.astype(np.float32, copy=False))
    y = _out((M, N), y_dt) if want_y else None
    acc = np.empty((M, N), np.int32) if want_acc else None
    ovf = lib().orc_gemm_i8_dequant(xq.ctypes.data, wq.ctypes.data, M, N, K, x_scale.ctypes.data,
                                    int(x_scale.size > 1) if per_row is None else int(per_row),
                                    w_scale.ctypes.data, _ptr(y), y_dt, _ptr(acc))
    if ovf:
        raise OverflowError(f"{ovf} int32 accumulators overflowed")
    return y, acc


def gemm_i8_dequant_at(xq, wq, x_scale, w_scale, rows, cols, y_dt=F32, per_row=None):
    xq, wq = _c(xq), _c(wq)
    K = xq.shape[1]
    rows = _c(np.asarray(rows, np.int64))
    cols = _c(np.asarray(cols, np.int64))
    x_scale = _c(x_scale.astype(np.float32, copy=False))
    w_scale = _c(w_scale.astype(np.float32, copy=False))
    if per_row is None:
        per_row = int(x_scale.size > 1)
    y = _out(rows.size, y_dt)
    acc = np.empty(rows.size, np.int32)
    lib().orc_gemm_i8_dequant_at(xq.ctypes.data, wq.ctypes.data, K, x_scale.ctypes.data,
                                 int(per_row), w_scale.ctypes.data, y_dt, rows.ctypes.data,
                                 cols.ctypes.data, rows.size, y.ctypes.data, acc.ctypes.data)
    return y, acc


def outlier_columns(x_f16, threshold):
    x = _c(x_f16).view(np.uint16)
    M, K = x.shape
    idx = np.empty(max(K, 1), np.int32)
    n = lib().orc_outlier_columns(x.ctypes.data, M, K, float(threshold), idx.ctypes.data)
    return idx[:n].copy()


def int8_mixed_matmul(x_f16, wq, w_scale, w_f16, threshold, y_dt=F16, want_y=True):
    """Returns dict(y, acc, xq, x_scale, idx)."""
    x = _c(x_f16).view(np.uint16)
    w16 = _c(w_f16).view(np.uint16)
    wq = _c(wq)
    w_scale = _c(w_scale.astype(np.float32, copy=False))
    M, K = x.shape
    N = wq.shape[0]
    y = _out((M, N), y_dt) if want_y else None
    acc = np.empty((M, N), np.int32)
    xq = np.empty((M, K), np.int8)
    xs = np.empty(M, np.float32)
    idx = np.empty(max(K, 1), np.int32)
    n = lib().orc_int8_mixed_matmul(x.ctypes.data, M, K, wq.ctypes.data, w_scale.ctypes.data,
                                    w16.ctypes.data, N, float(threshold), _ptr(y), y_dt,
                                    acc.ctypes.data, xq.ctypes.data, xs.ctypes.data,
                                    idx.ctypes.data)
    return {"y": y, "acc": acc, "xq": xq, "x_scale": xs, "idx": idx[:n].copy()}


def int8_mixed_prep(x_f16, threshold):
    """O, the quantized X~ and its row steps, without the product (N = 0):
    what the sampled evaluation below needs at full size."""
    x = _c(x_f16).view(np.uint16)
    M, K = x.shape
    xq = np.empty((M, K), np.int8)
    xs = np.empty(M, np.float32)
    idx = np.empty(max(K, 1), np.int32)
    dummy = np.zeros(1, np.int8)
    n = lib().orc_int8_mixed_matmul(x.ctypes.data, M, K, dummy.ctypes.data, None,
                                    None, 0, float(threshold), None, F16,
                                    None, xq.ctypes.data, xs.ctypes.data, idx.ctypes.data)
    return idx[:n].copy(), xq, xs


def int8_mixed_at(x_f16, xq, x_scale, wq, w_scale, w_f16, idx, rows, cols, y_dt=F16):
    x = _c(x_f16).view(np.uint16)
    w16 = _c(w_f16).view(np.uint16)
    K = x.shape[1]
    rows = _c(np.asarray(rows, np.int64))
    cols = _c(np.asarray(cols, np.int64))
    idx = _c(np.asarray(idx, np.int32))
    y = _out(rows.size, y_dt)
    acc = np.empty(rows.size, np.int32)
    lib().orc_int8_mixed_at(x.ctypes.data, K, _c(xq).ctypes.data,
                            _c(x_scale.astype(np.float32, copy=False)).ctypes.data,
                            _c(wq).ctypes.data, _c(w_scale.astype(np.float32, copy=False)).ctypes.data,
                            w16.ctypes.data, idx.ctypes.data, idx.size, y_dt, rows.ctypes.data,
                            cols.ctypes.data, rows.size, y.ctypes.data, acc.ctypes.data)
    return y, acc


def matmul_f64(x, w):
    x, w = _c(x), _c(w)
    M, K = x.shape
    N = w.shape[0]
    y = np.empty((M, N), np.float64)
    lib().orc_matmul_f64(x.ctypes.data, _dt(x), w.ctypes.data, _dt(w), M, N, K, y.ctypes.data)
    return y


def smoothed_matmul_f64(x, w, s):
    x, w = _c(x), _c(w)
    M, K = x.shape
    N = w.shape[0]
    s = _c(s.astype(np.float32, copy=False))
    y = np.empty((M, N), np.float64)
    lib().orc_smoothed_matmul_f64(x.ctypes.data, _dt(x), w.ctypes.data, _dt(w), s.ctypes.data,
                                  M, N, K, y.ctypes.data)
    return y


def f32_to_f16_bits(v: float) -> int:
    return lib().orc_f32_to_f16(v)


def f32_to_bf16_bits(v: float) -> int:
    return lib().orc_f32_to_bf16(v)


def round_half_even(v: float) -> float:
    return lib().orc_round_half_even(v)


def _f16_bits(x):
    x = _c(x)
    if x.dtype == np.float16:
        return x.view(np.uint16)
    raise TypeError("fp16 input expected")


def fold_norm(gamma, s, beta=None):
    """gamma' = fl(gamma / s), beta' = fl(beta / s) (the SmoothQuant tutorial
    page, section on folding into LayerNorm)."""
    gamma = _c(gamma.astype(np.float32))
    s = _c(s.astype(np.float32))
    g_out = np.empty_like(gamma)
    b = None if beta is None else _c(beta.astype(np.float32))
    b_out = None if b is None else np.empty_like(b)
    lib().orc_fold_norm(_ptr(gamma), _ptr(b), _ptr(s), gamma.size, _ptr(g_out), _ptr(b_out))
    return g_out, b_out


def norm_stats(x_f16, norm=NORM_LAYER, eps=1e-5):
    """Per-row (mu, rstd) in fp32 from exact row sums."""
    xb = _f16_bits(x_f16)
    M, K = xb.shape
    mu, rstd = np.empty(M, np.float32), np.empty(M, np.float32)
    lib().orc_norm_stats(_ptr(xb), M, K, norm, eps, _ptr(mu), _ptr(rstd))
    return mu, rstd


def norm_quantize(x_f16, gamma, beta=None, norm=NORM_LAYER, eps=1e-5,
                  mode=PER_TOKEN_DYNAMIC, static_scale=None, want_y=False):
    """Fused norm -> int8: returns (xq, x_scale) or (xq, x_scale, y fp32)."""
    xb = _f16_bits(x_f16)
    M, K = xb.shape
    gamma = _c(gamma.astype(np.float32))
    beta = None if beta is None else _c(beta.astype(np.float32))
    xq = np.empty((M, K), np.int8)
    xs = np.empty(M if mode == PER_TOKEN_DYNAMIC else 1, np.float32)
    st = None if static_scale is None else _c(static_scale.astype(np.float32))
    y = np.empty((M, K), np.float32) if want_y else None
    lib().orc_norm_quantize(_ptr(xb), M, K, norm, _ptr(gamma), _ptr(beta), eps, mode,
                            _ptr(st), _ptr(xq), _ptr(xs), _ptr(y))
    return (xq, xs, y) if want_y else (xq, xs)


# ------------------------------------------------------------ FP8 (e4m3)

def fp8_decode(codes):
    """uint8 e4m3fn codes -> float32 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, np.uint8)
    table = np.array([lib().orc_fp8_decode(i) for i in range(256)], np.float32)
    return table[c]


def fp8_encode(v):
    """float32 values with |v| <= 448 -> e4m3fn codes (nearest, ties even)."""
    v = np.asarray(v, np.float32)
    f = lib().orc_fp8_encode
    return np.array([f(float(t)) for t in v.reshape(-1)], np.uint8).reshape(v.shape)


def quantize_rows_fp8(v):
    v = _c(v.astype(np.float32, copy=False))
    R, K = v.shape
    q = np.empty((R, K), np.uint8)
    step = np.empty(R, np.float32)
    lib().orc_quantize_rows_fp8(v.ctypes.data, R, K, q.ctypes.data, step.ctypes.data)
    return q, step


def smooth_weights_fp8(w, s=None):
    w = _c(w)
    N, K = w.shape
    wq = np.empty((N, K), np.uint8)
    ws = np.empty(N, np.float32)
    if s is not None:
        s = _c(s.astype(np.float32, copy=False))
    lib().orc_smooth_weights_fp8(w.ctypes.data, _dt(w), N, K, _ptr(s), wq.ctypes.data,
                                 ws.ctypes.data)
    return wq, ws


def quantize_act_fp8(x, inv_s=None, mode=PER_TOKEN_DYNAMIC, static_scale=None):
    x = _c(x)
    M, K = x.shape
    xq = np.empty((M, K), np.uint8)
    xs = np.empty(M if mode == PER_TOKEN_DYNAMIC else 1, np.float32)
    if inv_s is not None:
        inv_s = _c(inv_s.astype(np.float32, copy=False))
    if static_scale is not None:
        static_scale = _c(np.asarray(static_scale, np.float32))
    lib().orc_quantize_act_fp8(x.ctypes.data, _dt(x), M, K, _ptr(inv_s), mode,
                               _ptr(static_scale), xq.ctypes.data, xs.ctypes.data)
    return xq, xs


def static_scale(act_amax, inv_s, qmax):
    act_amax = _c(act_amax.astype(np.float32, copy=False))
    if inv_s is not None:
        inv_s = _c(inv_s.astype(np.float32, copy=False))
    out = np.empty(2, np.float32)
    lib().orc_static_scale(act_amax.ctypes.data, _ptr(inv_s), act_amax.size, qmax,
                           out.ctypes.data)
    return out


def gemm_fp8_dequant(xq, wq, x_scale, w_scale, y_dt=F32, per_row=1):
    """(y, acc): acc the exact fp64 sum of the e4m3 products."""
    xq, wq = _c(xq), _c(wq)
    M, K = xq.shape
    N = wq.shape[0]
    x_scale = _c(np.asarray(x_scale, np.float32))
    w_scale = _c(np.asarray(w_scale, np.float32))
    y = _out((M, N), y_dt)
    acc = np.empty((M, N), np.float64)
    lib().orc_gemm_fp8_dequant(xq.ctypes.data, wq.ctypes.data, M, N, K, x_scale.ctypes.data,
                               per_row, w_scale.ctypes.data, y.ctypes.data, y_dt,
                               acc.ctypes.data)
    return y, acc


def gemm_fp8_dequant_at(xq, wq, x_scale, w_scale, rows, cols, y_dt=F32, per_row=1):
    xq, wq = _c(xq), _c(wq)
    K = xq.shape[1]
    x_scale = _c(np.asarray(x_scale, np.float32))
    w_scale = _c(np.asarray(w_scale, np.float32))
    rows = _c(np.asarray(rows, np.int64))
    cols = _c(np.asarray(cols, np.int64))
    n = rows.size
    y = _out((n,), y_dt)
    acc = np.empty(n, np.float64)
    lib().orc_gemm_fp8_dequant_at(xq.ctypes.data, wq.ctypes.data, K, x_scale.ctypes.data,
                                  per_row, w_scale.ctypes.data, y_dt, rows.ctypes.data,
                                  cols.ctypes.data, n, y.ctypes.data, acc.ctypes.data)
    return y, acc
