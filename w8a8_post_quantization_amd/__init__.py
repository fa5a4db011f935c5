"""MI355X (gfx950) W8A8 SmoothQuant linear-layer path - Python binding.

Thin ctypes marshalling over the C ABI in ``include/sq.h`` (``libsq.so``,
built from ``csrc/`` by ``build.py``).  Every step of the path runs in the
library's HIP kernels; this module only checks tensors, allocates outputs
with torch (device memory), passes raw pointers and the current HIP stream,
and raises on a non-zero status.  There is no CPU fallback: importing the
functions works anywhere, calling them needs the built library and a GPU.

Names follow the C ABI:
  absmax_reduce      a1  per-channel abs-max (calibration statistics)
  compute_scales     a2  smoothing factors s, 1/s and the static step
  smooth_weights     a3  W * s -> per-output-channel int8
  quantize_act       a4  fused X / s -> int8 (per-token or per-tensor)
  gemm_i8_dequant    a5  int8 GEMM with the outer-product dequant epilogue
  int8_mixed_matmul  a6  LLM.int8() mixed decomposition
  fold_norm          1/s folded into the preceding norm's gamma / beta
  norm_quantize_act  fused fp16 norm -> int8 (per-token or per-tensor)
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsq.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "sq.h")
TEST_HEADER = os.path.join(os.path.dirname(HERE), "include", "sq_test.h")

SQ_F32, SQ_F16, SQ_BF16 = 0, 1, 2
SQ_PER_TENSOR_STATIC, SQ_PER_TOKEN_DYNAMIC = 0, 1
SQ_NORM_LAYER, SQ_NORM_RMS = 0, 1

_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_F = ctypes.c_float

SIGNATURES = {
    "sq_status_str": (ctypes.c_char_p, [_I]),
    "sq_version": (_I, []),
    "sq_absmax_reduce": (_I, [_P, _I, _I64, _I64, _I, _P, _P]),
    "sq_compute_scales": (_I, [_P, _P, _I64, _F, _P, _P, _P, _P]),
    "sq_smooth_weights": (_I, [_P, _I, _I64, _I64, _P, _P, _P, _P]),
    "sq_smooth_weights_folded": (_I, [_P, _I, _I64, _I64, _P, _P, _P, _P, _P]),
    "sq_quantize_act": (_I, [_P, _I, _I64, _I64, _P, _I, _P, _P, _P, _P]),
    "sq_gemm_i8_dequant": (_I, [_P, _P, _I64, _I64, _I64, _P, _I, _P, _P, _I, _P, _P]),
    "sq_int8_mixed_matmul_workspace": (ctypes.c_size_t, [_I64, _I64, _I64]),
    "sq_int8_mixed_matmul": (_I, [_P, _I64, _I64, _P, _P, _P, _I64, _F, _P, ctypes.c_size_t,
                                  _P, _I, _P, _P, _P]),
    "sq_int8_mixed_matmul_noalloc": (_I, [_P, _I64, _I64, _P, _P, _P, _I64, _F, _P, _I, _P, _P,
                                          _P]),
    "sq_fold_norm": (_I, [_P, _P, _P, _I64, _P, _P, _P]),
    "sq_norm_quantize_act": (_I, [_P, _I, _I64, _I64, _I, _P, _P, _F, _I, _P, _P, _P, _P]),
    "sq_norm_quantize_act_kernel": (_I, [_P, _I, _I64, _I64, _I, _P, _P, _F, _I, _P, _P, _P, _P,
                                         _I]),
    "sq_static_scale": (_I, [_P, _P, _I64, _F, _P, _P]),
    "sq_smooth_weights_fp8": (_I, [_P, _I, _I64, _I64, _P, _P, _P, _P]),
    "sq_quantize_act_fp8": (_I, [_P, _I, _I64, _I64, _P, _I, _P, _P, _P, _P]),
    "sq_gemm_fp8_dequant": (_I, [_P, _P, _I64, _I64, _I64, _P, _I, _P, _P, _I, _P]),
    # coverage entry points (include/sq_test.h): the tiled GEMM's block shape forced
    "sq_gemm_i8_dequant_tile": (_I, [_P, _P, _I64, _I64, _I64, _P, _I, _P, _P, _I, _P, _P, _I]),
    "sq_gemm_fp8_dequant_tile": (_I, [_P, _P, _I64, _I64, _I64, _P, _I, _P, _P, _I, _P, _I]),
    "sq_int8_mixed_matmul_tile": (_I, [_P, _I64, _I64, _P, _P, _P, _I64, _F, _P, ctypes.c_size_t,
                                       _P, _I, _P, _P, _P, _I]),
}


class SQError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {lib().sq_status_str(status).decode()}")


def header_functions(path: str = HEADER, prefix: str = "sq_"):
    """Names of the functions a header declares (include/sq.h by default)."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(" + prefix + r"[a-z0-9_]+)\s*\(", text)))


def lib():
    """Load libsq.so; raises if it has not been built (no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run `python -m w8a8_post_quantization_amd.build` "
                              "(hipcc, gfx950) first; there is no CPU fallback")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _torch():
    import torch

    return torch


def _dt(t) -> int:
    torch = _torch()
    return {torch.float32: SQ_F32, torch.float16: SQ_F16, torch.bfloat16: SQ_BF16}[t.dtype]


def _tdt(code: int):
    torch = _torch()
    return {SQ_F32: torch.float32, SQ_F16: torch.float16, SQ_BF16: torch.bfloat16}[code]


def _check(t, name, dtypes=None, ndim=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D")
    return t.data_ptr()


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _call(name, *args):
    status = getattr(lib(), name)(*args)
    if status != 0:
        raise SQError(name, status)


def absmax_reduce(x, out=None, accumulate=False, stream=None):
    """a1: out[c] = max_r |x[r, c]| (running max into `out` if accumulate)."""
    torch = _torch()
    x2 = x.reshape(-1, x.shape[-1])
    _check(x2, "x", (torch.float32, torch.float16, torch.bfloat16))
    if out is None:
        out = torch.empty(x2.shape[1], dtype=torch.float32, device=x.device)
    _check(out, "out", (torch.float32,))
    _call("sq_absmax_reduce", x2.data_ptr(), _dt(x2), x2.shape[0], x2.shape[1],
          int(bool(accumulate)), out.data_ptr(), _stream(stream))
    return out


def compute_scales(act_amax, w_amax, alpha, static=False, stream=None):
    """a2: (s, inv_s) or (s, inv_s, static_scale[2])."""
    torch = _torch()
    _check(act_amax, "act_amax", (torch.float32,), 1)
    _check(w_amax, "w_amax", (torch.float32,), 1)
    K = act_amax.shape[0]
    s = torch.empty(K, dtype=torch.float32, device=act_amax.device)
    inv = torch.empty_like(s)
    st = torch.empty(2, dtype=torch.float32, device=act_amax.device) if static else None
    _call("sq_compute_scales", act_amax.data_ptr(), w_amax.data_ptr(), K, float(alpha),
          s.data_ptr(), inv.data_ptr(), _ptr(st), _stream(stream))
    return (s, inv, st) if static else (s, inv)


def smooth_weights(w, s=None, row_mul=None, stream=None):
    """a3: (wq int8 [N,K], w_scale fp32 [N]).  row_mul [N]: the next layer's
    inv_s folded into this layer's output channels (sq_smooth_weights_folded)."""
    torch = _torch()
    _check(w, "w", (torch.float32, torch.float16, torch.bfloat16), 2)
    if s is not None:
        _check(s, "s", (torch.float32,), 1)
    N, K = w.shape
    if row_mul is not None:
        _check(row_mul, "row_mul", (torch.float32,), 1)
        if row_mul.numel() != N:
            raise ValueError(f"row_mul has {row_mul.numel()} elements, w has {N} rows")
    if s is not None and s.numel() != K:
        raise ValueError(f"s has {s.numel()} elements, w has {K} columns")
    wq = torch.empty((N, K), dtype=torch.int8, device=w.device)
    ws = torch.empty(N, dtype=torch.float32, device=w.device)
    if row_mul is None:
        _call("sq_smooth_weights", w.data_ptr(), _dt(w), N, K, _ptr(s), wq.data_ptr(),
              ws.data_ptr(), _stream(stream))
    else:
        _call("sq_smooth_weights_folded", w.data_ptr(), _dt(w), N, K, _ptr(row_mul), _ptr(s),
              wq.data_ptr(), ws.data_ptr(), _stream(stream))
    return wq, ws


def quantize_act(x, inv_s=None, mode=SQ_PER_TOKEN_DYNAMIC, static_scale=None, out=None,
                 stream=None):
    """a4: (xq int8 [M,K], x_scale fp32 [M] or [1])."""
    torch = _torch()
    x2 = x.reshape(-1, x.shape[-1])
    _check(x2, "x", (torch.float32, torch.float16, torch.bfloat16))
    if inv_s is not None:
        _check(inv_s, "inv_s", (torch.float32,), 1)
    if static_scale is not None:
        _check(static_scale, "static_scale", (torch.float32,), 1)
    M, K = x2.shape
    if out is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
        xs = torch.empty(M if mode == SQ_PER_TOKEN_DYNAMIC else 1, dtype=torch.float32,
                         device=x.device)
    else:
        xq, xs = out
    _call("sq_quantize_act", x2.data_ptr(), _dt(x2), M, K, _ptr(inv_s), int(mode),
          _ptr(static_scale), xq.data_ptr(), xs.data_ptr(), _stream(stream))
    return xq, xs


def gemm_i8_dequant(xq, wq, x_scale, w_scale, out_dtype=None, with_acc=False, out=None,
                    stream=None, tile=None):
    """a5: y [M,N] (and acc int32 [M,N] if with_acc).  tile 0 | 1 | 2 | 3
    forces the tiled kernel's block shape (include/sq_test.h; same bits)."""
    torch = _torch()
    _check(xq, "xq", (torch.int8,), 2)
    _check(wq, "wq", (torch.int8,), 2)
    _check(x_scale, "x_scale", (torch.float32,), 1)
    _check(w_scale, "w_scale", (torch.float32,), 1)
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError("xq and wq disagree on K")
    per_row = 1 if (x_scale.numel() == M and M != 1) else 0
    if x_scale.numel() not in (1, M):
        raise ValueError("x_scale must have 1 or M elements")
    if w_scale.numel() != N:
        raise ValueError("w_scale must have N elements")
    y = out if out is not None else torch.empty(
        (M, N), dtype=out_dtype or torch.float32, device=xq.device)
    acc = torch.empty((M, N), dtype=torch.int32, device=xq.device) if with_acc else None
    if tile is None:
        _call("sq_gemm_i8_dequant", xq.data_ptr(), wq.data_ptr(), M, N, K, x_scale.data_ptr(),
              per_row, w_scale.data_ptr(), y.data_ptr(), _dt(y), _ptr(acc), _stream(stream))
    else:
        _call("sq_gemm_i8_dequant_tile", xq.data_ptr(), wq.data_ptr(), M, N, K,
              x_scale.data_ptr(), per_row, w_scale.data_ptr(), y.data_ptr(), _dt(y), _ptr(acc),
              _stream(stream), int(tile))
    return (y, acc) if with_acc else y


SQ_MIXED_SIDE_COLS = 128


def int8_mixed_matmul_workspace(M, N, K) -> int:
    return int(lib().sq_int8_mixed_matmul_workspace(M, N, K))


def int8_mixed_workspace_parts(M, N, K):
    """Byte offsets of the parts the workspace holds on return (include/sq.h):
    xq [M,K] int8, x_scale [M], colmax [K], mask [K] fp32, idx [K] int32,
    count int32, then (written when |O| <= side_cols) the side operands
    x_side [side_cols, M] and w_side [side_cols, N] fp32."""
    r = lambda b: (b + 255) // 256 * 256  # noqa: E731
    cap = min(K, SQ_MIXED_SIDE_COLS)
    off = {"xq": 0, "side_cols": cap}
    off["x_scale"] = off["xq"] + r(M * K)
    off["colmax"] = off["x_scale"] + r(4 * M)
    off["mask"] = off["colmax"] + r(4 * K)
    off["idx"] = off["mask"] + r(4 * K)
    off["count"] = off["idx"] + r(4 * K)
    off["x_side"] = off["count"] + 256
    off["w_side"] = off["x_side"] + r(4 * cap * M)
    off["total"] = off["w_side"] + r(4 * cap * N)
    return off


def int8_mixed_matmul(x, wq, w_scale, w_f16, threshold=6.0, out_dtype=None, workspace=None,
                      with_count=False, with_acc=False, stream=None, tile=None):
    """a6: LLM.int8() y [M,N], then (if asked) acc int32 [M,N] and |O| as a
    1-element int32 tensor: y, (y, cnt), (y, acc) or (y, acc, cnt)."""
    torch = _torch()
    _check(x, "x", (torch.float16,), 2)
    _check(wq, "wq", (torch.int8,), 2)
    _check(w_scale, "w_scale", (torch.float32,), 1)
    _check(w_f16, "w_f16", (torch.float16,), 2)
    M, K = x.shape
    N = wq.shape[0]
    need = int8_mixed_matmul_workspace(M, N, K)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    y = torch.empty((M, N), dtype=out_dtype or torch.float16, device=x.device)
    cnt = torch.zeros(1, dtype=torch.int32, device=x.device) if with_count else None
    acc = torch.empty((M, N), dtype=torch.int32, device=x.device) if with_acc else None
    args = (x.data_ptr(), M, K, wq.data_ptr(), w_scale.data_ptr(), w_f16.data_ptr(), N,
            float(threshold), workspace.data_ptr(), workspace.numel(), y.data_ptr(), _dt(y),
            _ptr(acc), _ptr(cnt), _stream(stream))
    if tile is None:
        _call("sq_int8_mixed_matmul", *args)
    else:
        _call("sq_int8_mixed_matmul_tile", *args, int(tile))
    out = (y,) + ((acc,) if with_acc else ()) + ((cnt,) if with_count else ())
    return out if len(out) > 1 else y


def int8_mixed_matmul_noalloc(x, wq, w_scale, w_f16, threshold=6.0, out=None, acc=None,
                              count=None, stream=None):
    """a6 without a workspace (the library's per-GPU array): writes y into
    `out` (required, [M,N]), and acc / |O| into `acc` / `count` when given.
    Allocates nothing."""
    torch = _torch()
    _check(x, "x", (torch.float16,), 2)
    _check(wq, "wq", (torch.int8,), 2)
    _check(w_scale, "w_scale", (torch.float32,), 1)
    _check(w_f16, "w_f16", (torch.float16,), 2)
    _check(out, "out", (torch.float32, torch.float16, torch.bfloat16), 2)
    M, K = x.shape
    N = wq.shape[0]
    _call("sq_int8_mixed_matmul_noalloc", x.data_ptr(), M, K, wq.data_ptr(), w_scale.data_ptr(),
          w_f16.data_ptr(), N, float(threshold), out.data_ptr(), _dt(out), _ptr(acc), _ptr(count),
          _stream(stream))
    return out


def fold_norm(gamma, s, beta=None, stream=None):
    """(gamma / s, beta / s or None): the smoothing folded into the norm."""
    torch = _torch()
    _check(gamma, "gamma", (torch.float32,), 1)
    _check(s, "s", (torch.float32,), 1)
    if beta is not None:
        _check(beta, "beta", (torch.float32,), 1)
    g_out = torch.empty_like(gamma)
    b_out = None if beta is None else torch.empty_like(beta)
    _call("sq_fold_norm", gamma.data_ptr(), _ptr(beta), s.data_ptr(), gamma.numel(),
          g_out.data_ptr(), _ptr(b_out), _stream(stream))
    return g_out, b_out


def norm_quantize_act(x, gamma, beta=None, norm=SQ_NORM_LAYER, eps=1e-5,
                      mode=SQ_PER_TOKEN_DYNAMIC, static_scale=None, out=None, stream=None,
                      kernel=None):
    """Fused fp16 norm -> int8: (xq int8 [M,K], x_scale fp32 [M] or [1]).
    kernel (tests only): 0 or 1 forces the block- or wave-per-row kernel
    through the coverage entry point of sq_test.h."""
    torch = _torch()
    x2 = x.reshape(-1, x.shape[-1])
    _check(x2, "x", (torch.float16,))
    _check(gamma, "gamma", (torch.float32,), 1)
    if beta is not None:
        _check(beta, "beta", (torch.float32,), 1)
    if static_scale is not None:
        _check(static_scale, "static_scale", (torch.float32,), 1)
    M, K = x2.shape
    if out is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
        xs = torch.empty(M if mode == SQ_PER_TOKEN_DYNAMIC else 1, dtype=torch.float32,
                         device=x.device)
    else:
        xq, xs = out
    args = (x2.data_ptr(), _dt(x2), M, K, int(norm), gamma.data_ptr(), _ptr(beta), float(eps),
            int(mode), _ptr(static_scale), xq.data_ptr(), xs.data_ptr(), _stream(stream))
    if kernel is None:
        _call("sq_norm_quantize_act", *args)
    else:
        _call("sq_norm_quantize_act_kernel", *args, int(kernel))
    return xq, xs


# ------------------------------------------------------------ FP8 (e4m3)

def static_scale(act_amax, inv_s=None, qmax=127.0, stream=None):
    """{step, 1/step} of a per-tensor static activation step (qmax 127 for
    int8, 448 for e4m3)."""
    torch = _torch()
    _check(act_amax, "act_amax", (torch.float32,), 1)
    if inv_s is not None:
        _check(inv_s, "inv_s", (torch.float32,), 1)
    out = torch.empty(2, dtype=torch.float32, device=act_amax.device)
    _call("sq_static_scale", act_amax.data_ptr(), _ptr(inv_s), act_amax.numel(), float(qmax),
          out.data_ptr(), _stream(stream))
    return out


def smooth_weights_fp8(w, s=None, stream=None):
    """a3 in e4m3: (wq uint8 [N,K] e4m3 codes, w_scale fp32 [N])."""
    torch = _torch()
    _check(w, "w", (torch.float32, torch.float16, torch.bfloat16), 2)
    if s is not None:
        _check(s, "s", (torch.float32,), 1)
    N, K = w.shape
    wq = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    ws = torch.empty(N, dtype=torch.float32, device=w.device)
    _call("sq_smooth_weights_fp8", w.data_ptr(), _dt(w), N, K, _ptr(s), wq.data_ptr(),
          ws.data_ptr(), _stream(stream))
    return wq, ws


def quantize_act_fp8(x, inv_s=None, mode=SQ_PER_TOKEN_DYNAMIC, static_scale=None, stream=None):
    """a4 in e4m3: (xq uint8 [M,K] e4m3 codes, x_scale fp32 [M] or [1])."""
    torch = _torch()
    x2 = x.reshape(-1, x.shape[-1])
    _check(x2, "x", (torch.float32, torch.float16, torch.bfloat16))
    if inv_s is not None:
        _check(inv_s, "inv_s", (torch.float32,), 1)
    if static_scale is not None:
        _check(static_scale, "static_scale", (torch.float32,), 1)
    M, K = x2.shape
    xq = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    xs = torch.empty(M if mode == SQ_PER_TOKEN_DYNAMIC else 1, dtype=torch.float32,
                     device=x.device)
    _call("sq_quantize_act_fp8", x2.data_ptr(), _dt(x2), M, K, _ptr(inv_s), int(mode),
          _ptr(static_scale), xq.data_ptr(), xs.data_ptr(), _stream(stream))
    return xq, xs


def gemm_fp8_dequant(xq, wq, x_scale, w_scale, out_dtype=None, out=None, stream=None,
                     tile=None):
    """f4: y [M,N] = fl(acc * fl(x_scale * w_scale)) with acc the fp32 sum of
    the e4m3 products (K % 128 == 0)."""
    torch = _torch()
    _check(xq, "xq", (torch.uint8,), 2)
    _check(wq, "wq", (torch.uint8,), 2)
    _check(x_scale, "x_scale", (torch.float32,), 1)
    _check(w_scale, "w_scale", (torch.float32,), 1)
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError(f"K mismatch: xq {tuple(xq.shape)}, wq {tuple(wq.shape)}")
    per_row = 1 if (x_scale.numel() == M and M != 1) else 0
    if not per_row and x_scale.numel() != 1:
        raise ValueError(f"x_scale has {x_scale.numel()} elements for M = {M}")
    if w_scale.numel() != N:
        raise ValueError(f"w_scale has {w_scale.numel()} elements for N = {N}")
    dt = out_dtype or torch.float16
    y = out if out is not None else torch.empty((M, N), dtype=dt, device=xq.device)
    if tile is None:
        _call("sq_gemm_fp8_dequant", xq.data_ptr(), wq.data_ptr(), M, N, K, x_scale.data_ptr(),
              int(per_row), w_scale.data_ptr(), y.data_ptr(), _dt(y), _stream(stream))
    else:
        _call("sq_gemm_fp8_dequant_tile", xq.data_ptr(), wq.data_ptr(), M, N, K,
              x_scale.data_ptr(), int(per_row), w_scale.data_ptr(), y.data_ptr(), _dt(y),
              _stream(stream), int(tile))
    return y
