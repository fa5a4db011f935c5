"""Seeded synthetic inputs for the W8A8 path (shared by tests, bench and smoke).

Holds no quantization arithmetic: it draws numbers from the counter-based
SplitMix64 generator in ``gen.c`` and shapes them into the workloads below.
Both the GPU path and the CPU oracle receive the very same host arrays.

Workload recipes (stream ids: 1 = X, 2 = W, 3 = outlier channels,
4 = outlier factors, 5 = outlier row draws, 6 = second/calibration X,
7 = outlier signs, 8 = outlier magnitudes, 10+i = i-th weight of a layer set,
20 = norm gamma, 21 = norm beta):

* ``linear_layer`` - one linear layer, X ~ N(0,1) [M,K] with a few fixed
  channels multiplied by per-channel factors, W ~ N(0, std) [N,K].
* ``prefill_30b``  - X fp16 [256, 7168], 6 channels x U(20,100);
  W fp16 [28672, 7168] ~ N(0, 0.025).
* ``decoder_1024`` - hidden-1024 layer set: X fp16 [4096,1024] and
  [4096,3072] with floor(1% K) channels x30; W ~ N(0, 0.03) for
  q [2048,1024], k/v/o [1024,1024], gate/up [3072,1024], down [1024,3072].
* ``decode_8192``  - X fp16 [M, 8192] (M in 1, 8, 32) and calibration
  X fp16 [512, 8192] sharing 4 channels x50; W fp16 [28672, 8192] ~ N(0, 0.02).
* ``llm_int8_2048`` - X fp16 [2048, 4096] ~ N(0,1) with 6 planted dims: in
  each, every row independently with p = 0.5 gets sign * U(18, 22);
  W fp16 [4096, 4096] ~ N(0, 0.02).
* ``single_1024``  - X fp32 [16, 1024] ~ N(0,1), channel 0 x50,
  W fp32 [1024, 1024] ~ N(0, 0.03).
* ``norm_params``  - the parameters of the norm before a layer: gamma fp32
  [K] ~ N(1, 0.1), beta fp32 [K] ~ N(0, 0.05).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


def build() -> str:
    """Compile gen.c into libsynth.so with gcc (CPU only)."""
    import subprocess

    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-o", LIB_PATH + ".tmp", os.path.join(_HERE, "gen.c"), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        L.synth_normal_f32.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_double,
                                       ctypes.c_double, ctypes.c_void_p, ctypes.c_int64]
        L.synth_uniform_f64.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p,
                                        ctypes.c_int64]
        L.synth_raw_u64.argtypes = [ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int64]
        _lib = L
    return _lib


def normal(seed: int, stream: int, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    lib().synth_normal_f32(seed, stream, mean, std, out.ctypes.data, out.size)
    return out


def uniform(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    lib().synth_uniform_f64(seed, stream, out.ctypes.data, n)
    return out


def raw_u64(key: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    lib().synth_raw_u64(key, out.ctypes.data, n)
    return out


def choose(seed: int, stream: int, K: int, count: int) -> np.ndarray:
    """`count` distinct channels out of K by partial Fisher-Yates, sorted."""
    u = uniform(seed, stream, count)
    perm = np.arange(K, dtype=np.int64)
    for i in range(count):
        j = i + int(u[i] * (K - i))
        perm[i], perm[j] = perm[j], perm[i]
    return np.sort(perm[:count])


def _to(a64: np.ndarray, dtype) -> np.ndarray:
    """Round to fp32 (RN), then to the storage dtype (fp16 RNE) if asked."""
    a32 = a64.astype(np.float32)
    return a32 if dtype == np.float32 else a32.astype(dtype)


def activations(seed, stream, M, K, channels, factors, dtype=np.float16):
    x = normal(seed, stream, (M, K)).astype(np.float64)
    if len(channels):
        x[:, channels] *= np.asarray(factors, dtype=np.float64)[None, :]
    return _to(x, dtype)


def weights(seed, stream, N, K, std, dtype=np.float16):
    w = normal(seed, stream, (N, K), std=std)
    return w if dtype == np.float32 else w.astype(dtype)


def linear_layer(seed, M, N, K, n_outliers, factor_lo, factor_hi, w_std,
                 dtype=np.float16, x_stream=1, w_stream=2):
    """Generic outlier-channel linear layer; returns (X, W, channels)."""
    ch = choose(seed, 3, K, n_outliers) if n_outliers else np.zeros(0, np.int64)
    if factor_lo == factor_hi:
        f = np.full(len(ch), float(factor_lo))
    else:
        f = factor_lo + (factor_hi - factor_lo) * uniform(seed, 4, len(ch))
    X = activations(seed, x_stream, M, K, ch, f, dtype)
    W = weights(seed, w_stream, N, K, w_std, dtype)
    return X, W, ch


def single_1024():
    x = normal(0, 1, (16, 1024)).astype(np.float64)
    x[:, 0] *= 50.0
    X = x.astype(np.float32)
    W = weights(0, 2, 1024, 1024, 0.03, np.float32)
    return {"X": X, "W": W, "alpha": 0.5, "channels": np.array([0])}


def prefill_30b(M=256, N=28672, K=7168, seed=2):
    X, W, ch = linear_layer(seed, M, N, K, 6, 20.0, 100.0, 0.025)
    return {"X": X, "W": W, "alpha": 0.5, "channels": ch}


DECODER_1024_WEIGHTS = [("q", 2048, 1024), ("k", 1024, 1024), ("v", 1024, 1024),
                        ("o", 1024, 1024), ("gate", 3072, 1024), ("up", 3072, 1024),
                        ("down", 1024, 3072)]


def decoder_1024(M=4096, seed=3, scale=1):
    """Hidden-1024 decoder-layer GEMM set; `scale` divides every size for a
    small variant (scale=1 is the full workload)."""
    Ms = M // scale
    out = {}
    for stream, K in ((1, 1024), (6, 3072)):
        Kd = K // scale
        n = max(1, int(0.01 * Kd))
        ch = choose(seed, 3 + (stream == 6) * 10, Kd, n)
        out[f"X{K}"] = activations(seed, stream, Ms, Kd, ch, np.full(n, 30.0))
    out["W"] = {}
    for i, (name, N, K) in enumerate(DECODER_1024_WEIGHTS):
        out["W"][name] = weights(seed, 10 + i, N // scale, K // scale, 0.03)
    return out


def decode_8192(M, N=28672, K=8192, seed=4, with_weights=True):
    ch = choose(seed, 3, K, 4)
    f = np.full(4, 50.0)
    out = {"X": activations(seed, 1, M, K, ch, f),
           "X_cal": activations(seed, 6, 512, K, ch, f),
           "alpha": 0.5, "channels": ch}
    if with_weights:
        out["W"] = weights(seed, 2, N, K, 0.02)
    return out


def llm_int8_2048(M=2048, N=4096, K=4096, seed=5, n_dims=6):
    x = normal(seed, 1, (M, K)).astype(np.float64)
    dims = choose(seed, 3, K, n_dims)
    hit = uniform(seed, 5, M * n_dims).reshape(M, n_dims) < 0.5
    sign = np.where(uniform(seed, 7, M * n_dims).reshape(M, n_dims) < 0.5, -1.0, 1.0)
    mag = 18.0 + 4.0 * uniform(seed, 8, M * n_dims).reshape(M, n_dims)
    for t, d in enumerate(dims):
        x[hit[:, t], d] = (sign * mag)[hit[:, t], t]
    X = _to(x, np.float16)
    W = weights(seed, 2, N, K, 0.02)
    return {"X": X, "W": W, "dims": dims, "threshold": 6.0}


def stream_act(M=65536, K=7168, seed=6):
    X, _, ch = linear_layer(seed, M, 1, K, 6, 20.0, 100.0, 0.025)
    return {"X": X, "channels": ch}


def norm_params(K, seed=7):
    """(gamma, beta) fp32 [K] of the norm that feeds a layer."""
    return normal(seed, 20, (K,), std=0.1, mean=1.0), normal(seed, 21, (K,), std=0.05)
