"""Sweep of the migration strength alpha: quantization error of the W8A8
SmoothQuant linear layer on the synthetic workloads (a report, not a
benchmark).

For each alpha the layer runs through the library's kernels - column
abs-max of X and W, s_j = x_j^alpha / w_j^(1-alpha), W diag(s) per output
channel to int8, X diag(s)^-1 to int8 (per tensor or per token), the int8
GEMM with its dequant - and is compared with the fp64 product on a sample
of rows.  "none" is the same int8 path with no smoothing (s = 1).

Reported per alpha:
  y_err   ||Y_int8 - X W^T||_F / ||X W^T||_F
  x_err   ||diag(dx) Xq diag(s) - X||_F / ||X||_F      (activation side)
  w_err   ||diag(dw) Wq diag(s)^-1 - W||_F / ||W||_F   (weight side)
  x_zero, w_zero   fraction of int8 codes that are 0 (values lost to
          rounding: a plain, defined stand-in for the "truncation" the
          lpnh.cn write-up tabulates in §6.1, which it does not define)
  x_ratio  max_j / median_j of x_j / s_j (the activation outlier ratio
          left after smoothing); w_ratio the same for s_j w_j.

The SmoothQuant tutorial page, section 缩放因子, defines alpha's two ends
(alpha = 0: s = 1/w_j, everything left on the activations; alpha = 1:
s = x_j, everything moved to the weights) and section 缩放的代价 argues the
weight side is unaffected under per-input-row quantization; with the
per-output-channel weights used here w_err does grow with alpha, which is
the trade-off the sweep shows.

    python alpha_sweep.py [--config prefill_30b] [--mode static|token]
                          [--alphas 0,0.1,...,1] [--rows 256]
"""
from __future__ import annotations

import argparse
import json
import sys

import numpy as np

import synth

STATIC, TOKEN = "static", "token"


class GpuBackend:
    """The quantized path through the library's kernels (device tensors in,
    numpy out)."""

    def __init__(self):
        import torch

        import w8a8_post_quantization_amd as sq

        if not torch.cuda.is_available():
            raise RuntimeError("the GPU backend needs a GPU")
        self.torch, self.sq = torch, sq
        self._dev = {}
        sq.lib()

    def _d(self, a):
        # the same host array (X, W) is uploaded once per sweep
        key = (id(a), a.shape, a.dtype.str)
        hit = self._dev.get(key)
        if hit is not None and hit[0] is a:
            return hit[1]
        t = self.torch.from_numpy(np.ascontiguousarray(a)).cuda()
        if a.nbytes > (1 << 20):
            self._dev[key] = (a, t)
        return t

    def _h(self, t):
        return t.detach().cpu().numpy()

    def absmax(self, a):
        return self._h(self.sq.absmax_reduce(self._d(a)))

    def scales(self, x_amax, w_amax, alpha, static):
        r = [self._h(t) for t in self.sq.compute_scales(self._d(x_amax), self._d(w_amax), alpha,
                                                          static=static)]
        return r[0], r[1], (r[2] if static else None)

    def smooth_weights(self, w, s):
        wq, ws = self.sq.smooth_weights(self._d(w), None if s is None else self._d(s))
        return wq, ws

    def quantize_act(self, x, inv_s, static_scale):
        mode = self.sq.SQ_PER_TENSOR_STATIC if static_scale is not None else \
            self.sq.SQ_PER_TOKEN_DYNAMIC
        return self.sq.quantize_act(self._d(x), None if inv_s is None else self._d(inv_s), mode,
                                    None if static_scale is None else self._d(static_scale))

    def gemm(self, xq, wq, xs, ws):
        return self._h(self.sq.gemm_i8_dequant(xq, wq, xs, ws, out_dtype=self.torch.float32))

    def rows(self, t, idx):
        if isinstance(t, np.ndarray):
            return t[idx]
        return self._h(t[self.torch.from_numpy(idx).cuda()])

    def host(self, t):
        return t if isinstance(t, np.ndarray) else self._h(t)


def _f64(a):
    if a.dtype == np.uint16:  # raw bfloat16 bits
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def _ratio(v):
    v = np.asarray(v, np.float64)
    return float(v.max() / np.median(v))


def sweep(X, W, alphas, mode, backend, sample_rows=256, seed=0, X_cal=None):
    """Rows of dicts, one per alpha (None = no smoothing).  X_cal: the
    calibration activations the channel maxima come from (default X)."""
    static = mode == STATIC
    M, N = X.shape[0], W.shape[0]
    rng = np.random.default_rng(seed)
    xr = np.sort(rng.choice(M, size=min(M, sample_rows), replace=False))
    wr = np.sort(rng.choice(N, size=min(N, 4 * sample_rows), replace=False))
    X64, W64 = _f64(X), _f64(W)
    ref = X64[xr] @ W64.T
    x_amax = backend.absmax(X if X_cal is None else X_cal)
    w_amax = backend.absmax(W)
    out = []
    for a in alphas:
        if a is None:
            s = inv_s = None
            st = None
            if static:
                m = np.float32(x_amax.max())
                st = np.array([m / np.float32(127), np.float32(127) / m], np.float32)
            s_eff = np.ones(X.shape[1])
        else:
            s, inv_s, st = backend.scales(x_amax, w_amax, a, static)
            s_eff = s.astype(np.float64)
        wq, ws = backend.smooth_weights(W, s)
        xq, xs = backend.quantize_act(X, inv_s, st)
        y = backend.gemm(xq, wq, xs, ws)
        y = backend.host(y)[xr].astype(np.float64)
        xq_s = backend.rows(xq, xr).astype(np.float64)
        xs_h = backend.host(xs).astype(np.float64)
        dx = xs_h[xr][:, None] if xs_h.size > 1 else xs_h[0]
        wq_s = backend.rows(wq, wr).astype(np.float64)
        dw = backend.host(ws).astype(np.float64)[wr][:, None]
        out.append({
            "alpha": "none" if a is None else round(float(a), 3),
            "y_err": _rel(y, ref),
            "x_err": _rel(xq_s * dx * s_eff[None, :], X64[xr]),
            "w_err": _rel(wq_s * dw / s_eff[None, :], W64[wr]),
            "x_zero": float((xq_s == 0).mean()),
            "w_zero": float((wq_s == 0).mean()),
            "x_ratio": _ratio(x_amax / s_eff),
            "w_ratio": _ratio(w_amax * s_eff),
        })
    return out


CONFIGS = {
    "single_1024": lambda: synth.single_1024(),
    "prefill_30b": lambda: synth.prefill_30b(),
    "decoder_1024_q": lambda: {"X": synth.decoder_1024()["X1024"],
                               "W": synth.decoder_1024()["W"]["q"]},
    "decoder_1024_down": lambda: {"X": synth.decoder_1024()["X3072"],
                                  "W": synth.decoder_1024()["W"]["down"]},
    # decode: 32 tokens, the maxima from the 512-token calibration batch
    "decode_8192_m32": lambda: synth.decode_8192(32),
}


def mixed_errors(X, W, thresholds, backend, sample_rows=256, seed=0):
    """LLM.int8() on a layer: for each outlier threshold (inf = no outlier
    columns, the plain vector-wise int8 product) the relative Frobenius
    error of Y against the fp64 product on sampled rows, and |O|; then the
    SmoothQuant per-token path (alpha 0.5) on the same layer for comparison."""
    torch, sq = backend.torch, backend.sq
    rng = np.random.default_rng(seed)
    xr = np.sort(rng.choice(X.shape[0], size=min(X.shape[0], sample_rows), replace=False))
    ref = _f64(X)[xr] @ _f64(W).T
    xd, wd = backend._d(X), backend._d(W)
    wq, ws = sq.smooth_weights(wd)
    out = []
    for t in thresholds:
        y, cnt = sq.int8_mixed_matmul(xd, wq, ws, wd, t, out_dtype=torch.float32,
                                      with_count=True)
        out.append({"method": f"LLM.int8(), threshold {t}", "n_outliers": int(backend._h(cnt)[0]),
                    "y_err": _rel(backend._h(y)[xr].astype(np.float64), ref)})
    row = sweep(X, W, [0.5], TOKEN, backend, sample_rows, seed)[0]
    out.append({"method": "SmoothQuant, alpha 0.5, per-token", "n_outliers": 0,
                "y_err": row["y_err"]})
    return out


def markdown(rows, title):
    lines = [f"### {title}", "",
             "| alpha | y_err | x_err | w_err | x_zero | w_zero | x_ratio | w_ratio |",
             "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {r['alpha']} | {r['y_err']:.4f} | {r['x_err']:.4f} | {r['w_err']:.4f} | "
                     f"{r['x_zero']:.3f} | {r['w_zero']:.3f} | {r['x_ratio']:.1f} | "
                     f"{r['w_ratio']:.1f} |")
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--config", default="all", choices=["all", *CONFIGS])
    ap.add_argument("--mode", default="both", choices=["both", STATIC, TOKEN])
    ap.add_argument("--alphas", default="0,0.1,0.2,0.3,0.4,0.5,0.6,0.7,0.8,0.9,1")
    ap.add_argument("--rows", type=int, default=256)
    ap.add_argument("--json", action="store_true", help="one JSON line per table")
    args = ap.parse_args(argv)
    alphas = [None] + [float(a) for a in args.alphas.split(",")]
    backend = GpuBackend()
    names = list(CONFIGS) if args.config == "all" else [args.config]
    modes = [STATIC, TOKEN] if args.mode == "both" else [args.mode]
    for name in names:
        cfg = CONFIGS[name]()
        for mode in modes:
            rows = sweep(cfg["X"], cfg["W"], alphas, mode, backend, args.rows,
                         X_cal=cfg.get("X_cal"))
            title = f"{name}, X {'per-tensor static' if mode == STATIC else 'per-token'}"
            if args.json:
                print(json.dumps({"config": name, "mode": mode, "rows": rows}))
            else:
                print(markdown(rows, title) + "\n", flush=True)
    if args.config == "all":
        cfg = synth.llm_int8_2048()
        rows = mixed_errors(cfg["X"], cfg["W"], [float("inf"), 6.0], backend, args.rows)
        if args.json:
            print(json.dumps({"config": "llm_int8_2048", "rows": rows}))
        else:
            lines = ["### llm_int8_2048 (X fp16 [2048,4096], 6 outlier dims of ~20)", "",
                     "| method | \\|O\\| | y_err |", "|---|---|---|"]
            lines += [f"| {r['method']} | {r['n_outliers']} | {r['y_err']:.4f} |" for r in rows]
            print("\n".join(lines) + "\n", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
