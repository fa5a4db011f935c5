"""Benchmark of the W8A8 SmoothQuant linear-layer path on one MI355X.

A step is one per-call pass of the SmoothQuant W8A8 linear layer at the
30B-class prefill shape (X fp16 [256, 7168] with 6 outlier channels x
U(20,100), W fp16 [28672, 7168] ~ N(0, 0.025), alpha = 0.5, per-token int8 X,
per-output-channel int8 W, bf16 out):

  a4  X * (1/s) -> int8 per token      a5  int8 GEMM + c_x (x) c_w dequant

with the weights cold: each step reads the next of three int8 weight copies
(616 MB, more than twice the 256 MB last-level cache), as a layer's weights
are when a model runs.  The offline steps (a1 abs-max of X and W, a2 the
smoothing factors, a3 W * s -> int8) are timed separately under `kernels`.

`value` is the step's int8 GEMM work (2*M*N*K ops) divided by the step time
(TOPS).  `roofline` is the prefill GEMM's (the step's dominant kernel)
against the int8 MFMA peak, with its fractions of the MFMA rate this GPU
reaches in a loop with no memory traffic and of the HBM-attainable ceiling
min(peak, ops/bytes x 8 TB/s).  Kernel-level extras follow: the GEMM with
warm weights, decode GEMMs at M = 1, 8, 32 (HBM GB/s), activation
quantization and abs-max on a 940 MB stream, the LLM.int8() mixed matmul,
the hidden-1024 decoder GEMM set and the fused norm -> int8 quantizer.  All
inputs are seeded synthetic data, generated on the host and resident in HBM
before any timed region.  `cpu_baseline` times the CPU oracle on the same
per-call pass over a bounded slice of the output channels on this host, and
the other workloads' GEMMs beside it.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5033.0      # MI355X dense int8 MFMA (256 CU x 2.4 GHz x 8192 ops/clk)
PEAK_FP8_TFLOPS = 5033.0     # MI355X dense fp8 MFMA (the same rate per clock)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
METRIC = "W8A8 GEMM TOPS + % INT8 MFMA peak (prefill); decode GB/s as % of HBM peak"


def profile_streams():
    """The activation-stream kernels of the extras (X fp16 [65536, 7168], 940
    MB) launched eagerly 3 times each: column abs-max, the per-token
    quantizer with 1/s, and the fused LayerNorm (with beta) -> per-token
    int8, so that a counter run sees one dispatch per launch."""
    import torch

    import w8a8_post_quantization_amd as sq

    L = sq.lib()
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(1)
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: t.data_ptr()  # noqa: E731
    U = lambda n, scale: torch.rand(n, generator=g, device=dev) * scale + scale * 0.1  # noqa: E731

    def chk(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what}: {L.sq_status_str(rc).decode()}")

    M, K = 65536, 7168
    X = torch.randn((M, K), dtype=torch.float16, generator=g, device=dev)
    X[:, :6] *= 50.0
    inv, gam, bet = U(K, 1.0), U(K, 1.0), U(K, 0.1)
    xq = torch.empty((M, K), dtype=torch.int8, device=dev)
    xs = torch.empty(M, dtype=torch.float32, device=dev)
    am = torch.empty(K, dtype=torch.float32, device=dev)
    ran = []
    for name, fn in (
            ("absmax", lambda: chk(L.sq_absmax_reduce(P(X), 1, M, K, 0, P(am), sp), "absmax")),
            ("quantize", lambda: chk(L.sq_quantize_act(P(X), 1, M, K, P(inv), 1, None, P(xq),
                                                       P(xs), sp), "quantize")),
            ("norm_quantize", lambda: chk(L.sq_norm_quantize_act(P(X), 1, M, K, 0, P(gam), P(bet),
                                                                 1e-5, 1, None, P(xq), P(xs),
                                                                 sp), "norm"))):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ran.append(name)
    print(json.dumps({"profile_streams": ran}), flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="keep running warm-up steps until this much time has passed (the "
                         "GPU's clocks take about a second under load to settle)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="only the step itself")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain elementwise copy of 1 GiB (3 launches): the "
                         "reference that scales the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--profile-gemms", action="store_true",
                    help="only run the GEMM workloads eagerly, a few launches each, for "
                         "rocprofv3 counter runs (MFMA utilisation, HBM bytes)")
    ap.add_argument("--profile-streams", action="store_true",
                    help="only run the 940 MB activation-stream kernels (abs-max, per-token "
                         "quantizer, fused norm -> int8) eagerly, 3 launches each, for "
                         "rocprofv3 counter runs")
    return ap.parse_args()


# Measured HBM traffic of a kernel comes from rocprofv3 counter runs kept in
# profiles/ (a fenced ```json block in the summary).  It is reported only
# while the kernel's sources still hash to what the counters were taken on.
TRAFFIC_FILES = {"a3_smooth_weights": "a3_smooth_weights_prefill_30b_traffic.md",
                 "a5_gemm": "a5_gemm_prefill_30b_traffic.md"}
KERNEL_SOURCES = {"a3_smooth_weights": ["w8a8_post_quantization_amd/csrc/quant.hip",
                                        "w8a8_post_quantization_amd/csrc/sq_device.h"],
                  "a5_gemm": ["w8a8_post_quantization_amd/csrc/gemm.hip",
                              "w8a8_post_quantization_amd/csrc/sq_device.h"]}


def sources_sha256(kernel):
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch from the committed counter summary, or None."""
    name = TRAFFIC_FILES.get(kernel)
    if name is None:
        return None
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    start = text.find("```json")
    if start < 0:
        return None
    end = text.find("```", start + 7)
    rec = json.loads(text[start + 7:end])
    if rec.get("sources_sha256") != sources_sha256(kernel):
        return None
    return rec["hbm_bytes_per_launch"]


def copy_calibration():
    import torch

    n = 1 << 28  # int32 elements: 1 GiB read and 1 GiB written per launch
    src = torch.arange(n, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": 4 * n, "bytes_written": 4 * n,
                                           "launches": 3}}), flush=True)


class Timer:
    """HIP event pairs on torch's current stream (the stream every call
    below is launched on)."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def run(self, name, fn):
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.pairs.setdefault(name, []).append((a, b))

    def avg_us(self, name):
        ps = self.pairs[name]
        return 1000.0 * sum(a.elapsed_time(b) for a, b in ps) / len(ps)


def profile_gemms():
    """Each GEMM workload launched eagerly (no graph), 3 times, so that a
    counter run sees one dispatch per launch: the prefill shape in int8 and
    e4m3 (3 rotating weight copies, beyond the last-level cache), the batched
    q|k|v GEMM of the hidden-1024 layer, decode at M = 1, 8, 32, and the
    LLM.int8() call on its 2048 x 4096 x 4096 workload."""
    import torch

    import w8a8_post_quantization_amd as sq

    L = sq.lib()
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(1)
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: t.data_ptr()  # noqa: E731
    R = lambda *shape: torch.randint(-127, 128, shape, dtype=torch.int8, generator=g,  # noqa: E731
                                     device=dev)
    U = lambda n, scale: torch.rand(n, generator=g, device=dev) * scale + scale * 0.1  # noqa: E731

    def F8(*shape):
        mag = torch.randint(0, 0x7F, shape, dtype=torch.int32, generator=g, device=dev)
        sgn = torch.randint(0, 2, shape, dtype=torch.int32, generator=g, device=dev) << 7
        return (mag | sgn).to(torch.uint8)

    def chk(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what}: {L.sq_status_str(rc).decode()}")

    ran = []
    for name, M, N, K, ydt in (("prefill_30b", 256, 28672, 7168, 2), ("qkv_1024", 4096, 4096, 1024, 1),
                               ("decode_M1", 1, 28672, 8192, 1), ("decode_M8", 8, 28672, 8192, 1),
                               ("decode_M32", 32, 28672, 8192, 1)):
        for kind, gen, fn in (("i8", R, L.sq_gemm_i8_dequant), ("f8", F8, L.sq_gemm_fp8_dequant)):
            ws_ = [gen(N, K) for _ in range(3)]
            x = gen(M, K)
            xs, ws = U(M, 1e-2), U(N, 1e-3)
            y = torch.empty((M, N), dtype=torch.bfloat16 if ydt == 2 else torch.float16, device=dev)
            for w in ws_:
                if kind == "i8":
                    chk(fn(P(x), P(w), M, N, K, P(xs), 1, P(ws), P(y), ydt, None, sp), name)
                else:
                    chk(fn(P(x), P(w), M, N, K, P(xs), 1, P(ws), P(y), ydt, sp), name)
            torch.cuda.synchronize()
            ran.append(f"{name}_{kind}")
            del ws_
    # LLM.int8() on its workload (fp16 X with 6 outlier columns of ~20 in
    # about half the rows): the side-term GEMM among its kernels.
    M, N, K = 2048, 4096, 4096
    x = torch.randn((M, K), generator=g, device=dev)
    x[:, torch.randperm(K, generator=g, device=dev)[:6]] *= 20.0
    x = x.half()
    w16 = (torch.randn((N, K), generator=g, device=dev) * 0.02).half()
    wq = torch.empty((N, K), dtype=torch.int8, device=dev)
    ws = torch.empty(N, dtype=torch.float32, device=dev)
    chk(L.sq_smooth_weights(P(w16), 1, N, K, None, P(wq), P(ws), sp), "llm_int8 weights")
    need = L.sq_int8_mixed_matmul_workspace(M, N, K)
    work = torch.empty(need, dtype=torch.uint8, device=dev)
    y = torch.empty((M, N), dtype=torch.float16, device=dev)
    for _ in range(3):
        chk(L.sq_int8_mixed_matmul(P(x), M, K, P(wq), P(ws), P(w16), N, 6.0, P(work), need, P(y), 1,
                                   None, None, sp), "llm_int8")
    torch.cuda.synchronize()
    ran.append("llm_int8")
    print(json.dumps({"profile_gemms": ran}), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.profile_gemms:
        profile_gemms()
        return
    if args.profile_streams:
        profile_streams()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    import w8a8_post_quantization_amd as sq

    L = sq.lib()
    torch.cuda.init()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def T(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def chk(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what}: {L.sq_status_str(rc).decode()}")

    # ------------------------------------------------------------ inputs
    M, N, K = 256, 28672, 7168
    cfg = synth.prefill_30b(M, N, K)
    X, W = T(cfg["X"]), T(cfg["W"])
    del cfg
    f32 = dict(dtype=torch.float32, device=dev)
    xamax, wamax = torch.empty(K, **f32), torch.empty(K, **f32)
    s, inv_s = torch.empty(K, **f32), torch.empty(K, **f32)
    NCOPY = 3  # 3 x 205 MB of int8 weights: beyond the 256 MB last-level cache
    wqs = [torch.empty((N, K), dtype=torch.int8, device=dev) for _ in range(NCOPY)]
    ws = torch.empty(N, **f32)
    xq = torch.empty((M, K), dtype=torch.int8, device=dev)
    xs = torch.empty(M, **f32)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    P = lambda t: t.data_ptr()  # noqa: E731

    # The offline part of the layer (calibration statistics, smoothing
    # factors, weight quantization): timed per kernel, not part of a step.
    offline = [
        ("a1_absmax_x", lambda: chk(L.sq_absmax_reduce(P(X), 1, M, K, 0, P(xamax), sp), "a1x")),
        ("a1_absmax_w", lambda: chk(L.sq_absmax_reduce(P(W), 1, N, K, 0, P(wamax), sp), "a1w")),
        ("a2_scales", lambda: chk(L.sq_compute_scales(P(xamax), P(wamax), K, 0.5, P(s), P(inv_s),
                                                      None, sp), "a2")),
        ("a3_smooth_weights", lambda: chk(L.sq_smooth_weights(P(W), 1, N, K, P(s), P(wqs[0]),
                                                              P(ws), sp), "a3")),
    ]
    for _, fn in offline:
        fn()
    for c in range(1, NCOPY):  # the same quantized weights in distinct memory
        chk(L.sq_smooth_weights(P(W), 1, N, K, P(s), P(wqs[c]), P(ws), sp), "a3")
    torch.cuda.synchronize()

    def a4():
        chk(L.sq_quantize_act(P(X), 1, M, K, P(inv_s), 1, None, P(xq), P(xs), sp), "a4")

    def a5(i):
        chk(L.sq_gemm_i8_dequant(P(xq), P(wqs[i % NCOPY]), M, N, K, P(xs), 1, P(ws), P(y), 2,
                                 None, sp), "a5")

    bytes_per_call = {  # algorithmic HBM bytes of one launch
        "a1_absmax_x": M * K * 2 + 4 * K,
        "a1_absmax_w": N * K * 2 + 4 * K,
        "a2_scales": 4 * 4 * K,
        "a3_smooth_weights": N * K * 2 + N * K + 4 * K + 4 * N,
        "a4_quantize_act": M * K * 2 + M * K + 4 * K + 4 * M,
        "a5_gemm": M * K + N * K + M * N * 2 + 4 * M + 4 * N,
    }
    gemm_ops = 2.0 * M * N * K

    # Warm-up: at least W steps and at least --warmup-seconds of them, with a
    # synchronization every 32 steps so that host time tracks GPU time.
    n_warm = 0
    t_warm = time.perf_counter()
    while n_warm < args.warmup or time.perf_counter() - t_warm < args.warmup_seconds:
        a4()
        a5(n_warm)
        n_warm += 1
        if n_warm % 32 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    # Per-kernel breakdown, in passes of their own (an event pair around every
    # launch adds gaps between kernels): the step's two kernels, then the
    # offline ones (a3 writes the first weight copy again, same bits).
    tm = Timer(torch)
    for i in range(args.steps):
        tm.run("a4_quantize_act", a4)
        tm.run("a5_gemm", lambda: a5(i))
    for _ in range(max(3, args.steps // 4)):
        for name, fn in offline:
            tm.run(name, fn)
    torch.cuda.synchronize()
    per_kernel = {}
    for name in ("a1_absmax_x", "a1_absmax_w", "a2_scales", "a3_smooth_weights",
                 "a4_quantize_act", "a5_gemm"):
        us = tm.avg_us(name)
        per_kernel[name] = {"us": round(us, 2),
                            "GBs": round(bytes_per_call[name] / us / 1e3, 1),
                            "offline": name not in ("a4_quantize_act", "a5_gemm")}
    per_kernel["a5_gemm"]["TOPS"] = round(gemm_ops / per_kernel["a5_gemm"]["us"] / 1e6, 1)

    # Timed steps: events around the whole run, and around each GEMM launch
    # (its live duration, on the stream it runs on, for the roofline).
    live = Timer(torch)
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        a4()
        live.run("a5_gemm", lambda: a5(i))
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    dom_us = live.avg_us("a5_gemm")
    achieved = gemm_ops / dom_us / 1e6
    attainable = min(PEAK_INT8_TOPS, gemm_ops / bytes_per_call["a5_gemm"] * PEAK_HBM_GBS / 1e3)
    roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_INT8_TOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_INT8_TOPS, 4),
            "traffic": measured_traffic("a5_gemm"),
            "kernel": "a5_gemm (gemm_pp 256x128 tiles, int8 MFMA 32x32x32)",
            "kernel_us": round(dom_us, 2), "ops_per_launch": gemm_ops,
            "algorithmic_bytes_per_launch": bytes_per_call["a5_gemm"],
            "hbm_attainable": round(attainable, 1),
            "frac_attainable": round(achieved / attainable, 4)}
    value = gemm_ops / (ms_per_step * 1e-3) / 1e12

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_steps_run": n_warm,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8",
        "data": "synthetic (seeded SplitMix64 normals with planted outlier channels)",
        "config": {"workload": "prefill_30b: SmoothQuant W8A8 linear layer per call "
                               "(a4 quantize + a5 GEMM, weights cold: 3 rotating copies)",
                   "M": M, "N": N, "K": K, "alpha": 0.5,
                   "x": "fp16, 6 channels x U(20,100)", "w": "fp16 N(0,0.025)",
                   "act_quant": "per-token dynamic", "y": "bf16"},
        "roofline": roof, "kernels": per_kernel, "wall_s_timed": round(wall, 3),
    }
    del X, W, wqs

    if not args.no_extras:
        out["extras"] = extras(torch, L, sp, T, chk)
        mp = out["extras"].get("measured_peaks", {}).get("int8_mfma")
        if mp:
            roof["frac_measured_mfma"] = round(achieved / mp["rate"], 4)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


def _time_loop(torch, fns, iters):
    """Average GPU us per call of fns[i % len(fns)] over `iters` calls.

    The calls are captured once into a HIP graph and the graph is replayed,
    so the figure is the kernels' own time, not the host's launch rate (the
    short kernels here take less time than a Python-level launch).  Each fn
    launches on torch's current stream, which is the capture stream.  Five
    untimed replays come first: on this GPU the first replays of a new
    workload ran up to 25 % slower than its steady state (the cold prefill
    GEMM: 83 us, then 73, then 66-68)."""
    for f in fns:
        f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(iters):
            fns[i % len(fns)]()
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 3
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return 1000.0 * a.elapsed_time(b) / (iters * reps)


def measured_peaks(torch):
    """What simple kernels get from this GPU (include/sq_peaks.h): the int8
    and e4m3 matrix-core rate of an MFMA loop with no memory traffic, the
    HBM rate of a 1 GiB read and of a 1 GiB -> 512 MiB 2:1 stream (the
    quantizers' mix), and the shader clock sustained under each (clock
    counter ticks over real-time counter ticks, times the real-time rate)."""
    from w8a8_post_quantization_amd import build as hip_build

    if not os.path.exists(hip_build.PEAKS_LIB_PATH):
        raise RuntimeError(f"{hip_build.PEAKS_LIB_PATH} is missing: build first")
    L = ctypes.CDLL(hip_build.PEAKS_LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.sqp_mfma_loop.argtypes = [i32, i32, i32, vp, vp, vp]
    L.sqp_read_stream.argtypes = [vp, sz, i32, vp, vp, vp]
    L.sqp_rw_stream.argtypes = [vp, sz, vp, i32, i32, vp, vp]
    L.sqp_clock_rates.argtypes = [vp, vp]
    dev = torch.device("cuda:0")
    wall_khz, peak_khz = ctypes.c_int(0), ctypes.c_int(0)
    if L.sqp_clock_rates(ctypes.byref(wall_khz), ctypes.byref(peak_khz)) != 0:
        raise RuntimeError("clock-rate query failed")
    clk = torch.zeros(4, dtype=torch.int64, device=dev)
    sink = torch.zeros(8192, dtype=torch.int32, device=dev)

    def timed(launch, reps=5):
        sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for _ in range(2):
            if launch(sp) != 0:
                raise RuntimeError("peak probe launch failed")
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            launch(sp)
        b.record()
        torch.cuda.synchronize()
        sec = a.elapsed_time(b) / reps / 1e3
        c = clk.cpu().tolist()   # samples of the last launch (its first wave)
        return sec, (c[1] - c[0]) / (c[3] - c[2]) * wall_khz.value / 1e3

    res = {}
    blocks, iters = 512, 20000   # 2 blocks of 4 waves per CU: 2 waves per SIMD
    for fp8, name, per in ((0, "int8_mfma", 65536), (1, "fp8_mfma", 131072)):
        sec, sclk = timed(lambda sp: L.sqp_mfma_loop(fp8, iters, blocks, sink.data_ptr(),
                                                      clk.data_ptr(), sp))
        rate = blocks * 4 * iters * 4 * per / sec / 1e12
        peak = PEAK_INT8_TOPS if fp8 == 0 else PEAK_FP8_TFLOPS
        res[name] = {"rate": round(rate, 1), "unit": "TOPS" if fp8 == 0 else "TFLOP/s",
                     "frac_of_spec": round(rate / peak, 4), "sclk_MHz": round(sclk, 0)}
    res["clocks_MHz"] = {"wall_counter": wall_khz.value / 1e3, "peak_sclk": peak_khz.value / 1e3}
    nbytes = 1 << 30
    x = torch.randint(-(1 << 31), (1 << 31) - 1, (nbytes // 4,), dtype=torch.int32, device=dev)
    y = torch.empty(nbytes // 8, dtype=torch.int32, device=dev)
    sec, sclk = timed(lambda sp: L.sqp_read_stream(x.data_ptr(), nbytes, 4096, sink.data_ptr(),
                                                      clk.data_ptr(), sp))
    res["hbm_read"] = {"GBs": round(nbytes / sec / 1e9, 1),
                       "frac_hbm": round(nbytes / sec / 1e9 / PEAK_HBM_GBS, 4),
                       "sclk_MHz": round(sclk, 0)}
    sec, sclk = timed(lambda sp: L.sqp_rw_stream(x.data_ptr(), nbytes, y.data_ptr(), 8192, 1,
                                                    clk.data_ptr(), sp))
    res["hbm_rw_2to1"] = {"GBs": round(1.5 * nbytes / sec / 1e9, 1),
                          "frac_hbm": round(1.5 * nbytes / sec / 1e9 / PEAK_HBM_GBS, 4),
                          "sclk_MHz": round(sclk, 0)}
    del x, y
    return res


def extras(torch, L, _sp, T, chk):
    import synth

    dev = torch.device("cuda:0")

    class _CurStream:  # ctypes argument: torch's current stream at call time
        @property
        def _as_parameter_(self):
            return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    sp = _CurStream()
    P = lambda t: t.data_ptr()  # noqa: E731
    res = {}

    # Prefill GEMM with cold weights: 3 int8 weight copies (616 MB) rotate.
    M, N, K = 256, 28672, 7168
    g = torch.Generator(device=dev).manual_seed(1)
    R = lambda *shape: torch.randint(-127, 128, shape, dtype=torch.int8, generator=g,  # noqa: E731
                                     device=dev)
    U = lambda n, scale: torch.rand(n, generator=g, device=dev) * scale + scale * 0.1  # noqa: E731
    wqs = [R(N, K) for _ in range(3)]
    ws, xq, xs = U(N, 1e-3), R(M, K), U(M, 1e-2)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    fns = [lambda w=w: chk(L.sq_gemm_i8_dequant(P(xq), P(w), M, N, K, P(xs), 1, P(ws), P(y), 2,
                                                None, sp), "gemm") for w in wqs]
    us = _time_loop(torch, fns, 30)
    tops = 2.0 * M * N * K / us / 1e6
    gemm_bytes = M * K + N * K + M * N * 2 + 4 * M + 4 * N
    attainable = min(PEAK_INT8_TOPS, 2.0 * M * N * K / gemm_bytes * PEAK_HBM_GBS / 1e3)
    res["gemm_prefill_cold"] = {"us": round(us, 2), "TOPS": round(tops, 1),
                                "frac_int8_peak": round(tops / PEAK_INT8_TOPS, 4),
                                "hbm_attainable_TOPS": round(attainable, 1),
                                "frac_attainable": round(tops / attainable, 4)}
    us_w = _time_loop(torch, fns[:1], 30)
    res["gemm_prefill_warm"] = {"us": round(us_w, 2),
                                "TOPS": round(2.0 * M * N * K / us_w / 1e6, 1)}
    # Context, not a target: the vendor int8 GEMM (torch._int_mm, hipBLASLt;
    # int32 out, no dequant epilogue) on the same operands, cold and warm.
    vendor = {}
    try:
        fns_v = [lambda w=w: torch._int_mm(xq, w.t()) for w in wqs]
        for name, f in (("cold", fns_v), ("warm", fns_v[:1])):
            us_v = _time_loop(torch, f, 20)
            vendor[name] = {"us": round(us_v, 2), "TOPS": round(2.0 * M * N * K / us_v / 1e6, 1)}
    except RuntimeError as e:  # not every build ships the int8 path
        vendor = {"error": str(e)[:120]}
    res["vendor_int8_mm_prefill"] = vendor
    del wqs

    # The same prefill GEMM on the e4m3 path (finite codes: NaN codes never
    # occur in quantized data).
    def F8(*shape):
        mag = torch.randint(0, 0x7F, shape, dtype=torch.int32, generator=g, device=dev)
        sgn = torch.randint(0, 2, shape, dtype=torch.int32, generator=g, device=dev) << 7
        return (mag | sgn).to(torch.uint8)
    wqs = [F8(N, K) for _ in range(3)]
    xq8 = F8(M, K)
    fns = [lambda w=w: chk(L.sq_gemm_fp8_dequant(P(xq8), P(w), M, N, K, P(xs), 1, P(ws), P(y),
                                                 2, sp), "gemm fp8") for w in wqs]
    us = _time_loop(torch, fns, 30)
    tf = 2.0 * M * N * K / us / 1e6
    res["fp8_gemm_prefill_cold"] = {"us": round(us, 2), "TFLOPS": round(tf, 1),
                                    "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
                                    "frac_attainable": round(tf / attainable, 4)}
    us_w = _time_loop(torch, fns[:1], 30)
    res["fp8_gemm_prefill_warm"] = {"us": round(us_w, 2),
                                    "TFLOPS": round(2.0 * M * N * K / us_w / 1e6, 1)}
    del wqs

    # Decode: M in {1, 8, 32}, K = 8192, N = 28672, 3 rotating weight copies.
    M, N, K = 32, 28672, 8192
    wqs = [R(N, K) for _ in range(3)]
    ws = U(N, 1e-3)
    dec = {}
    for m in (1, 8, 32):
        xq, xs = R(m, K), U(m, 1e-2)
        y = torch.empty((m, N), dtype=torch.float16, device=dev)
        fns = [lambda w=w, xq=xq, xs=xs, y=y, m=m: chk(L.sq_gemm_i8_dequant(
            P(xq), P(w), m, N, K, P(xs), 1, P(ws), P(y), 1, None, sp), "decode") for w in wqs]
        us = _time_loop(torch, fns, 30)
        b = N * K + m * K + m * N * 2 + 4 * m + 4 * N
        dec[f"M{m}"] = {"us": round(us, 2), "GBs": round(b / us / 1e3, 1),
                        "frac_hbm": round(b / us / 1e3 / PEAK_HBM_GBS, 4)}
    res["decode"] = dec
    del wqs
    wqs = [F8(N, K) for _ in range(3)]
    dec = {}
    for m in (1, 8, 32):
        xq, xs = F8(m, K), U(m, 1e-2)
        y = torch.empty((m, N), dtype=torch.float16, device=dev)
        fns = [lambda w=w, xq=xq, xs=xs, y=y, m=m: chk(L.sq_gemm_fp8_dequant(
            P(xq), P(w), m, N, K, P(xs), 1, P(ws), P(y), 1, sp), "decode fp8") for w in wqs]
        us = _time_loop(torch, fns, 30)
        b = N * K + m * K + m * N * 2 + 4 * m + 4 * N
        dec[f"M{m}"] = {"us": round(us, 2), "GBs": round(b / us / 1e3, 1),
                        "frac_hbm": round(b / us / 1e3 / PEAK_HBM_GBS, 4)}
    res["fp8_decode"] = dec
    del wqs

    # Activation quantization and abs-max on a 940 MB stream (X fp16 [65536, 7168]).
    M, K = 65536, 7168
    Xs = torch.randn((M, K), dtype=torch.float16, generator=g, device=dev)
    Xs[:, :6] *= 50.0
    inv = U(K, 1.0)
    xq = torch.empty((M, K), dtype=torch.int8, device=dev)
    xs = torch.empty(M, dtype=torch.float32, device=dev)
    am = torch.empty(K, dtype=torch.float32, device=dev)
    us = _time_loop(torch, [lambda: chk(L.sq_quantize_act(P(Xs), 1, M, K, P(inv), 1, None, P(xq),
                                                          P(xs), sp), "quant")], 10)
    b = M * K * 3 + 4 * K + 4 * M
    res["quantize_stream"] = {"us": round(us, 2), "GBs": round(b / us / 1e3, 1),
                              "frac_hbm": round(b / us / 1e3 / PEAK_HBM_GBS, 4)}
    us = _time_loop(torch, [lambda: chk(L.sq_quantize_act_fp8(
        P(Xs), 1, M, K, P(inv), 1, None, P(xq), P(xs), sp), "quant fp8")], 10)
    res["fp8_quantize_stream"] = {"us": round(us, 2), "GBs": round(b / us / 1e3, 1),
                                  "frac_hbm": round(b / us / 1e3 / PEAK_HBM_GBS, 4)}
    us = _time_loop(torch, [lambda: chk(L.sq_absmax_reduce(P(Xs), 1, M, K, 0, P(am), sp),
                                        "absmax")], 10)
    b = M * K * 2 + 4 * K
    res["absmax_stream"] = {"us": round(us, 2), "GBs": round(b / us / 1e3, 1),
                            "frac_hbm": round(b / us / 1e3 / PEAK_HBM_GBS, 4)}
    # Fused norm (smoothing folded into gamma / beta) -> per-token int8 on
    # the same stream, and on the prefill activations.
    gam, bet = U(K, 1.0), U(K, 0.1)
    us = _time_loop(torch, [lambda: chk(L.sq_norm_quantize_act(
        P(Xs), 1, M, K, 0, P(gam), P(bet), 1e-5, 1, None, P(xq), P(xs), sp), "normq")], 10)
    b = M * K * 3 + 8 * K + 4 * M
    res["norm_quant_stream"] = {"us": round(us, 2), "GBs": round(b / us / 1e3, 1),
                                "frac_hbm": round(b / us / 1e3 / PEAK_HBM_GBS, 4)}
    Mp = 256
    us = _time_loop(torch, [lambda: chk(L.sq_norm_quantize_act(
        P(Xs), 1, Mp, K, 0, P(gam), P(bet), 1e-5, 1, None, P(xq), P(xs), sp), "normq")], 50)
    res["norm_quant_prefill"] = {"us": round(us, 2),
                                 "GBs": round((Mp * K * 3 + 8 * K + 4 * Mp) / us / 1e3, 1)}
    del Xs, xq

    # LLM.int8() mixed matmul, X fp16 [2048, 4096] with 6 planted dims, tau = 6.
    cfg = synth.llm_int8_2048()
    Xm, Wm = T(cfg["X"]), T(cfg["W"])
    M, K = Xm.shape
    N = Wm.shape[0]
    wq = torch.empty((N, K), dtype=torch.int8, device=dev)
    ws = torch.empty(N, dtype=torch.float32, device=dev)
    chk(L.sq_smooth_weights(P(Wm), 1, N, K, None, P(wq), P(ws), sp), "wq")
    need = L.sq_int8_mixed_matmul_workspace(M, N, K)
    wsp = torch.empty(need, dtype=torch.uint8, device=dev)
    y = torch.empty((M, N), dtype=torch.float16, device=dev)
    cnt = torch.zeros(1, dtype=torch.int32, device=dev)
    us = _time_loop(torch, [lambda: chk(L.sq_int8_mixed_matmul(
        P(Xm), M, K, P(wq), P(ws), P(Wm), N, 6.0, P(wsp), need, P(y), 1, None, P(cnt), sp),
        "mixed")],
        20)
    res["llm_int8_2048"] = {"us": round(us, 2), "n_outliers": int(cnt.item()),
                            "TOPS": round(2.0 * M * N * K / us / 1e6, 1)}

    # Hidden-1024 decoder GEMM set, M = 4096 (alpha only changes values).
    M = 4096
    total_us, total_ops, per = 0.0, 0.0, {}
    for name, n, k in synth.DECODER_1024_WEIGHTS:
        xq, wq, xs, ws = R(M, k), R(n, k), U(M, 1e-2), U(n, 1e-3)
        y = torch.empty((M, n), dtype=torch.float16, device=dev)
        us = _time_loop(torch, [lambda: chk(L.sq_gemm_i8_dequant(
            P(xq), P(wq), M, n, k, P(xs), 1, P(ws), P(y), 1, None, sp), "dec1024")], 50)
        ops = 2.0 * M * n * k
        per[name] = {"us": round(us, 2), "TOPS": round(ops / us / 1e6, 1)}
        total_us += us
        total_ops += ops
    res["decoder_1024"] = {"per_gemm": per, "total_us": round(total_us, 2),
                           "TOPS": round(total_ops / total_us / 1e6, 1),
                           "frac_int8_peak": round(total_ops / total_us / 1e6 / PEAK_INT8_TOPS, 4)}
    # The same layer with shared-input groups batched: q|k|v share one s and
    # become one GEMM (N = 4096), gate|up another (N = 6144).
    dims = {n: (nn, kk) for n, nn, kk in synth.DECODER_1024_WEIGHTS}
    groups = [("qkv", ("q", "k", "v")), ("o", ("o",)), ("gate_up", ("gate", "up")),
              ("down", ("down",))]
    total_us, total_ops, per = 0.0, 0.0, {}
    for gname, members in groups:
        n = sum(dims[m][0] for m in members)
        k = dims[members[0]][1]
        xq, wq, xs, ws = R(M, k), R(n, k), U(M, 1e-2), U(n, 1e-3)
        y = torch.empty((M, n), dtype=torch.float16, device=dev)
        us = _time_loop(torch, [lambda: chk(L.sq_gemm_i8_dequant(
            P(xq), P(wq), M, n, k, P(xs), 1, P(ws), P(y), 1, None, sp), "dec1024b")], 50)
        ops = 2.0 * M * n * k
        per[gname] = {"N": n, "K": k, "us": round(us, 2), "TOPS": round(ops / us / 1e6, 1)}
        total_us += us
        total_ops += ops
    res["decoder_1024_batched"] = {
        "per_gemm": per, "total_us": round(total_us, 2),
        "TOPS": round(total_ops / total_us / 1e6, 1),
        "frac_int8_peak": round(total_ops / total_us / 1e6 / PEAK_INT8_TOPS, 4)}
    # ... and on the e4m3 path.
    total_us, total_ops, per = 0.0, 0.0, {}
    for gname, members in groups:
        n = sum(dims[m][0] for m in members)
        k = dims[members[0]][1]
        xq, wq, xs, ws = F8(M, k), F8(n, k), U(M, 1e-2), U(n, 1e-3)
        y = torch.empty((M, n), dtype=torch.float16, device=dev)
        us = _time_loop(torch, [lambda: chk(L.sq_gemm_fp8_dequant(
            P(xq), P(wq), M, n, k, P(xs), 1, P(ws), P(y), 1, sp), "dec1024 fp8")], 50)
        ops = 2.0 * M * n * k
        per[gname] = {"N": n, "K": k, "us": round(us, 2), "TFLOPS": round(ops / us / 1e6, 1)}
        total_us += us
        total_ops += ops
    res["fp8_decoder_1024_batched"] = {
        "per_gemm": per, "total_us": round(total_us, 2),
        "TFLOPS": round(total_ops / total_us / 1e6, 1),
        "frac_fp8_peak": round(total_ops / total_us / 1e6 / PEAK_FP8_TFLOPS, 4)}
    res["measured_peaks"] = measured_peaks(torch)
    return res


def cpu_baseline(seconds):
    """The CPU oracle on this host.  The step's per-call pass (a4 quantize,
    a5 GEMM) over all 256 tokens and K = 7168 but only the first n output
    channels, n sized for about `seconds` of work on all host threads, and
    again on one thread (about a quarter of that); reported in TOPS of the
    slice's GEMM work over the slice's time.  Beside it, on all threads, the
    other workloads at full shape: the hidden-1024 decoder GEMM set
    (M = 4096, 7 GEMMs), decode (M = 32, N = 28672, K = 8192) and LLM.int8()
    (2048 x 4096 x 4096, threshold 6)."""
    import oracle
    import synth

    threads = oracle.set_num_threads(0)
    M, K = 256, 7168

    def run(ncols):
        X, W, _ = synth.linear_layer(2, M, ncols, K, 6, 20.0, 100.0, 0.025)
        xa = oracle.absmax_cols(X)
        wa = oracle.absmax_cols(W)
        s_, inv_ = oracle.compute_scales(xa, wa, 0.5)
        wq_, ws_ = oracle.smooth_weights(W, s_)
        t0 = time.perf_counter()
        xq_, xs_ = oracle.quantize_act(X, inv_, oracle.PER_TOKEN_DYNAMIC)
        oracle.gemm_i8_dequant(xq_, wq_, xs_, ws_, y_dt=oracle.BF16, want_acc=False)
        return time.perf_counter() - t0

    n = 256
    t = run(n)
    n = int(max(256, min(28672, n * seconds / max(t, 1e-3))))
    t = run(n)
    ops = 2.0 * M * n * K
    oracle.set_num_threads(1)
    n1 = 64
    t1 = run(n1)
    n1 = int(max(64, min(28672, n1 * seconds / 4 / max(t1, 1e-3))))
    t1 = run(n1)
    oracle.set_num_threads(0)

    rng = np.random.default_rng(0)
    others = {}

    def gemm_time(Mg, Ng, Kg, ydt):
        xq_ = rng.integers(-127, 128, (Mg, Kg), dtype=np.int8)
        wq_ = rng.integers(-127, 128, (Ng, Kg), dtype=np.int8)
        xs_ = rng.uniform(1e-3, 1e-2, Mg).astype(np.float32)
        ws_ = rng.uniform(1e-4, 1e-3, Ng).astype(np.float32)
        t0 = time.perf_counter()
        oracle.gemm_i8_dequant(xq_, wq_, xs_, ws_, y_dt=ydt, want_acc=False)
        return time.perf_counter() - t0

    tot_t, tot_ops = 0.0, 0.0
    for _, ng, kg in synth.DECODER_1024_WEIGHTS:   # 256 of the 4096 token rows
        tot_t += gemm_time(256, ng, kg, oracle.F16)
        tot_ops += 2.0 * 256 * ng * kg
    others["decoder_1024"] = {"s": round(tot_t, 2), "TOPS": round(tot_ops / tot_t / 1e12, 6),
                              "sample": "the 7 GEMMs on 256 of the 4096 token rows"}
    td = gemm_time(32, 28672, 8192, oracle.F16)
    others["decode_8192_M32"] = {"s": round(td, 2),
                                 "GBs": round(28672 * 8192 / td / 1e9, 3), "sample": "full"}
    cfg = synth.llm_int8_2048()
    Xm, Wm = cfg["X"], cfg["W"]
    wq_, ws_ = oracle.smooth_weights(Wm, None)
    rows = np.repeat(np.arange(0, 2048, 32), 4096)
    cols = np.tile(np.arange(4096), 64)
    t0 = time.perf_counter()
    idx, xq_, xs_ = oracle.int8_mixed_prep(Xm, 6.0)
    oracle.int8_mixed_at(Xm, xq_, xs_, wq_, ws_, Wm, idx, rows, cols)
    tm_ = time.perf_counter() - t0
    others["llm_int8_2048"] = {"s": round(tm_, 2),
                               "TOPS": round(2.0 * rows.size * 4096 / tm_ / 1e12, 6),
                               "sample": "outlier detection and X~ quantization in full, then "
                                         "64 of the 2048 output rows"}

    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(ops / t / 1e12, 6), "unit": "TOPS", "cores": threads, "kind": "oracle",
            "cpu": model,
            "sample": f"per-call pass (a4 quantize + a5 GEMM) on X [256,7168] and the first {n} "
                      f"of 28672 output channels of W ({t:.1f} s)",
            "one_thread": {"value": round(2.0 * M * n1 * K / t1 / 1e12, 6), "unit": "TOPS",
                           "sample": f"the same pass over the first {n1} output channels "
                                     f"({t1:.1f} s)"},
            "other_workloads_all_threads": others}


if __name__ == "__main__":
    main()
