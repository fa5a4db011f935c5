"""GPU parity of the output-channel fold and of the shared-input batched
GEMMs of a hidden-1024 decoder layer, against the CPU oracle on the same
seeded inputs.

The SmoothQuant tutorial page, section 融入前序线性层的权重 and its table of
fold positions: down_proj's smoothing is folded into up_proj's output
channels and o_proj's into v_proj's; q/k/v share the input of one norm and
gate/up the input of another, so each group has one s (from the column
maxima of all its weights) and its weights can be concatenated into one
GEMM (N = 4096 for q|k|v, N = 6144 for gate|up).

Bars: int8 codes, per-row steps and narrowed outputs bit-exact; the
batched GEMM equals the separate GEMMs bit for bit (every output element is
one exact int32 sum and one dequant product).
"""
import numpy as np
import pytest

import oracle
import synth
import w8a8_post_quantization_amd as sq
from tests.gpu_util import assert_bits_equal, dev, host, log, to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t

    if not _t.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    sq.lib()
    return _t


def _pos(seed, stream, n, lo=0.05, spread=2.0):
    return (np.abs(synth.normal(seed, stream, (n,))) * spread + lo).astype(np.float32)


def _w(dt, N, K, seed):
    a = synth.normal(seed, 1, (N, K), std=0.03)
    if dt == "f32":
        return a
    if dt == "f16":
        return a.astype(np.float16)
    return to_bf16_bits(a)


# Shapes cover every quantizer variant: wave per row with 2/4/16 vectors per
# lane, the streamed long-row form, and the block-per-row form.
@pytest.mark.parametrize("N,K,dt,with_s", [
    (3072, 1024, "f16", True),    # up_proj of the decoder layer
    (1024, 1024, "f16", True),    # v_proj
    (2100, 2048, "f16", True),
    (2500, 96, "f32", True),
    (1000, 4096, "bf16", True),   # block per row
    (37, 2064, "f16", False),     # block per row, no column factor, tail vector
    (50, 16400, "f16", True),     # streamed rows
    (0, 64, "f16", True)])
def test_fold_smooth_weights_parity(torch, N, K, dt, with_s):
    w = _w(dt, N, K, N + K)
    r = _pos(N + K, 2, N, lo=0.02, spread=3.0)
    s = _pos(N + K, 3, K) if with_s else None
    log(f"fold_smooth_weights N={N} K={K} {dt} s={with_s}")
    wt = dev(w, torch)
    wq, ws = sq.smooth_weights(wt, None if s is None else dev(s, torch), row_mul=dev(r, torch))
    wq_o, ws_o = oracle.fold_smooth_weights(w, r, s)
    assert_bits_equal(host(ws, torch), ws_o, "w_scale")
    assert_bits_equal(host(wq, torch), wq_o, "wq")


def _group(cfg, names):
    return np.concatenate([cfg["W"][n] for n in names], axis=0)


@pytest.mark.parametrize("names", [("q", "k", "v"), ("gate", "up")])
def test_shared_scales_and_batched_gemm(torch, names):
    """One s for a group that shares its input; the group's weights
    concatenated into one GEMM equal the separate GEMMs."""
    cfg = synth.decoder_1024()
    X = cfg["X1024"]
    Wg = _group(cfg, names)
    log(f"shared scales {'|'.join(names)}")
    # running max over the members == max over the concatenation == oracle
    wa = sq.absmax_reduce(dev(cfg["W"][names[0]], torch))
    for n in names[1:]:
        sq.absmax_reduce(dev(cfg["W"][n], torch), out=wa, accumulate=True)
    wa_cat = sq.absmax_reduce(dev(Wg, torch))
    wa_o = oracle.absmax_cols(Wg)
    assert_bits_equal(host(wa, torch), wa_o, "shared w amax (running)")
    assert_bits_equal(host(wa_cat, torch), wa_o, "shared w amax (concatenated)")
    xa_o = oracle.absmax_cols(X)
    s_o, inv_o = oracle.compute_scales(xa_o, wa_o, 0.5)

    log(f"batched weights {'|'.join(names)} [{Wg.shape[0]},{Wg.shape[1]}]")
    wq, ws = sq.smooth_weights(dev(Wg, torch), dev(s_o, torch))
    wq_o, ws_o = oracle.smooth_weights(Wg, s_o)
    assert_bits_equal(host(ws, torch), ws_o, "w_scale")
    assert_bits_equal(host(wq, torch), wq_o, "wq")
    xq, xs = sq.quantize_act(dev(X, torch), dev(inv_o, torch))
    xq_o, xs_o = oracle.quantize_act(X, inv_o)
    assert_bits_equal(host(xq, torch), xq_o, "xq")

    log(f"batched gemm {'|'.join(names)}")
    y, acc = sq.gemm_i8_dequant(xq, wq, xs, ws, out_dtype=torch.float16, with_acc=True)
    # the oracle on every output
    y_o, acc_o = oracle.gemm_i8_dequant(xq_o, wq_o, xs_o, ws_o, y_dt=oracle.F16, per_row=1)
    assert_bits_equal(host(acc, torch), acc_o, "batched int32 sums")
    assert_bits_equal(host(y, torch), y_o, "batched y")
    # each member's own GEMM gives the same columns
    n0 = 0
    for n in names:
        Wm = cfg["W"][n]
        log(f"member gemm {n} [{Wm.shape[0]},{Wm.shape[1]}]")
        wq_m, ws_m = sq.smooth_weights(dev(Wm, torch), dev(s_o, torch))
        y_m = sq.gemm_i8_dequant(xq, wq_m, xs, ws_m, out_dtype=torch.float16)
        assert_bits_equal(host(y_m, torch), host(y, torch)[:, n0:n0 + Wm.shape[0]], f"{n} columns")
        n0 += Wm.shape[0]


def test_folded_mlp_chain(torch):
    """gate|up batched with down_proj's 1/s folded into up's rows only, the
    product act(gate) * up formed by the caller, quantized with no
    smoothing multiply, then down_proj smoothed by s: the int8 chain tracks
    the fp64 MLP, and its intermediate activation is h / s."""
    cfg = synth.decoder_1024()
    X = cfg["X1024"]
    Wgate, Wup, Wdown = cfg["W"]["gate"], cfg["W"]["up"], cfg["W"]["down"]
    F = Wgate.shape[0]
    silu = lambda t: t / (1.0 + np.exp(-t))
    x64 = X.astype(np.float64)
    h = silu(x64 @ Wgate.astype(np.float64).T) * (x64 @ Wup.astype(np.float64).T)
    y_ref = h @ Wdown.astype(np.float64).T

    # shared input smoothing of gate|up, down_proj's smoothing from h
    Wgu = np.concatenate([Wgate, Wup], axis=0)
    s_in, inv_in = oracle.compute_scales(oracle.absmax_cols(X), oracle.absmax_cols(Wgu), 0.5)
    s_d, inv_d = oracle.compute_scales(np.abs(h).max(axis=0).astype(np.float32),
                                       oracle.absmax_cols(Wdown), 0.5)
    row_mul = np.concatenate([np.ones(F, np.float32), inv_d])

    log("folded mlp weights")
    wq, ws = sq.smooth_weights(dev(Wgu, torch), dev(s_in, torch), row_mul=dev(row_mul, torch))
    wq_o, ws_o = oracle.fold_smooth_weights(Wgu, row_mul, s_in)
    assert_bits_equal(host(ws, torch), ws_o, "gate|up w_scale")
    assert_bits_equal(host(wq, torch), wq_o, "gate|up wq")
    dq, ds = sq.smooth_weights(dev(Wdown, torch), dev(s_d, torch))
    dq_o, ds_o = oracle.smooth_weights(Wdown, s_d)
    assert_bits_equal(host(dq, torch), dq_o, "down wq")

    log("folded mlp chain")
    xq, xs = sq.quantize_act(dev(X, torch), dev(inv_in, torch))
    gu = sq.gemm_i8_dequant(xq, wq, xs, ws, out_dtype=torch.float32)
    g32, u32 = gu[:, :F], gu[:, F:]
    hf = (g32 / (1.0 + torch.exp(-g32)) * u32).contiguous()   # caller's glue, fp32
    hq, hs = sq.quantize_act(hf)                                # no 1/s multiply
    y = sq.gemm_i8_dequant(hq, dq, hs, ds, out_dtype=torch.float32)
    y = host(y, torch).astype(np.float64)
    rel = np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref)
    h_scaled = host(hf, torch).astype(np.float64) * s_d
    rel_h = np.linalg.norm(h_scaled - h) / np.linalg.norm(h)
    print(f"\nfolded MLP rel. error vs fp64: y {rel:.4f}, h*s vs h {rel_h:.4f}")
    assert rel_h < 0.03, rel_h
    assert rel < 0.05, rel
