"""numpy <-> device marshalling and bit-level comparisons for the GPU tests."""
import sys

import numpy as np


def log(msg):
    """Name the case on stdout before each GPU step (flushed)."""
    print(f"[gpu-case] {msg}", flush=True)


def dev(a, torch):
    """Host numpy array -> GPU tensor (uint16 arrays are raw bfloat16 bits)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def host(t, torch):
    """GPU tensor -> numpy (bfloat16 as raw uint16 bits)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bits(a):
    a = np.asarray(a)
    if a.dtype in (np.float32, np.int32):
        return a.view(np.uint32)
    if a.dtype in (np.float16, np.uint16, np.int16):
        return a.view(np.uint16)
    return a


def assert_bits_equal(got, want, what):
    g, w = bits(got), bits(want)
    assert g.shape == w.shape, f"{what}: shape {g.shape} vs {w.shape}"
    bad = np.nonzero(g != w)
    if bad[0].size:
        i = tuple(b[0] for b in bad)
        raise AssertionError(f"{what}: {bad[0].size} of {g.size} differ; first at {i}: "
                             f"got {np.asarray(got)[i]!r} want {np.asarray(want)[i]!r}")


def ulp_dist(a, b):
    ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


def to_bf16_bits(a32):
    """fp32 numpy -> bfloat16 bits by round-to-nearest-even (input builder)."""
    u = np.asarray(a32, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
