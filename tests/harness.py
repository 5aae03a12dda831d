"""Test helpers: run a fusion on the GPU through the C ABI and compare it
with the oracle.  Test infrastructure (it may call the oracle)."""
from __future__ import annotations

import numpy as np

NP_STORAGE = {"f32": np.float32, "bf16": np.uint16, "f16": np.uint16, "s8": np.int8,
              "u8": np.uint8, "s32": np.int32, "s4": np.uint8, "u4": np.uint8}  # s4/u4: packed bytes


def to_device(buf: np.ndarray):
    import torch
    b = np.ascontiguousarray(buf)
    if b.dtype == np.uint16:
        b = b.view(np.int16)
    return torch.from_numpy(b).cuda()


def from_device(t, dtype: str) -> np.ndarray:
    import torch
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.view(torch.int16)
    return t.cpu().numpy().view(NP_STORAGE[dtype])


def run_gpu(nodes, params, fusion=None, reps: int = 1):
    """Compile (unless `fusion` is given), launch `reps` times, return (out, fusion)."""
    import torch
    import compiler_hlo_amd as H
    f = fusion or H.Fusion(nodes)
    dev = [to_device(p) for p in params]
    out = None
    for _ in range(reps):
        out = f(*dev, out=out)
    torch.cuda.synchronize()
    return from_device(out, nodes[-1]["dtype"]), f


def f32_ord(a: np.ndarray) -> np.ndarray:
    i = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    return np.where(i >= 0, i, -(i & 0x7FFFFFFF))


def bf16_ord(bits: np.ndarray) -> np.ndarray:
    i = np.asarray(bits, np.uint16).astype(np.int64)
    return np.where(i < 0x8000, i, -(i & 0x7FFF))


def ulp_dist_f32(a, b) -> np.ndarray:
    return np.abs(f32_ord(a) - f32_ord(b))


def ulp_dist_bf16(a_bits, b_bits) -> np.ndarray:
    return np.abs(bf16_ord(a_bits) - bf16_ord(b_bits))


def nan_mask_f32(a):
    return np.isnan(np.asarray(a, np.float32))


def nan_mask_bf16(bits):
    b = np.asarray(bits, np.uint16)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)


def nan_mask_f16(bits):
    b = np.asarray(bits, np.uint16)
    return ((b & 0x7C00) == 0x7C00) & ((b & 0x03FF) != 0)


def nan_mask_16(bits, dtype: str):
    return nan_mask_f16(bits) if dtype == "f16" else nan_mask_bf16(bits)


def assert_bitexact(got: np.ndarray, want: np.ndarray, dtype: str):
    if dtype == "f32":
        gn, wn = nan_mask_f32(got), nan_mask_f32(want)
        assert np.array_equal(gn, wn), "NaN positions differ"
        g, w = got.view(np.uint32)[~gn], want.view(np.uint32)[~wn]
    elif dtype in ("bf16", "f16"):
        gn, wn = nan_mask_16(got, dtype), nan_mask_16(want, dtype)
        assert np.array_equal(gn, wn), "NaN positions differ"
        g, w = got[~gn], want[~wn]
    else:
        g, w = got, want
    bad = np.flatnonzero(g != w)
    assert bad.size == 0, "%d of %d elements differ; first at %d: got %r want %r" % (
        bad.size, g.size, bad[0], g[bad[0]], w[bad[0]])


def assert_ulp(got, want, dtype: str, max_ulp: int):
    if dtype == "f32":
        gn, wn = nan_mask_f32(got), nan_mask_f32(want)
        assert np.array_equal(gn, wn), "NaN positions differ"
        d = ulp_dist_f32(got[~gn], want[~wn])
    else:  # bf16 or f16: ordinal distance of the 16-bit sign-magnitude patterns
        gn, wn = nan_mask_16(got, dtype), nan_mask_16(want, dtype)
        assert np.array_equal(gn, wn), "NaN positions differ"
        d = ulp_dist_bf16(got[~gn], want[~wn])
    worst = int(d.max()) if d.size else 0
    assert worst <= max_ulp, "max distance %d ulp > %d (%d elements over)" % (
        worst, max_ulp, int((d > max_ulp).sum()))
    return d


def oracle_points_threaded(nodes, params, points, workers: int | None = None):
    """oracle.evaluate_points over row chunks in a thread pool.  The oracle
    is single-threaded C called through ctypes, which releases the GIL, and it
    keeps no shared state while evaluating, so the chunks run in parallel on
    the host's cores (at most 16, the host share of one GPU)."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    pts = np.ascontiguousarray(np.asarray(points, dtype=np.int64))
    oracle.lib()  # load once, before the threads
    workers = workers or max(1, min(16, os.cpu_count() or 1))
    chunks = np.array_split(np.arange(pts.shape[0]), workers * 4)
    with ThreadPoolExecutor(workers) as ex:
        parts = list(ex.map(lambda ix: oracle.evaluate_points(nodes, params, pts[ix]), [c for c in chunks if c.size]))
    vals = np.concatenate([v for v, _ in parts])
    aux = np.concatenate([a for _, a in parts])
    return vals, aux

