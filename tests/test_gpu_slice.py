"""GPU parity of slice and dynamic_slice (StableHLO Specification,
"dynamic_slice"; Operation semantics, DynamicSlice; slice's start_indices /
limit_indices in "Programs") through every hero, against the oracle.

Slices move data only, so every case is bit-exact: the elementwise ops around
them are exact (negate, add of integers, converts, max/min) or compared with
the same rounding on both sides.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W
from harness import assert_bitexact, run_gpu, to_device, from_device

pytestmark = pytest.mark.gpu

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_examples.json")))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import compiler_hlo_amd  # noqa: F401  (fails loudly without the library)
    yield


def say(*a):
    print(*a, flush=True)


def ints_f32(g, n, lo=-4, hi=4):
    return g.integers(lo, hi, n, endpoint=True).astype(np.float32)


@pytest.mark.parametrize("start,limit,strides", [
    ([3, 8], [290, 512], [1, 1]),      # start a multiple of the 128-bit width
    ([3, 5], [297, 517], [1, 1]),      # misaligned along the minor dim
    ([0, 1], [300, 520], [2, 3]),      # strided in both dims
    ([299, 0], [300, 520], [1, 1]),    # one row
    ([7, 7], [7, 100], [1, 1]),        # empty
])
def test_slice_loop(start, limit, strides):
    g = W.rng(401)
    x = W.normal_f32(g, 300 * 520)
    out = [-(-(b - a) // k) for a, b, k in zip(start, limit, strides)]
    s = W.Spec()
    p = s.parameter(0, "f32", [300, 520])
    q = s.slice(p, start, limit, strides, "f32", out)
    s.unary("negate", q, "f32", out)
    got, f = run_gpu(s.nodes, [x])
    say("slice", start, limit, strides, "->", f.plan()["hero"], "V", f.plan()["vector_elems"])
    assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "f32")


@pytest.mark.parametrize("dtype", ["bf16", "s8", "s4"])
def test_slice_loop_narrow_types(dtype):
    """Slices of 16-, 8- and 4-bit arrays, converted to f32 (exact)."""
    g = W.rng(402)
    dims = [97, 260]
    n = dims[0] * dims[1]
    if dtype == "bf16":
        x = W.normal_bf16(g, n)
    elif dtype == "s8":
        x = W.integers(g, n, -128, 127, np.int8)
    else:
        x = W.integers(g, (n + 1) // 2, 0, 255, np.uint8)
    for start, limit, strides in (([1, 16], [90, 240], [1, 1]), ([2, 3], [95, 257], [1, 1]),
                                  ([0, 1], [97, 260], [3, 2])):
        out = [-(-(b - a) // k) for a, b, k in zip(start, limit, strides)]
        s = W.Spec()
        p = s.parameter(0, dtype, dims)
        q = s.slice(p, start, limit, strides, dtype, out)
        s.convert(q, "f32", out)
        got, _ = run_gpu(s.nodes, [x])
        assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "f32")


def test_slice_transpose_hero():
    """transpose(slice(x)) and slice(transpose(x)) with ragged tiles: the
    transpose hero, bit-exact."""
    g = W.rng(403)
    x = W.normal_f32(g, 1000 * 1536)
    s = W.Spec()
    p = s.parameter(0, "f32", [1000, 1536])
    q = s.slice(p, [7, 64], [993, 1472], [1, 1], "f32", [986, 1408])
    s.transpose(q, [1, 0], "f32", [1408, 986])
    got, f = run_gpu(s.nodes, [x])
    assert f.plan()["hero"] == "transpose"
    assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "f32")
    s = W.Spec()
    p = s.parameter(0, "f32", [1000, 1536])
    t = s.transpose(p, [1, 0], "f32", [1536, 1000])
    q = s.slice(t, [5, 3], [1531, 999], [1, 1], "f32", [1526, 996])
    s.unary("negate", q, "f32", [1526, 996])
    got, f = run_gpu(s.nodes, [x])
    assert f.plan()["hero"] == "transpose"
    assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "f32")


@pytest.mark.parametrize("reducer", ["add", "max"])
def test_slice_reduces(reducer):
    """Row and column reduces of a slice; integer-valued inputs make the sums
    exact in any order, so both are bit-exact."""
    g = W.rng(404)
    x = ints_f32(g, 520 * 3000)
    init = 0.0 if reducer == "add" else float("-inf")
    for rdim, hero in ((1, "row_reduce"), (0, "column_reduce")):
        s = W.Spec()
        p = s.parameter(0, "f32", [520, 3000])
        q = s.slice(p, [5, 11], [515, 2990], [1, 1], "f32", [510, 2979])
        out = [2979] if rdim == 0 else [510]
        s.reduce(q, [rdim], reducer, init, "f32", out)
        got, f = run_gpu(s.nodes, [x])
        assert f.plan()["hero"] == hero
        assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "f32")


def _dyn_spec(dims, sizes, start_dtype, dtype="f32", then=None):
    s = W.Spec()
    p = s.parameter(0, dtype, dims)
    starts = [s.parameter(1 + d, start_dtype, []) for d in range(len(dims))]
    q = s.dynamic_slice(p, starts, sizes, dtype)
    if then:
        then(s, q)
    return s


def _start_buf(v, dtype):
    if dtype == "s4":
        return np.array([v & 0xF], np.uint8)
    return np.array(v, {"s32": np.int32, "u8": np.uint8, "s8": np.int8}[dtype])


@pytest.mark.parametrize("start_dtype", ["s32", "u8", "s4"])
def test_dynamic_slice_new_starts_every_launch(start_dtype):
    """One handle, launched with several start values -- in range, negative,
    past the end (both clamps) -- each bit-exact against the oracle.  The
    start indices are read on the device at every launch."""
    import torch
    import compiler_hlo_amd as H
    g = W.rng(405)
    dims, sizes = [300, 520], [64, 200]
    x = W.normal_f32(g, 300 * 520)
    s = _dyn_spec(dims, sizes, start_dtype,
                  then=lambda s, q: s.unary("negate", q, "f32", sizes))
    f = H.Fusion(s.nodes)
    dx = to_device(x)
    lo = {"s32": -50, "u8": 0, "s4": -8}[start_dtype]
    hi = {"s32": 700, "u8": 255, "s4": 7}[start_dtype]
    starts = [(0, 0), (5, 3), (lo, lo), (hi, hi), (min(236, hi), min(320, hi)), (min(100, hi), hi),
              (lo, min(17, hi))]
    for a, b in starts:
        ps = [x, _start_buf(a, start_dtype), _start_buf(b, start_dtype)]
        out = f(dx, to_device(ps[1]), to_device(ps[2]))
        torch.cuda.synchronize()
        assert_bitexact(from_device(out, "f32"), oracle.evaluate(s.nodes, ps), "f32")
    say("dynamic_slice", start_dtype, "launches:", len(starts))


def test_dynamic_slice_through_transpose_and_reduce():
    g = W.rng(406)
    x = ints_f32(g, 1000 * 1536)
    # transpose of a dynamic slice (ragged, misaligned start)
    s = _dyn_spec([1000, 1536], [900, 1300], "s32",
                  then=lambda s, q: s.transpose(q, [1, 0], "f32", [1300, 900]))
    for a, b in ((13, 77), (-5, 4000), (100, 236)):
        ps = [x, np.array(a, np.int32), np.array(b, np.int32)]
        got, f = run_gpu(s.nodes, ps)
        assert f.plan()["hero"] == "transpose"
        assert_bitexact(got, oracle.evaluate(s.nodes, ps), "f32")
    # row and column reduces of a dynamic slice
    for rdim, out, hero in ((1, [900], "row_reduce"), (0, [1300], "column_reduce")):
        s = _dyn_spec([1000, 1536], [900, 1300], "s32",
                      then=lambda s, q: s.reduce(q, [rdim], "add", 0.0, "f32", out))
        for a, b in ((13, 77), (99, 1)):
            ps = [x, np.array(a, np.int32), np.array(b, np.int32)]
            got, f = run_gpu(s.nodes, ps)
            assert f.plan()["hero"] == hero
            assert_bitexact(got, oracle.evaluate(s.nodes, ps), "f32")


def test_dynamic_slice_constant_starts_and_page_example():
    """The pages' 4x4 example (starts -1 and 3 clamp to 0 and 2), with the
    starts as constants and as parameters."""
    G = GOLD["dynamic_slice"]
    x = np.array(G["operand"], np.int32).astype(np.float32).ravel()
    for as_const in (True, False):
        s = W.Spec()
        p = s.parameter(0, "f32", [4, 4])
        if as_const:
            st = [s.constant(v, "s32", []) for v in G["start_indices"]]
            ps = [x]
        else:
            st = [s.parameter(1 + d, "s32", []) for d in range(2)]
            ps = [x] + [np.array(v, np.int32) for v in G["start_indices"]]
        s.dynamic_slice(p, st, G["slice_sizes"], "f32")
        got, _ = run_gpu(s.nodes, ps)
        assert got.reshape(2, 2).tolist() == G["result"]
        assert_bitexact(got, oracle.evaluate(s.nodes, ps), "f32")


def test_dynamic_slice_bf16_rank3_with_layouts():
    """A rank-3 bf16 operand stored column-major, sliced along every dim,
    negated and converted to f32 (both exact), written row-major."""
    g = W.rng(407)
    dims, sizes = [6, 130, 96], [3, 100, 64]
    x = W.normal_bf16(g, int(np.prod(dims)))
    s = W.Spec()
    p = s.parameter(0, "bf16", dims, [0, 1, 2])
    st = [s.parameter(1 + d, "s32", []) for d in range(3)]
    q = s.dynamic_slice(p, st, sizes, "bf16")
    n = s.unary("negate", q, "bf16", sizes)
    s.convert(n, "f32", sizes)
    for starts in ((1, 7, 9), (5, -2, 40), (2, 29, 32)):
        ps = [x] + [np.array(v, np.int32) for v in starts]
        got, _ = run_gpu(s.nodes, ps)
        assert_bitexact(got, oracle.evaluate(s.nodes, ps), "f32")
