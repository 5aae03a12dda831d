"""Pins of the CPU oracle against what the pages and mathematics fix.

Every test here runs on the CPU and checks the oracle against something other
than itself: values printed in the pages' worked examples (tests/golden/),
closed forms, library routines with the same definition (numpy transpose,
reshape, float32 arithmetic), exhaustive enumeration, and exact rational
arithmetic.  None of them re-types the oracle's own formula.
"""
import itertools
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import Spec, quant_type, rng, normal_f32

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_examples.json")))


def f32_bits(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


def ev(spec, params):
    return oracle.evaluate(spec.nodes, params)


# --------------------------------------------------------------------------
# Layout (Shapes and layout)
# --------------------------------------------------------------------------
def test_layout_2x3_example():
    g = GOLD["layout_2x3"]
    names = [c for row in g["logical"] for c in row]
    for m2m, key in (([0, 1], "m2m_0_1"), ([1, 0], "m2m_1_0")):
        mem = [None] * 6
        for i in range(2):
            for j in range(3):
                mem[oracle.linear_index([2, 3], m2m, [i, j])] = g["logical"][i][j]
        assert mem == g[key]
    # through evaluation: decode with {0,1}, re-encode with {1,0}
    phys = np.array([names.index(c) for c in g["m2m_0_1"]], dtype=np.float32)
    s = Spec()
    p = s.parameter(0, "f32", [2, 3], [0, 1])
    s.transpose(p, [0, 1], "f32", [2, 3], m2m=[1, 0])
    out = ev(s, [phys])
    assert [names[int(v)] for v in out] == g["m2m_1_0"]


def test_default_layout_is_major_to_minor():
    s = Spec()
    p = s.parameter(0, "f32", [2, 3, 4])
    s.transpose(p, [0, 1, 2], "f32", [2, 3, 4])
    x = np.arange(24, dtype=np.float32)
    # numpy's C order is major-to-minor: the identity re-encoding is a no-op
    assert np.array_equal(ev(s, [x]), x)


def test_loop_emitter_map_equals_row_major_linearization():
    """The loop emitter's (th_x, bl_x)[v] -> (i, j, k) map followed by the
    linear index with the default layout equals the page's flattened map
    th_x*4 + bl_x*512 + v, over the whole domain."""
    g = GOLD["loop_map_gelu"]
    th = np.arange(g["th_x"], dtype=np.int64)
    for bl0 in range(0, g["bl_x"], 4096):
        bl = np.arange(bl0, bl0 + 4096, dtype=np.int64)
        T, B, V = np.meshgrid(th, bl, np.arange(g["vec"]), indexing="ij")
        i, j = B // 4096, (B // 8) % 512
        k = (B % 8) * 512 + T * 4 + V
        idx = np.stack([i.ravel(), j.ravel(), k.ravel()], axis=1)
        lin = oracle.linear_indices(g["dims"], [2, 1, 0], idx)
        assert np.array_equal(lin, (T * 4 + B * 512 + V).ravel())


def test_layout_bijective_all_small_shapes():
    """For every shape of rank <= 3 with dims in {1,2,3} and every m2m, the
    linear index is a bijection onto [0, n) and matches numpy's reading of a
    buffer laid out major-to-minor in the order m2m reversed."""
    import itertools
    for rank in range(1, 4):
        for dims in itertools.product([1, 2, 3], repeat=rank):
            n = int(np.prod(dims))
            idx = np.array(list(itertools.product(*[range(d) for d in dims])), dtype=np.int64)
            for m2m in itertools.permutations(range(rank)):
                lin = oracle.linear_indices(list(dims), list(m2m), idx)
                assert sorted(lin.tolist()) == list(range(n))
                # numpy: physical buffer reshaped major->minor = dims[m2m[::-1]]
                buf = np.arange(n)
                phys = buf.reshape([dims[d] for d in m2m[::-1]])
                logical = np.transpose(phys, np.argsort(list(m2m[::-1])))
                assert np.array_equal(logical.reshape(-1), lin)


# --------------------------------------------------------------------------
# Indexing transforms
# --------------------------------------------------------------------------
def test_transpose_map_20x40():
    g = GOLD["transpose_map_20x40"]
    s = Spec()
    p = s.parameter(0, "f32", g["in_dims"], [1, 0])
    s.transpose(p, [1, 0], "f32", g["out_dims"], m2m=[1, 0])
    x = np.arange(800, dtype=np.float32)
    out = ev(s, [x]).reshape(g["out_dims"])
    xin = x.reshape(g["in_dims"])
    for d0 in range(40):
        for d1 in range(20):
            assert out[d0, d1] == xin[d1, d0]


def test_transpose_3d_shapes_and_non_involutions():
    """Transpose against numpy.transpose (same definition: result dim d is
    operand dim perm[d]) for every permutation of rank 3 and 4, including the
    non-involutions that distinguish a permutation from its inverse."""
    import itertools
    for dims in ([2, 3, 4], [2, 1, 3, 2]):
        x = np.arange(int(np.prod(dims)), dtype=np.float32)
        for perm in itertools.permutations(range(len(dims))):
            out_dims = [dims[p] for p in perm]
            s = Spec()
            p = s.parameter(0, "f32", dims)
            s.transpose(p, perm, "f32", out_dims)
            got = ev(s, [x]).reshape(out_dims)
            assert np.array_equal(got, np.transpose(x.reshape(dims), perm))
    g = GOLD["transpose_shapes_20x160x170"]
    assert [g["in_dims"][p] for p in (2, 1, 0)] == g["out_dims"]


def test_broadcast_in_dim_example():
    g = GOLD["broadcast_in_dim"]
    s = Spec()
    p = s.parameter(0, "f32", [1, 3])
    s.broadcast_in_dim(p, g["broadcast_dimensions"], "f32", g["result_dims"])
    out = ev(s, [np.array(g["operand"], dtype=np.float32).ravel()])
    assert out.reshape(g["result_dims"]).tolist() == g["result"]


def test_broadcast_against_numpy():
    """broadcast_in_dim of [3,1] into [2,3,4] with dims {1,2}: numpy broadcasting."""
    s = Spec()
    p = s.parameter(0, "f32", [3, 1])
    s.broadcast_in_dim(p, [1, 2], "f32", [2, 3, 4])
    x = np.array([7, 8, 9], dtype=np.float32)
    got = ev(s, [x]).reshape(2, 3, 4)
    assert np.array_equal(got, np.broadcast_to(x.reshape(1, 3, 1), (2, 3, 4)))


def test_reshape_examples():
    g = GOLD["reshape_2x3_to_3x2"]
    s = Spec()
    p = s.parameter(0, "f32", [2, 3])
    s.reshape(p, "f32", [3, 2])
    assert ev(s, [np.array(g["operand"], np.float32).ravel()]).reshape(3, 2).tolist() == g["result"]
    c = GOLD["collapse"]
    v = np.array(c["v"], dtype=np.float32).ravel()
    for key, dims in (("v012", [24]), ("v01", [4, 6]), ("v12", [8, 3])):
        s = Spec()
        p = s.parameter(0, "f32", [4, 2, 3])
        s.reshape(p, "f32", dims)
        assert ev(s, [v]).reshape(dims).tolist() == c[key]


def test_reshape_with_layouts_against_numpy():
    """Reshape is defined on logical order: with a column-major operand the
    result still follows numpy's C-order reshape of the logical array."""
    x = np.arange(24, dtype=np.float32)
    s = Spec()
    p = s.parameter(0, "f32", [4, 6], [0, 1])       # column-major storage
    s.reshape(p, "f32", [2, 12], m2m=[1, 0])
    logical = x.reshape(6, 4).T                     # numpy reading of {0,1}
    assert np.array_equal(ev(s, [x]).reshape(2, 12), logical.reshape(2, 12))


# --------------------------------------------------------------------------
# Elementwise arithmetic
# --------------------------------------------------------------------------
def _binary(op, lhs, rhs, dtype="f32"):
    lhs = np.asarray(lhs, dtype=np.float32)
    s = Spec()
    a = s.parameter(0, dtype, list(lhs.shape))
    b = s.parameter(1, dtype, list(lhs.shape))
    s.binary(op, a, b, dtype, list(lhs.shape))
    return ev(s, [lhs.ravel(), np.asarray(rhs, dtype=np.float32).ravel()]).reshape(lhs.shape)


@pytest.mark.parametrize("op", ["add", "multiply", "maximum"])
def test_integer_examples(op):
    g = GOLD[op]
    assert _binary(op, g["lhs"], g["rhs"]).tolist() == g["result"]


def test_f32_add_mul_match_ieee_float32():
    """f32 add/multiply/divide/subtract equal numpy's IEEE binary32 ops on random
    operands spanning many binades (including subnormal results)."""
    g = rng(11)
    a = (g.standard_normal(20000) * np.exp2(g.integers(-140, 100, 20000))).astype(np.float32)
    b = (g.standard_normal(20000) * np.exp2(g.integers(-140, 100, 20000))).astype(np.float32)
    with np.errstate(all="ignore"):
        for op, ref in (("add", a + b), ("multiply", a * b), ("subtract", a - b),
                        ("divide", a / b)):
            s = Spec()
            x = s.parameter(0, "f32", [a.size])
            y = s.parameter(1, "f32", [a.size])
            s.binary(op, x, y, "f32", [a.size])
            got = ev(s, [a, b])
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), op


def test_negate_abs_minimum_maximum_match_numpy():
    """negate and abs are exact sign operations; minimum and maximum of
    nonzero, non-NaN operands pick an operand (signed zeros and NaN are in the
    special-value test)."""
    g = rng(12)
    a = (g.standard_normal(20000) * np.exp2(g.integers(-140, 100, 20000))).astype(np.float32)
    b = (g.standard_normal(20000) * np.exp2(g.integers(-140, 100, 20000))).astype(np.float32)
    for op, ref in (("negate", -a), ("abs", np.abs(a))):
        s = Spec()
        x = s.parameter(0, "f32", [a.size])
        s.unary(op, x, "f32", [a.size])
        assert np.array_equal(ev(s, [a]).view(np.uint32), ref.view(np.uint32)), op
    for op, ref in (("minimum", np.minimum(a, b)), ("maximum", np.maximum(a, b))):
        s = Spec()
        x = s.parameter(0, "f32", [a.size])
        y = s.parameter(1, "f32", [a.size])
        s.binary(op, x, y, "f32", [a.size])
        assert np.array_equal(ev(s, [a, b]).view(np.uint32), ref.view(np.uint32)), op


def test_convert_s32_to_f32_and_rounding():
    g = GOLD["convert_s32_f32"]
    s = Spec()
    p = s.parameter(0, "s32", [3])
    s.convert(p, "f32", [3])
    assert ev(s, [np.array(g["input"], np.int32)]).tolist() == g["result"]
    # int -> float rounds to nearest even: 2^24+1 -> 2^24, 2^24+3 -> 2^24+4
    big = np.array([2 ** 24 + 1, 2 ** 24 + 3, -(2 ** 24) - 1], np.int32)
    s = Spec()
    p = s.parameter(0, "s32", [3])
    s.convert(p, "f32", [3])
    assert ev(s, [big]).tolist() == [2.0 ** 24, 2.0 ** 24 + 4, -(2.0 ** 24)]


def _bf16_value(bits):
    return float(oracle.bf16_bits_to_f32(np.array([bits], np.uint16))[0])


def _is_rne(exact: Fraction, r: float, p: int, emin: int) -> bool:
    """Property check of round-to-nearest-even to a p-bit format, with exact
    rationals: r is representable, no representable value is nearer, and at a
    tie r has an even last significand bit."""
    if r == 0:
        e = emin
    else:
        e = max(math.frexp(abs(r))[1] - 1, emin)
    q = Fraction(2) ** (e - (p - 1))
    fr = Fraction(r)
    m = fr / q
    if m.denominator != 1:
        return False
    err = abs(exact - fr)
    if err > q / 2:
        # r may sit at the bottom of a binade where the spacing below halves
        return False
    if err == q / 2 and int(m) % 2 != 0:
        return False
    # the lower neighbour inside a binade boundary has spacing q/2
    if r != 0 and abs(fr) == Fraction(2) ** e and e > emin:
        lower = abs(fr) - q / 2
        if abs(abs(exact) - lower) < err:
            return False
    return True


def test_f32_to_bf16_rne_pages_constants():
    """The GELU constants of the reproducer HLO round to the bf16 constants
    printed in the emitted function (XLA:GPU Emitters)."""
    g = GOLD["gelu_bf16_constants"]
    for v, printed in zip(g["hlo"], g["mlir_bf16_printed"]):
        s = Spec()
        s.constant(v, "bf16", [1])
        bits = int(ev(s, [])[0])
        val = _bf16_value(bits)
        # the printed 6-significant-digit value identifies a unique bf16
        assert abs(val - printed) <= 5e-7 * max(1.0, abs(printed)) + 1e-12, (v, val, printed)
        assert _is_rne(Fraction(np.float32(v).item()), val, 8, -126)
    # exact bit patterns implied by the printed values
    bits = []
    for v in g["hlo"]:
        s = Spec()
        s.constant(v, "bf16", [1])
        bits.append(int(ev(s, [])[0]))
    assert bits == [0x3F00, 0x3F80, 0x3F4C, 0x3D37]


def test_f32_to_bf16_convert_property_sample():
    """convert f32 -> bf16 is RNE: exact-rational property check on a sample
    of f32 patterns, including ties, subnormals and the overflow boundary."""
    g = rng(12)
    bits = g.integers(0, 2 ** 32, 4000, dtype=np.uint64).astype(np.uint32)
    extra = np.array([0x3F808000, 0x3F818000, 0x3F80C000, 0x00008000, 0x00018000,
                      0x7F7F7FFF, 0x7F7F8000, 0x80008000], np.uint32)
    bits = np.concatenate([bits, extra])
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    s = Spec()
    p = s.parameter(0, "f32", [f.size])
    s.convert(p, "bf16", [f.size])
    out = ev(s, [f])
    vals = oracle.bf16_bits_to_f32(out)
    maxbf = Fraction(2) ** 127 * (2 - Fraction(1, 128))
    for x, r in zip(f.tolist(), vals.tolist()):
        ex = Fraction(x)
        if math.isinf(r):
            assert abs(ex) >= maxbf + Fraction(2) ** (127 - 8), x
        else:
            assert _is_rne(ex, r, 8, -126), (x, r)


def test_reduce_precision_example():
    g = GOLD["reduce_precision_e5m10"]
    vals = [struct.unpack("<d", struct.pack("<Q", int(h, 16)))[0] if h.startswith("0x") else float(h)
            for h in g["input_hex"]]
    got = [oracle.round_format(v, 11, -14, 15) for v in vals]
    for x, want in zip(got, g["output"]):
        if want == "inf":
            assert math.isinf(x) and x > 0
        elif want == "nan":
            assert math.isnan(x)
        else:
            assert x == want


def test_exp_log_page_values():
    """exp and log of the printed examples: the oracle's f32 results are the
    f32 roundings of the page's f64 values."""
    for op, key in (("exponential", "exponential_f64"), ("log", "log_f64")):
        g = GOLD[key]
        x = np.array(g["input"], np.float32)
        s = Spec()
        p = s.parameter(0, "f32", [4])
        s.unary(op, p, "f32", [4])
        out = ev(s, [x])
        want = np.array(g["output"], dtype=np.float64).astype(np.float32)
        assert np.array_equal(out.view(np.uint32), want.view(np.uint32)), op
    assert [f32_bits(v) for v in np.array(GOLD["exponential_f64"]["output"]).astype(np.float32)] == \
        [0x3F800000, 0x402DF854, 0x40EC7326, 0x41A0AF2E]


def test_exp_bf16_exhaustive():
    """bf16 exp over all 65536 inputs is the RNE of exp(x): checked against
    numpy's float64 exp with a bound far below half a bf16 ulp."""
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = oracle.bf16_bits_to_f32(allbits)
    fin = np.isfinite(x)
    s = Spec()
    p = s.parameter(0, "bf16", [65536])
    s.unary("exponential", p, "bf16", [65536])
    out = oracle.bf16_bits_to_f32(ev(s, [allbits]))
    with np.errstate(over="ignore"):
        ref = np.exp(x.astype(np.float64))
    for xi, r, e in zip(x[fin].tolist(), out[fin].tolist(), ref[fin].tolist()):
        if math.isinf(e) or e > 3.3e38:
            assert math.isinf(r) or r >= 3.3e38
            continue
        if r == 0.0:
            assert e < 2.0 ** -133, xi
            continue
        ulp = 2.0 ** (max(math.frexp(r)[1] - 1, -126) - 7)
        assert abs(e - r) <= ulp * (0.5 + 1e-6), (xi, r, e)
    assert np.all(np.isnan(out[~fin & np.isnan(x)]))


@pytest.mark.parametrize("op,ref", [("tanh", np.tanh), ("log", np.log)])
def test_tanh_log_bf16_exhaustive(op, ref):
    """bf16 tanh and log over all 65536 inputs are the RNE of the exact value:
    within half a bf16 ulp (plus 1e-6 of one, for numpy's float64 error) of
    numpy's float64 result, the sign and zero of tanh kept (tanh(-0) = -0),
    log of a negative number NaN, log(+-0) = -inf, tanh(+-inf) = +-1."""
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = oracle.bf16_bits_to_f32(allbits)
    s = Spec()
    p = s.parameter(0, "bf16", [65536])
    s.unary(op, p, "bf16", [65536])
    out = oracle.bf16_bits_to_f32(ev(s, [allbits]))
    with np.errstate(divide="ignore", invalid="ignore"):
        want = ref(x.astype(np.float64))
    for xi, r, e in zip(x.tolist(), out.tolist(), want.tolist()):
        if math.isnan(e):
            assert math.isnan(r), (xi, r)
        elif math.isinf(e) or e == 0.0:
            assert r == e and math.copysign(1.0, r) == math.copysign(1.0, e), (xi, r, e)
        else:
            ulp = 2.0 ** (max(math.frexp(r)[1] - 1, -126) - 7)
            assert abs(e - r) <= ulp * (0.5 + 1e-6), (xi, r, e)
    if op == "tanh":
        m = ~np.isnan(x)
        assert np.array_equal(np.signbit(out[m]), np.signbit(x[m]))
        assert out[allbits == 0x7F80][0] == 1.0 and out[allbits == 0xFF80][0] == -1.0


@pytest.mark.parametrize("op,ref", [("exponential", np.exp), ("tanh", np.tanh), ("log", np.log)])
def test_exp_tanh_log_f16_exhaustive(op, ref):
    """f16 exp, tanh and log over all 65536 inputs are the RNE of the exact
    value: within half an f16 ulp (subnormal spacing 2^-24 below 2^-14) of
    numpy's float64 result, with overflow to +inf past the largest f16
    (65504, rounding boundary 65520), and the signs, zeros, infinities and
    NaNs of each op's definition."""
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = allbits.view(np.float16).astype(np.float32)
    s = Spec()
    p = s.parameter(0, "f16", [65536])
    s.unary(op, p, "f16", [65536])
    out = ev(s, [allbits]).view(np.float16).astype(np.float64)
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        want = ref(x.astype(np.float64))
    for xi, r, e in zip(x.tolist(), out.tolist(), want.tolist()):
        if math.isnan(e):
            assert math.isnan(r), (xi, r)
        elif math.isinf(e) or abs(e) >= 65520.0:
            assert math.isinf(r) and (r > 0) == (e > 0), (xi, r, e)
        elif e == 0.0:
            assert r == e and math.copysign(1.0, r) == math.copysign(1.0, e), (xi, r, e)
        else:
            ulp = 2.0 ** (max(math.frexp(abs(r) if r else 2.0 ** -24)[1] - 1, -14) - 10)
            assert abs(e - r) <= ulp * (0.5 + 1e-6), (xi, r, e)


# IEEE 754-2019 maximum and minimum over {NaN, -0, +0, -inf, +inf, 1.5},
# written out by hand (row = lhs, column = rhs): NaN propagates from either
# side, and -0 orders below +0.
_SPECIALS = [float("nan"), -0.0, 0.0, float("-inf"), float("inf"), 1.5]
_MAXIMUM_TABLE = [
    ["nan", "nan", "nan", "nan", "nan", "nan"],
    ["nan", "-0", "+0", "-0", "inf", "1.5"],
    ["nan", "+0", "+0", "+0", "inf", "1.5"],
    ["nan", "-0", "+0", "-inf", "inf", "1.5"],
    ["nan", "inf", "inf", "inf", "inf", "inf"],
    ["nan", "1.5", "1.5", "1.5", "inf", "1.5"],
]
_MINIMUM_TABLE = [
    ["nan", "nan", "nan", "nan", "nan", "nan"],
    ["nan", "-0", "-0", "-inf", "-0", "-0"],
    ["nan", "-0", "+0", "-inf", "+0", "+0"],
    ["nan", "-inf", "-inf", "-inf", "-inf", "-inf"],
    ["nan", "-0", "+0", "-inf", "inf", "1.5"],
    ["nan", "-0", "+0", "-inf", "1.5", "1.5"],
]


def _spelled(v: float) -> str:
    if math.isnan(v):
        return "nan"
    if v == 0:
        return "-0" if math.copysign(1, v) < 0 else "+0"
    if math.isinf(v):
        return "inf" if v > 0 else "-inf"
    return repr(v)


@pytest.mark.parametrize("op,table", [("maximum", _MAXIMUM_TABLE), ("minimum", _MINIMUM_TABLE)])
def test_maximum_minimum_special_value_tables(op, table):
    """StableHLO Specification, "maximum" / "minimum": the IEEE-754 operations
    (2019 edition: NaN-propagating, -0 < +0), against tables spelled out by
    hand."""
    vals = _SPECIALS
    a = np.array([v for v in vals for _ in vals], np.float32)
    b = np.array([w for _ in vals for w in vals], np.float32)
    got = _binary(op, a.reshape(6, 6), b.reshape(6, 6)).ravel()
    spelled = [_spelled(v) for v in got.tolist()]
    want = [c for row in table for c in row]
    assert spelled == want


@pytest.mark.parametrize("reducer,row,want", [
    ("min", [0.0, -0.0], "-0"), ("min", [-0.0, 0.0], "-0"), ("min", [0.0, 0.0], "+0"),
    ("min", [3.0, float("nan"), -5.0], "nan"), ("min", [float("nan")] * 3, "nan"),
    ("min", [float("inf"), float("inf")], "inf"), ("min", [], "inf"),
    ("max", [-0.0, 0.0], "+0"), ("max", [0.0, -0.0], "+0"), ("max", [-0.0, -0.0], "-0"),
    ("max", [3.0, float("nan"), -5.0], "nan"), ("max", [-5.0, 2.0, float("nan")], "nan"),
])
def test_reduce_min_max_signed_zeros_and_nan(reducer, row, want):
    """reduce with maximum / minimum (StableHLO Specification, "reduce"): the
    order-free fold of the IEEE operations from init (+inf for min, -inf for
    max).  Rows over {+0, -0} and rows holding NaN, spelled out by hand."""
    init = float("inf") if reducer == "min" else float("-inf")
    n = len(row)
    s = Spec()
    p = s.parameter(0, "f32", [1, n])
    s.reduce(p, [1], reducer, init, "f32", [1])
    got = ev(s, [np.array(row, np.float32)])
    assert _spelled(float(got[0])) == want


def test_special_values():
    """The special values of exp and log."""
    x = np.array([1.0, 0.0, -0.0, -1.0, float("inf"), float("nan")], np.float32)
    s = Spec()
    p = s.parameter(0, "f32", [6])
    s.unary("log", p, "f32", [6])
    lg = ev(s, [x])
    assert lg[0] == 0 and math.copysign(1, lg[0]) > 0
    assert lg[1] == -np.inf and lg[2] == -np.inf and np.isnan(lg[3])
    assert lg[4] == np.inf and np.isnan(lg[5])
    x = np.array([float("-inf"), float("inf"), float("nan"), 0.0, -200.0, 100.0], np.float32)
    s = Spec()
    p = s.parameter(0, "f32", [6])
    s.unary("exponential", p, "f32", [6])
    ex = ev(s, [x])
    assert ex[0] == 0 and math.copysign(1, ex[0]) > 0 and ex[1] == np.inf
    assert np.isnan(ex[2]) and ex[3] == 1.0 and ex[4] == 0.0 and ex[5] == np.inf


# --------------------------------------------------------------------------
# Reduce
# --------------------------------------------------------------------------
def test_reduce_examples():
    g = GOLD["reduce_sum_1x6"]
    s = Spec()
    p = s.parameter(0, "f32", [1, 6])
    s.reduce(p, g["dimensions"], "add", g["init"], "f32", [1])
    assert ev(s, [np.array(g["input"], np.float32).ravel()]).tolist() == g["result"]
    g = GOLD["reduce_3d"]
    x = np.tile(np.array(g["slice"], np.float32).ravel(), 4)
    for dims, out_dims, key in (([0], [2, 3], "dim0"), ([2], [4, 2], "dim2"),
                                ([0, 1], [3], "dims01"), ([0, 1, 2], [], "all")):
        s = Spec()
        p = s.parameter(0, "f32", [4, 2, 3])
        s.reduce(p, dims, "add", 0.0, "f32", out_dims)
        got = ev(s, [x])
        want = g[key]
        assert (got.reshape(out_dims).tolist() if out_dims else got[0]) == want


def test_reduce_exact_on_integers_any_layout():
    """Integer-valued inputs: sums are exact, so the oracle equals numpy's
    integer sum for every reduced-dimension choice and input layout."""
    import itertools
    g = rng(13)
    dims = [3, 4, 5]
    xi = g.integers(-4, 5, 60)
    x = xi.astype(np.float32)
    for m2m in itertools.permutations(range(3)):
        # physical buffer for layout m2m of the logical array xi.reshape(dims)
        phys = np.transpose(xi.reshape(dims), list(m2m[::-1])).ravel().astype(np.float32)
        for red in ([0], [1], [2], [0, 2], [1, 2]):
            kept = [d for d in range(3) if d not in red]
            s = Spec()
            p = s.parameter(0, "f32", dims, list(m2m))
            s.reduce(p, red, "add", 0.0, "f32", [dims[d] for d in kept])
            got = ev(s, [phys])
            assert np.array_equal(got, xi.reshape(dims).sum(axis=tuple(red)).ravel())
    assert x.size == 60


def test_reduce_max_any_order():
    g = rng(14)
    x = g.uniform(-100, 100, 3 * 50).astype(np.float32)
    s = Spec()
    p = s.parameter(0, "f32", [50, 3])
    s.reduce(p, [0], "max", float("-inf"), "f32", [3])
    assert np.array_equal(ev(s, [x]), x.reshape(50, 3).max(axis=0))


def test_reduce_sum_close_to_fsum():
    """f32 reduce-add equals math.fsum of the operands rounded to f32."""
    g = rng(15)
    x = normal_f32(g, 5000)
    s = Spec()
    p = s.parameter(0, "f32", [5000])
    s.reduce(p, [0], "add", 0.0, "f32", [])
    assert ev(s, [x])[0] == np.float32(math.fsum(x.astype(np.float64).tolist()))


# --------------------------------------------------------------------------
# Quantization (StableHLO Specification "Types"; StableHLO Quantization)
# --------------------------------------------------------------------------
def _dequant_spec(dims, q):
    s = Spec()
    p = s.parameter(0, "s8", dims, quant=q)
    s.op("uniform_dequantize", [p], "f32", dims)
    return s


def test_per_axis_dequantize_slices():
    g = GOLD["per_axis_type"]
    q = quant_type("s8", g["scales"], g["zero_points"], qdim=g["qdim"])
    allq = np.arange(-128, 128, dtype=np.int8)
    # every q value appears in every slice t[:, j, :]
    x = np.resize(allq, 4 * 3 * 2 * 11)[: 4 * 3 * 2]
    for shift in range(0, 256, 24):
        xs = np.roll(allq, shift)[:24].astype(np.int8)
        out = ev(_dequant_spec(g["dims"], q), [xs]).reshape(g["dims"])
        xl = xs.reshape(g["dims"])
        for j in range(3):
            sc = np.float32(g["scales"][j])
            want = sc * (xl[:, j, :].astype(np.float32) - np.float32(g["zero_points"][j]))
            assert np.array_equal(out[:, j, :].view(np.uint32), want.astype(np.float32).view(np.uint32))
    assert x.size == 24
    # specific values: each slice's zero point maps to 0.0
    xs = np.broadcast_to(np.array([20, 10, 30], np.int8).reshape(1, 3, 1), (4, 3, 2)).copy()
    assert np.all(ev(_dequant_spec(g["dims"], q), [xs.ravel()]) == 0.0)


def test_per_tensor_dequantize_example_type():
    g = GOLD["per_tensor_type"]
    q = quant_type("s8", [g["scale"]], [g["zero_point"]])
    xs = np.array([50, 0, 127, -128], np.int8)
    out = ev(_dequant_spec([4], q), [xs])
    want = np.float32(g["scale"]) * (xs.astype(np.float32) - np.float32(g["zero_point"]))
    assert np.array_equal(out, want.astype(np.float32))
    assert out[0] == 0.0 and out[1] == np.float32(-0.5)


def _quant_spec(n, q, src="f32"):
    s = Spec()
    p = s.parameter(0, src, [n])
    s.op("uniform_quantize", [p], "s8", [n], quant=q)
    return s


def test_quantize_ties_to_even():
    g = GOLD["round_nearest_even"]
    q = quant_type("s8", [1.0], [0])
    out = ev(_quant_spec(5, q), [np.array(g["input"], np.float32)])
    assert out.tolist() == [int(v) for v in g["even"]]
    assert out.tolist() != [int(v) for v in g["afz"]]


def test_quantize_clamp_example():
    g = GOLD["clamp"]
    q = quant_type("s8", [1.0], [0], storage_min=g["min"], storage_max=g["max"])
    out = ev(_quant_spec(3, q), [np.array(g["operand"], np.float32)])
    assert out.tolist() == g["result"]


def test_quantize_divides_then_rounds_then_adds_zero_point():
    """Reading adopted for uniform_quantize: t = f32(y / scale) by IEEE
    division, ties-to-even, zero point added as an integer, then clamp.
    Checked against numpy's float32 division and rint on many values, and on
    the cases where dividing and multiplying by the reciprocal differ."""
    g = rng(16)
    y = (g.standard_normal(200000) * 2.0).astype(np.float32)
    for scale, zp in ((0.02, 0), (0.02, 7), (0.0137, -20)):
        q = quant_type("s8", [scale], [zp])
        got = ev(_quant_spec(y.size, q), [y]).astype(np.int64)
        t = (y / np.float32(scale)).astype(np.float32)
        want = np.clip(np.rint(t).astype(np.int64) + zp, -128, 127)
        assert np.array_equal(got, want)
    # zero point after rounding: 0.5 + 7 -> rint(0.5) + 7 = 7, not rint(7.5) = 8
    q = quant_type("s8", [1.0], [7])
    assert ev(_quant_spec(1, q), [np.array([0.5], np.float32)]).tolist() == [7]
    # Near the rounding ties, dividing by the scale and multiplying by its
    # rounded reciprocal give different integers; the oracle must divide.
    sc = np.float32(0.02)
    centers = ((np.arange(-130, 130) + 0.5) * 0.02).astype(np.float32).view(np.int32)
    yt = np.concatenate([(centers + off).view(np.float32) for off in range(-40, 41)])
    recip = (yt * (np.float32(1.0) / sc)).astype(np.float32)
    diff = np.rint(yt / sc) != np.rint(recip)
    assert diff.sum() > 10
    q = quant_type("s8", [0.02], [0])
    got = ev(_quant_spec(yt.size, q), [yt]).astype(np.int64)
    assert np.array_equal(got, np.clip(np.rint(yt / sc).astype(np.int64), -128, 127))


def test_requantize_identity_per_axis():
    """quantize(dequantize(q)) == q for every storage value and slice of the
    pages' per-axis type (t[4,3,2], qdim 1, {0.2:20, 0.1:10, 0.3:30})."""
    g = GOLD["per_axis_type"]
    qa = quant_type("s8", g["scales"], g["zero_points"], qdim=1)
    allq = np.arange(-128, 128, dtype=np.int8)
    for j in range(3):
        dims = [256, 3, 1]
        x = np.zeros((256, 3, 1), np.int8)
        x[:, :, 0] = allq[:, None]
        s = Spec()
        p = s.parameter(0, "s8", dims, quant=qa)
        d = s.op("uniform_dequantize", [p], "f32", dims)
        s.op("uniform_quantize", [d], "s8", dims, quant=qa)
        out = ev(s, [x.ravel()])
        assert np.array_equal(out, x.ravel()), j


def test_requantize_direct():
    """uniform_quantize of a quantized operand (requantize) dequantizes first."""
    qi = quant_type("s8", [0.1], [3])
    qo = quant_type("s8", [0.05], [-2])
    x = np.arange(-128, 128, dtype=np.int8)
    s = Spec()
    p = s.parameter(0, "s8", [256], quant=qi)
    s.op("uniform_quantize", [p], "s8", [256], quant=qo)
    got = ev(s, [x]).astype(np.int64)
    deq = (np.float32(0.1) * (x.astype(np.float32) - np.float32(3))).astype(np.float32)
    want = np.clip(np.rint((deq / np.float32(0.05)).astype(np.float32)).astype(np.int64) - 2, -128, 127)
    assert np.array_equal(got, want)


# --------------------------------------------------------------------------
# f16 and u8 (element types beyond the configs)
# --------------------------------------------------------------------------
def test_f16_convert_and_add_match_numpy_float16():
    """f32 -> f16 rounds to nearest even (numpy's float16 conversion); f16 add
    is the f32 sum of the operands rounded to f16 (exact in f32 before the
    rounding, so it is the correctly rounded f16 sum)."""
    g = rng(121)
    x = np.concatenate([g.standard_normal(4000).astype(np.float32) * 300,
                        np.array([65504, 65519.99, 65520, 6.1e-5, 5.96e-8, 2.98e-8, -0.0], np.float32)])
    s = Spec()
    p = s.parameter(0, "f32", [x.size])
    s.convert(p, "f16", [x.size])
    got = ev(s, [x])
    assert np.array_equal(got.view(np.uint16), x.astype(np.float16).view(np.uint16))
    a = (g.standard_normal(4000) * 30).astype(np.float16)
    b = (g.standard_normal(4000) * 30).astype(np.float16)
    s = Spec()
    pa = s.parameter(0, "f16", [4000])
    pb = s.parameter(1, "f16", [4000])
    s.binary("add", pa, pb, "f16", [4000])
    got = ev(s, [a.view(np.uint16), b.view(np.uint16)])
    assert np.array_equal(got.view(np.uint16), (a + b).view(np.uint16))


def test_u8_quantize_range_and_zero_point():
    """u8 storage: [0, 255]; zero point 128 puts real 0 mid-range."""
    q = quant_type("u8", [0.5], [128])
    y = np.array([0.0, 0.25, 0.75, -64.0, -64.25, -64.5, 63.5, 63.75, 1e6, -1e6], np.float32)
    s = Spec()
    p = s.parameter(0, "f32", [y.size])
    s.op("uniform_quantize", [p], "u8", [y.size], quant=q)
    got = ev(s, [y]).astype(np.int64).tolist()
    assert got == [128, 128, 130, 0, 0, 0, 255, 255, 255, 0]


# --------------------------------------------------------------------------
# si4 / ui4 (Specification, "Types": 4-bit integers).  Packing reading: two
# elements per byte in physical order, the even linear index in the low four
# bits.  The expected values are worked by hand from that reading.
# --------------------------------------------------------------------------
def test_s4_u4_decode_worked_bytes():
    raw = np.array([0x21, 0xF8, 0x7E], np.uint8)
    for dt, want in (("s4", [1, 2, -8, -1, -2, 7]), ("u4", [1, 2, 8, 15, 14, 7])):
        s = Spec()
        p = s.parameter(0, dt, [6])
        s.convert(p, "f32", [6])
        assert ev(s, [raw]).tolist() == want
    # the same bytes as a [2,3] array stored column-major: linear order is
    # (0,0) (1,0) (0,1) (1,1) (0,2) (1,2)
    s = Spec()
    p = s.parameter(0, "s4", [2, 3], [0, 1])
    s.convert(p, "f32", [2, 3], [1, 0])
    assert ev(s, [raw]).reshape(2, 3).tolist() == [[1, -8, -2], [2, -1, 7]]


def test_s4_u4_round_trip_every_byte():
    """Decoding then encoding every byte value gives it back; an odd count
    leaves the last byte's high nibble zero."""
    raw = np.arange(256, dtype=np.uint8)
    for dt in ("s4", "u4"):
        s = Spec()
        s.parameter(0, dt, [512])
        assert np.array_equal(ev(s, [raw]), raw)
        s = Spec()
        p = s.parameter(0, dt, [512])
        s.convert(p, "f32", [512])
        vals = ev(s, [raw])
        lo, hi = raw & 0xF, raw >> 4
        if dt == "s4":
            lo = np.where(lo >= 8, lo.astype(np.int64) - 16, lo)
            hi = np.where(hi >= 8, hi.astype(np.int64) - 16, hi)
        assert np.array_equal(vals, np.stack([lo, hi], 1).ravel().astype(np.float32))
    q = quant_type("s4", [1.0], [0])
    s = Spec()
    p = s.parameter(0, "f32", [3])
    s.op("uniform_quantize", [p], "s4", [3], quant=q)
    assert ev(s, [np.array([-1.0, 3.0, -8.0], np.float32)]).tolist() == [0x3F, 0x08]


def test_s4_u4_quantize_rounds_clamps_and_packs():
    y = np.array([-100.0, -8.4, -7.6, -0.5, 0.5, 1.5, 6.6, 100.0], np.float32)
    for dt, zp, want in (("s4", 0, [0x88, 0x08, 0x20, 0x77]), ("u4", 8, [0x00, 0x80, 0xA8, 0xFF])):
        q = quant_type(dt, [1.0], [zp])
        s = Spec()
        p = s.parameter(0, "f32", [y.size])
        s.op("uniform_quantize", [p], dt, [y.size], quant=q)
        assert ev(s, [y]).tolist() == want
    # per-axis dequantize of si4 along dim 1 with scales (0.5, 0.25) and zero
    # points (1, -2): real = scale * (q - zp)
    q = quant_type("s4", [0.5, 0.25], [1, -2], qdim=1)
    s = Spec()
    p = s.parameter(0, "s4", [2, 2], quant=q)
    s.op("uniform_dequantize", [p], "f32", [2, 2])
    # bytes: row 0 = (7, -8) -> 0x87; row 1 = (-1, 2) -> 0x2F
    assert ev(s, [np.array([0x87, 0x2F], np.uint8)]).reshape(2, 2).tolist() == [[3.0, -1.5], [-1.0, 1.0]]


# --------------------------------------------------------------------------
# Index transforms (StableHLO Specification: reverse, iota, pad, concatenate)
# --------------------------------------------------------------------------
def test_reverse_iota_pad_concatenate_page_examples():
    G = GOLD["reverse"]
    x = np.array(G["operand"], np.int32)
    s = Spec()
    p = s.parameter(0, "s32", list(x.shape))
    s.reverse(p, G["dimensions"], "s32", list(x.shape))
    assert ev(s, [x]).reshape(x.shape).tolist() == G["result"]
    G = GOLD["iota"]
    for d, key in ((0, "dim0"), (1, "dim1")):
        s = Spec()
        s.iota(d, "s32", G["dims"])
        assert ev(s, []).reshape(G["dims"]).tolist() == G[key]
    G = GOLD["pad"]
    x = np.array(G["operand"], np.int32)
    s = Spec()
    p = s.parameter(0, "s32", list(x.shape))
    v = s.parameter(1, "s32", [])
    out = np.array(G["result"])
    s.pad(p, v, G["edge_padding_low"], G["edge_padding_high"], G["interior_padding"], "s32", list(out.shape))
    assert ev(s, [x, np.array(G["padding_value"], np.int32)]).reshape(out.shape).tolist() == G["result"]
    G = GOLD["concatenate"]
    a, b = np.array(G["input0"], np.int32), np.array(G["input1"], np.int32)
    s = Spec()
    pa = s.parameter(0, "s32", list(a.shape))
    pb = s.parameter(1, "s32", list(b.shape))
    s.concatenate([pa, pb], G["dimension"], "s32", [4, 2])
    assert ev(s, [a, b]).reshape(4, 2).tolist() == G["result"]


def _np_pad(x, pv, lo, hi, interior):
    """Interior padding by strided assignment, then edges: np.pad for positive
    amounts and slicing for negative ones."""
    inner = [(n - 1) * (i + 1) + 1 if n else 0 for n, i in zip(x.shape, interior)]
    y = np.full(inner, pv, x.dtype)
    y[tuple(slice(None, None, i + 1) for i in interior)] = x
    y = np.pad(y, [(max(l, 0), max(h, 0)) for l, h in zip(lo, hi)], constant_values=pv)
    return y[tuple(slice(-min(l, 0), y.shape[d] + min(h, 0)) for d, (l, h) in enumerate(zip(lo, hi)))]


def test_index_transforms_against_numpy():
    g = rng(71)
    for shape in [(2, 3), (3, 1, 4), (5,), (2, 2, 2, 3)]:
        x = g.standard_normal(shape).astype(np.float32)
        r = len(shape)
        for dims in itertools.chain.from_iterable(itertools.combinations(range(r), k) for k in range(r + 1)):
            s = Spec()
            p = s.parameter(0, "f32", list(shape))
            s.reverse(p, dims, "f32", list(shape))
            assert np.array_equal(ev(s, [x]).reshape(shape), np.flip(x, dims) if dims else x)
        for d in range(r):
            s = Spec()
            s.iota(d, "f32", list(shape))
            want = np.broadcast_to(np.arange(shape[d]).reshape([-1 if k == d else 1 for k in range(r)]), shape)
            assert np.array_equal(ev(s, []).reshape(shape), want.astype(np.float32))
            other = list(shape)
            other[d] = 2
            y = g.standard_normal(other).astype(np.float32)
            out = list(shape)
            out[d] += 2
            s = Spec()
            pa = s.parameter(0, "f32", list(shape))
            pb = s.parameter(1, "f32", other)
            s.concatenate([pa, pb, pa], d, "f32", [out[k] + (shape[d] if k == d else 0) for k in range(r)])
            assert np.array_equal(ev(s, [x, y]).reshape(np.concatenate([x, y, x], d).shape),
                                  np.concatenate([x, y, x], d))
        for _ in range(6):
            lo = g.integers(-1, 3, r).tolist()
            hi = g.integers(-1, 3, r).tolist()
            it = g.integers(0, 3, r).tolist()
            out = [n + l + max(n - 1, 0) * i + h for n, l, h, i in zip(shape, lo, hi, it)]
            if min(out) < 1:
                continue
            s = Spec()
            p = s.parameter(0, "f32", list(shape))
            v = s.parameter(1, "f32", [])
            s.pad(p, v, lo, hi, it, "f32", out)
            want = _np_pad(x, np.float32(-7.5), lo, hi, it)
            assert np.array_equal(ev(s, [x, np.array(-7.5, np.float32)]).reshape(out), want)


# --------------------------------------------------------------------------
# slice and dynamic_slice (StableHLO Specification, "dynamic_slice";
# Operation semantics, DynamicSlice; the start_indices / limit_indices
# attributes of slice in "Programs")
# --------------------------------------------------------------------------
@pytest.mark.parametrize("key,dtype", [("dynamic_slice", "s32"), ("dynamic_slice_1d", "f32"),
                                       ("dynamic_slice_2d", "f32")])
@pytest.mark.parametrize("starts_as", ["parameters", "constants"])
def test_dynamic_slice_page_examples(key, dtype, starts_as):
    G = GOLD[key]
    x = np.array(G["operand"], {"s32": np.int32, "f32": np.float32}[dtype])
    s = Spec()
    p = s.parameter(0, dtype, list(x.shape))
    params = [x]
    starts = []
    for d, v in enumerate(G["start_indices"]):
        if starts_as == "parameters":
            starts.append(s.parameter(1 + d, "s32", []))
            params.append(np.array(v, np.int32))
        else:
            starts.append(s.constant(v, "s32", []))
    s.dynamic_slice(p, starts, G["slice_sizes"], dtype)
    assert ev(s, params).reshape(G["slice_sizes"]).tolist() == G["result"]


def test_dynamic_slice_clamps_starts_against_numpy():
    """Brute force on small shapes: every start from -3 to dim + 2 (so both
    clamps are hit) and every size 0..dim, against numpy basic slicing of
    the start clamped into [0, dim - size]."""
    g = rng(73)
    for shape in [(5,), (3, 4), (2, 3, 4)]:
        x = g.standard_normal(shape).astype(np.float32)
        r = len(shape)
        for _ in range(40):
            sizes = [int(g.integers(0, n + 1)) for n in shape]
            starts = [int(g.integers(-3, n + 3)) for n in shape]
            s = Spec()
            p = s.parameter(0, "f32", list(shape))
            st = [s.parameter(1 + d, "s32", []) for d in range(r)]
            s.dynamic_slice(p, st, sizes, "f32")
            got = ev(s, [x] + [np.array(v, np.int32) for v in starts]).reshape(sizes)
            lo = [min(max(v, 0), n - z) for v, n, z in zip(starts, shape, sizes)]
            want = x[tuple(slice(a, a + z) for a, z in zip(lo, sizes))]
            assert np.array_equal(got, want), (shape, starts, sizes)


def test_slice_against_numpy_strides_and_layouts():
    """slice(x, start, limit, strides) = x[start:limit:strides] per dim, the
    result shape ceil((limit - start) / strides); operand and result in
    row-major and column-major layouts."""
    g = rng(74)
    for shape in [(7,), (5, 6), (3, 4, 5)]:
        x = g.standard_normal(shape).astype(np.float32)
        r = len(shape)
        for _ in range(30):
            start = [int(g.integers(0, n + 1)) for n in shape]
            limit = [int(g.integers(a, n + 1)) for a, n in zip(start, shape)]
            strides = [int(g.integers(1, 4)) for _ in shape]
            out = [-(-(b - a) // k) for a, b, k in zip(start, limit, strides)]
            want = x[tuple(slice(a, b, k) for a, b, k in zip(start, limit, strides))]
            assert list(want.shape) == out
            for m2m_in, m2m_out in ((None, None), (list(range(r)), None), (None, list(range(r)))):
                s = Spec()
                p = s.parameter(0, "f32", list(shape), m2m_in)
                s.slice(p, start, limit, strides, "f32", out, m2m_out)
                xin = x.ravel() if m2m_in is None else x.transpose().ravel()
                got = ev(s, [xin])
                got = got.reshape(out) if m2m_out is None else got.reshape(out[::-1]).transpose()
                assert np.array_equal(got, want), (shape, start, limit, strides, m2m_in, m2m_out)


def test_slice_equals_dynamic_slice_with_constant_starts():
    g = rng(75)
    x = g.standard_normal((6, 9)).astype(np.float32)
    for start, size in (([1, 2], [3, 5]), ([0, 0], [6, 9]), ([5, 8], [1, 1]), ([2, 3], [0, 4])):
        a = Spec()
        p = a.parameter(0, "f32", [6, 9])
        a.slice(p, start, [s + z for s, z in zip(start, size)], [1, 1], "f32", size)
        b = Spec()
        p = b.parameter(0, "f32", [6, 9])
        c = [b.constant(v, "s32", []) for v in start]
        b.dynamic_slice(p, c, size, "f32")
        assert np.array_equal(ev(a, [x]), ev(b, [x]))


# --------------------------------------------------------------------------
# Variadic max/argmax reduce (Operation semantics, "Variadic Reduce")
# --------------------------------------------------------------------------
def _argmax_spec(dims, rdim, dtype="f32", init=float("-inf"), index_init=-1):
    s = Spec()
    p = s.parameter(0, dtype, list(dims))
    k = s.iota(rdim, "s32", list(dims))
    out = [d for i, d in enumerate(dims) if i != rdim]
    s.op("reduce", [p, k], "s32", out, dimensions=[rdim], reducer="argmax", init=init, index_init=index_init)
    return s


def test_argmax_is_the_last_index_of_the_maximum():
    """The fold f(max, argmax, v, i) = v >= max ? (v, i) : (max, argmax) in
    index order keeps the LAST index of the maximum: n - 1 - argmax of the
    reversed row (numpy's argmax keeps the first)."""
    g = rng(101)
    x = g.integers(-5, 5, (40, 33)).astype(np.float32)   # many ties
    for rdim in (0, 1):
        got = ev(_argmax_spec(x.shape, rdim), [x]).astype(np.int64)
        n = x.shape[rdim]
        want = n - 1 - np.argmax(np.flip(x, rdim), axis=rdim)
        assert np.array_equal(got, want)


def test_argmax_skips_nan_and_takes_values_equal_to_init():
    nan, ninf = float("nan"), float("-inf")
    rows = np.array([[1, nan, 3, nan, 3], [nan] * 5, [ninf, ninf, 2, ninf, ninf], [ninf] * 5], np.float32)
    got = ev(_argmax_spec(rows.shape, 1, index_init=-1), [rows]).astype(np.int64).tolist()
    assert got == [4, -1, 2, 4]


def test_argmax_with_an_index_init_inside_the_row():
    """Operation semantics, "Variadic Reduce": the fold starts from
    (init_value, index init) and an element replaces the running pair when
    value >= max.  With value init 2 and index init 7 (worked by hand): a
    row whose maximum equals the value init returns the last index holding
    it; a row that never reaches the init, or holds only NaN, returns 7."""
    nan = float("nan")
    rows = np.array([[1, 2, 0, 2, 1], [1, 0, 1, 0, 1], [nan] * 5, [3, 2, 3, 1, 2], [2, nan, 2, nan, nan]],
                    np.float32)
    got = ev(_argmax_spec(rows.shape, 1, init=2.0, index_init=7), [rows]).astype(np.int64).tolist()
    assert got == [3, 7, 7, 2, 2]
    got = ev(_argmax_spec(rows.shape, 1, init=2.0, index_init=0), [rows]).astype(np.int64).tolist()
    assert got == [3, 0, 0, 2, 2]


# --------------------------------------------------------------------------
# Elementwise ops on quantized tensors (StableHLO Specification, each op's
# semantics for quantized types: dequantize, op, quantize)
# --------------------------------------------------------------------------
def _qop(op, qts, xs, qout):
    s = Spec()
    ps = [s.parameter(k, "s8", [len(xs[0])], quant=qt) for k, qt in enumerate(qts)]
    s.op(op, ps, "s8", [len(xs[0])], quant=qout)
    return ev(s, xs).astype(np.int64)


def test_quantized_add_with_a_shared_power_of_two_scale_is_integer_addition():
    """scale 2^-2, zero point 0 everywhere: the reals are exact, their sum is
    exact, and dividing by the scale gives back q1 + q2 (clamped)."""
    qt = quant_type("s8", [0.25], [0])
    g = rng(51)
    a = g.integers(-128, 128, 4000).astype(np.int8)
    b = g.integers(-128, 128, 4000).astype(np.int8)
    got = _qop("add", [qt, qt], [a, b], qt)
    assert np.array_equal(got, np.clip(a.astype(np.int64) + b, -128, 127))


def test_quantized_maximum_minimum_with_one_type_are_storage_max_min():
    """dequantize is increasing and quantize(dequantize(q)) = q for one type
    (pinned by the per-axis requantize-identity test), so max/min of the
    reals come back as max/min of the storage values."""
    qt = quant_type("s8", [0.1], [5])
    a = np.arange(-128, 128, dtype=np.int8).repeat(256)
    b = np.tile(np.arange(-128, 128, dtype=np.int8), 256)
    assert np.array_equal(_qop("maximum", [qt, qt], [a, b], qt), np.maximum(a, b).astype(np.int64))
    assert np.array_equal(_qop("minimum", [qt, qt], [a, b], qt), np.minimum(a, b).astype(np.int64))


def test_quantized_negate_abs_with_zero_point_zero():
    qt = quant_type("s8", [0.3], [0])
    x = np.arange(-128, 128, dtype=np.int8)
    assert np.array_equal(_qop("negate", [qt], [x], qt), np.clip(-x.astype(np.int64), -128, 127))
    assert np.array_equal(_qop("abs", [qt], [x], qt), np.clip(np.abs(x.astype(np.int64)), -128, 127))


def test_quantized_add_worked_values_and_ties():
    """Different scales: 3*0.5 + 2*0.25 = 2.0 -> 2.0/0.5 + 1 = 5; and a sum
    that lands on a half-integer multiple of the result scale rounds to even:
    (1.5 + 1.0)/1.0 = 2.5 -> 2, (0.5 + 1.0)/1.0 = 1.5 -> 2."""
    a_t, b_t = quant_type("s8", [0.5], [0]), quant_type("s8", [0.25], [0])
    got = _qop("add", [a_t, b_t], [np.array([3], np.int8), np.array([2], np.int8)], quant_type("s8", [0.5], [1]))
    assert got.tolist() == [5]
    got = _qop("add", [a_t, a_t], [np.array([3, 1], np.int8), np.array([2, 2], np.int8)], quant_type("s8", [1.0], [0]))
    assert got.tolist() == [2, 2]


# --------------------------------------------------------------------------
# The pages' example program (StableHLO Specification, "Programs")
# --------------------------------------------------------------------------
def test_program_28x28_selection_weights():
    g = rng(17)
    image = g.uniform(-1, 1, 784).astype(np.float32)
    bias = g.uniform(-1, 1, 10).astype(np.float32)
    sel = g.choice(784, 10, replace=False)
    w = np.zeros((784, 10), np.float32)
    w[sel, np.arange(10)] = 1.0
    s = Spec()
    im = s.parameter(0, "f32", [28, 28])
    wt = s.parameter(1, "f32", [784, 10])
    bs = s.parameter(2, "f32", [1, 10])
    r = s.reshape(im, "f32", [1, 784])
    d = s.op("dot", [r, wt], "f32", [1, 10])
    a = s.binary("add", d, bs, "f32", [1, 10])
    z = s.constant(0.0, "f32", [1, 10])
    s.binary("maximum", a, z, "f32", [1, 10])
    out = ev(s, [image, w.ravel(), bias])
    want = np.maximum(image[sel] + bias, np.float32(0))
    assert np.array_equal(out, want)


def test_evaluate_points_matches_whole():
    s = Spec()
    p = s.parameter(0, "f32", [5, 7], [0, 1])
    e = s.unary("exponential", p, "f32", [5, 7])
    s.reduce(e, [1], "add", 0.0, "f32", [5])
    x = normal_f32(rng(18), 35)
    whole = ev(s, [x])
    vals, aux = oracle.evaluate_points(s.nodes, [x], [[i] for i in range(5)])
    assert np.array_equal(vals.astype(np.float32), whole)
    xl = x.reshape(7, 5).T.astype(np.float64)
    assert np.allclose(aux[:, 0], np.abs(np.exp(xl.astype(np.float32))).sum(axis=1), rtol=1e-6)


def test_exp_log_f32_correctly_rounded_sample():
    """f32 exp, log and tanh are correctly rounded: equal to numpy's float64 result
    rounded to f32 wherever that f64 value is not within 1e-12 (relative) of
    an f32 rounding boundary."""
    g = rng(19)
    for op, x, ref in (
        ("exponential", g.uniform(-87, 88, 100000).astype(np.float32), np.exp),
        ("log", np.exp2(g.uniform(-140, 127, 100000)).astype(np.float32), np.log),
        ("tanh", (g.standard_normal(100000) * np.exp2(g.integers(-12, 3, 100000))).astype(np.float32), np.tanh),
    ):
        s = Spec()
        p = s.parameter(0, "f32", [x.size])
        s.unary(op, p, "f32", [x.size])
        got = ev(s, [x])
        r64 = ref(x.astype(np.float64))
        want = r64.astype(np.float32)
        # distance of the f64 value to the midpoint between want and its neighbour
        nb = np.nextafter(want, np.where(r64 > want, np.inf, -np.inf).astype(np.float32))
        mid = (want.astype(np.float64) + nb.astype(np.float64)) / 2
        safe = np.abs(r64 - mid) > 1e-12 * np.abs(r64)
        assert safe.mean() > 0.999
        assert np.array_equal(got[safe].view(np.uint32), want[safe].view(np.uint32)), op
