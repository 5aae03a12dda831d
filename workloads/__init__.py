"""Seeded synthetic inputs and neutral fusion descriptions.

The tests, the benchmark and the smoke check use this module to build the
inputs and the node lists that they hand both to the product binding and to
the oracle; neither of those two imports it.  It holds NO arithmetic of the method: no layout mapping, no
rounding, no op semantics.  It only

  * draws random buffers from numpy's PCG64 with fixed seeds, directly in
    physical (storage) order -- the values are i.i.d., so their distribution
    does not depend on the layout the fusion declares for them; and
  * writes fusions down as plain node lists (dicts), each node stating its own
    result type the way HLO text does.

bf16 inputs are drawn as float32 and keep the upper 16 bits of the float32
pattern (truncation), which defines a bf16 distribution without using the
method's round-to-nearest-even conversion.
"""
from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------
# generators
# --------------------------------------------------------------------------
def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def uniform_f32(g: np.random.Generator, n: int, lo: float, hi: float) -> np.ndarray:
    return g.uniform(lo, hi, size=n).astype(np.float32)


def normal_f32(g: np.random.Generator, n: int, sigma: float = 1.0) -> np.ndarray:
    return (g.standard_normal(size=n) * sigma).astype(np.float32)


def normal_bf16(g: np.random.Generator, n: int, sigma: float = 1.0) -> np.ndarray:
    """bf16 bit patterns (uint16): upper half of a float32 normal draw."""
    f = normal_f32(g, n, sigma)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def integers(g: np.random.Generator, n: int, lo: int, hi: int, dtype) -> np.ndarray:
    """Uniform integers in [lo, hi] inclusive."""
    return g.integers(lo, hi, size=n, endpoint=True).astype(dtype)


# --------------------------------------------------------------------------
# node-list recorder (no shape inference: every node states its type)
# --------------------------------------------------------------------------
class Spec:
    def __init__(self):
        self.nodes: list[dict] = []

    def _add(self, **nd) -> int:
        self.nodes.append(nd)
        return len(self.nodes) - 1

    def parameter(self, index, dtype, dims, m2m=None, quant=None) -> int:
        return self._add(op="parameter", param=index, operands=[], dtype=dtype,
                         dims=list(dims), m2m=m2m, quant=quant)

    def constant(self, value, dtype, dims) -> int:
        return self._add(op="constant", operands=[], value=float(value), dtype=dtype,
                         dims=list(dims))

    def op(self, name, operands, dtype, dims, m2m=None, quant=None, **attrs) -> int:
        return self._add(op=name, operands=list(operands), dtype=dtype, dims=list(dims),
                         m2m=m2m, quant=quant, **attrs)

    def unary(self, name, x, dtype, dims, m2m=None) -> int:
        return self.op(name, [x], dtype, dims, m2m)

    def binary(self, name, a, b, dtype, dims, m2m=None) -> int:
        return self.op(name, [a, b], dtype, dims, m2m)

    def transpose(self, x, perm, dtype, dims, m2m=None) -> int:
        return self.op("transpose", [x], dtype, dims, m2m, permutation=list(perm))

    def broadcast_in_dim(self, x, bdims, dtype, dims, m2m=None) -> int:
        return self.op("broadcast_in_dim", [x], dtype, dims, m2m,
                       broadcast_dimensions=list(bdims))

    def reshape(self, x, dtype, dims, m2m=None) -> int:
        return self.op("reshape", [x], dtype, dims, m2m)

    def reduce(self, x, dims_to_reduce, reducer, init, dtype, dims, m2m=None) -> int:
        return self.op("reduce", [x], dtype, dims, m2m, dimensions=list(dims_to_reduce),
                       reducer=reducer, init=float(init))

    def reverse(self, x, dims_to_reverse, dtype, dims, m2m=None) -> int:
        return self.op("reverse", [x], dtype, dims, m2m, dimensions=list(dims_to_reverse))

    def iota(self, iota_dimension, dtype, dims, m2m=None) -> int:
        return self.op("iota", [], dtype, dims, m2m, iota_dimension=int(iota_dimension))

    def pad(self, x, padding_value, low, high, interior, dtype, dims, m2m=None) -> int:
        return self.op("pad", [x, padding_value], dtype, dims, m2m, edge_padding_low=list(low),
                       edge_padding_high=list(high), interior_padding=list(interior))

    def concatenate(self, inputs, dimension, dtype, dims, m2m=None) -> int:
        return self.op("concatenate", list(inputs), dtype, dims, m2m, dimension=int(dimension))

    def slice(self, x, start, limit, strides, dtype, dims, m2m=None) -> int:
        return self.op("slice", [x], dtype, dims, m2m, start_indices=list(start),
                       limit_indices=list(limit), strides=list(strides))

    def dynamic_slice(self, x, starts, sizes, dtype, m2m=None) -> int:
        """`starts`: one rank-0 integer node per dim of x."""
        return self.op("dynamic_slice", [x] + list(starts), dtype, list(sizes), m2m,
                       slice_sizes=list(sizes))

    def argmax(self, x, rdim, dims, index_init=-1, init=float("-inf"), m2m=None) -> int:
        """Variadic max/argmax reduce over `rdim` of x with an iota index
        operand; the result is the s32 index."""
        k = self.iota(rdim, "s32", dims)
        out = [d for i, d in enumerate(dims) if i != rdim]
        return self.op("reduce", [x, k], "s32", out, m2m, dimensions=[rdim], reducer="argmax",
                       init=float(init), index_init=int(index_init))

    def convert(self, x, dtype, dims, m2m=None) -> int:
        return self.op("convert", [x], dtype, dims, m2m)

    def set_root_layout(self, m2m) -> None:
        self.nodes[-1]["m2m"] = list(m2m)


def quant_type(storage, scales, zero_points, qdim=None, storage_min=None,
               storage_max=None) -> dict:
    q = {"storage": storage, "expressed": "f32", "qdim": qdim,
         "scales": np.asarray(scales, dtype=np.float32),
         "zero_points": np.asarray(zero_points, dtype=np.int64)}
    if storage_min is not None:
        q["storage_min"] = int(storage_min)
    if storage_max is not None:
        q["storage_max"] = int(storage_max)
    return q


def nbytes_of(dtype: str) -> int:
    return {"f32": 4, "bf16": 2, "f16": 2, "s8": 1, "u8": 1, "s32": 4}[dtype]


def numel(dims) -> int:
    n = 1
    for d in dims:
        n *= int(d)
    return n


# --------------------------------------------------------------------------
# The five workloads.  Each builder takes its shape so the tests can run the
# same fusion at small, ragged sizes; the defaults are the full sizes.
# A workload is (spec, params, meta) with params as flat physical buffers.
# --------------------------------------------------------------------------
def loop_log_transpose_add(n0=64, n1=None, seed=1):
    """p = param; l = log(p); t = transpose(l, {1,0}); out = add(l, t).

    Square f32[n,n], row-major; p ~ U(0.1, 10).  `l` is read through two index
    maps (identity and transposed)."""
    n1 = n0 if n1 is None else n1
    assert n0 == n1, "add(l, transpose(l)) needs a square operand"
    g = rng(seed)
    s = Spec()
    p = s.parameter(0, "f32", [n0, n1], [1, 0])
    l = s.unary("log", p, "f32", [n0, n1])
    t = s.transpose(l, [1, 0], "f32", [n1, n0])
    s.binary("add", l, t, "f32", [n0, n1], m2m=[1, 0])
    x = uniform_f32(g, n0 * n1, 0.1, 10.0)
    return s, [x], {"name": "loop_log_transpose_add", "elements": n0 * n1,
                    "bytes": 2 * 4 * n0 * n1}


def transpose_exp_f32(n0=4096, n1=4096, seed=2):
    """out = transpose(exp(x), {1,0}); x f32[n0,n1] ~ N(0,1), row-major in and out."""
    g = rng(seed)
    s = Spec()
    x = s.parameter(0, "f32", [n0, n1], [1, 0])
    e = s.unary("exponential", x, "f32", [n0, n1])
    s.transpose(e, [1, 0], "f32", [n1, n0], m2m=[1, 0])
    return s, [normal_f32(g, n0 * n1)], {"name": "transpose_exp_f32",
                                         "elements": n0 * n1, "bytes": 8 * n0 * n1}


def transpose_bf16_021(b=64, m=512, n=1024, seed=3):
    """out = transpose(x, {0,2,1}); x bf16[b,m,n] ~ N(0,1), row-major in and out."""
    g = rng(seed)
    s = Spec()
    x = s.parameter(0, "bf16", [b, m, n], [2, 1, 0])
    s.transpose(x, [0, 2, 1], "bf16", [b, n, m], m2m=[2, 1, 0])
    return s, [normal_bf16(g, b * m * n)], {"name": "transpose_bf16_021",
                                             "elements": b * m * n, "bytes": 4 * b * m * n}


def row_reduce_exp_add_bf16(d0=8, d2=1280, d3=16384, m2m=(3, 2, 1, 0), seed=4):
    """y = add(exp(x), broadcast(b, dims={3})) in bf16; out f32[d0,1,d2] =
    reduce-sum over dim 3 of convert(y, f32), init 0."""
    g = rng(seed)
    s = Spec()
    dims = [d0, 1, d2, d3]
    x = s.parameter(0, "bf16", dims, list(m2m))
    bb = s.parameter(1, "bf16", [d3], [0])
    e = s.unary("exponential", x, "bf16", dims)
    bc = s.broadcast_in_dim(bb, [3], "bf16", dims)
    y = s.binary("add", e, bc, "bf16", dims)
    c = s.convert(y, "f32", dims)
    s.reduce(c, [3], "add", 0.0, "f32", [d0, 1, d2], m2m=[2, 1, 0])
    xs = normal_bf16(g, d0 * d2 * d3)
    bs = normal_bf16(g, d3)
    n = d0 * d2 * d3
    return s, [xs, bs], {"name": "row_reduce_exp_add_bf16", "elements": n,
                         "bytes": 2 * n + 2 * d3 + 4 * d0 * d2}


def column_reduce_max_f32(r=16384, c=4096, m2m=(1, 0), seed=5):
    """out f32[c] = reduce-max over dim 0 of x f32[r,c], init -inf.
    x ~ U(-100, 100).  With m2m (0,1) the buffer holds the column-major
    storage; the test derives it from the row-major draw."""
    g = rng(seed)
    s = Spec()
    x = s.parameter(0, "f32", [r, c], list(m2m))
    s.reduce(x, [0], "max", float("-inf"), "f32", [c], m2m=[0])
    return s, [uniform_f32(g, r * c, -100.0, 100.0)], {
        "name": "column_reduce_max_f32", "elements": r * c, "bytes": 4 * r * c + 4 * c}


def quant_dequant_bias_requant(r=4096, c=4096, seed=6, out_scale=0.02, out_zp=0):
    """Per-axis dequantize (qdim=1) of q i8[r,c], add f32 bias[c] broadcast on
    dim 1, requantize per-tensor i8 (scale 0.02, zero point 0)."""
    g = rng(seed)
    q = integers(g, r * c, -128, 127, np.int8)
    scales = uniform_f32(g, c, 0.001, 0.05)
    zps = integers(g, c, -20, 20, np.int64)
    bias = normal_f32(g, c, 0.1)
    s = Spec()
    qin = quant_type("s8", scales, zps, qdim=1)
    qout = quant_type("s8", [out_scale], [out_zp])
    p = s.parameter(0, "s8", [r, c], [1, 0], quant=qin)
    bb = s.parameter(1, "f32", [c], [0])
    d = s.op("uniform_dequantize", [p], "f32", [r, c])
    bc = s.broadcast_in_dim(bb, [1], "f32", [r, c])
    y = s.binary("add", d, bc, "f32", [r, c])
    s.op("uniform_quantize", [y], "s8", [r, c], m2m=[1, 0], quant=qout)
    return s, [q, bias], {"name": "quant_dequant_bias_requant", "elements": r * c,
                          "bytes": 2 * r * c + 4 * c + 4 * c + 4 * c}


def quant_dequant_bias_requant_s4(r=4096, c=4096, seed=13, out_scale=0.05, out_zp=0):
    """The per-axis requantize of quant_dequant_bias_requant with si4 storage
    in and out: q si4[r,c] is drawn as random bytes (two random 4-bit values
    each), scales ~ U(0.001, 0.05), zero points U{-3..3}, bias f32[c] ~
    N(0, 0.1) broadcast on dim 1, requantized per-tensor si4 (scale 0.05,
    zero point 0)."""
    g = rng(seed)
    q = integers(g, (r * c + 1) // 2, 0, 255, np.uint8)
    scales = uniform_f32(g, c, 0.001, 0.05)
    zps = integers(g, c, -3, 3, np.int64)
    bias = normal_f32(g, c, 0.1)
    s = Spec()
    qin = quant_type("s4", scales, zps, qdim=1)
    qout = quant_type("s4", [out_scale], [out_zp])
    p = s.parameter(0, "s4", [r, c], [1, 0], quant=qin)
    bb = s.parameter(1, "f32", [c], [0])
    d = s.op("uniform_dequantize", [p], "f32", [r, c])
    bc = s.broadcast_in_dim(bb, [1], "f32", [r, c])
    y = s.binary("add", d, bc, "f32", [r, c])
    s.op("uniform_quantize", [y], "s4", [r, c], m2m=[1, 0], quant=qout)
    return s, [q, bias], {"name": "quant_dequant_bias_requant_s4", "elements": r * c,
                          "bytes": r * c + 9 * c}


def transpose3d_exp_abs(d0=20, d1=160, d2=170, seed=8):
    """out = abs(transpose(exp(x), {2,1,0})), x f32[d0,d1,d2] ~ N(0,1): the
    transpose emitter's example on XLA:GPU Emitters ("Transpose emitter"),
    with an elementwise op after the transpose."""
    g = rng(seed)
    s = Spec()
    x = s.parameter(0, "f32", [d0, d1, d2])
    e = s.unary("exponential", x, "f32", [d0, d1, d2])
    t = s.transpose(e, [2, 1, 0], "f32", [d2, d1, d0])
    s.unary("abs", t, "f32", [d2, d1, d0])
    n = d0 * d1 * d2
    return s, [normal_f32(g, n)], {"name": "transpose3d_exp_abs", "elements": n, "bytes": 8 * n}


def pad_reverse_concat_f32(n0=4096, n1=4096, m0=2048, seed=9):
    """out = concatenate([pad(x, low [1,0], high [1,0]), reverse(y, {0})], 0)
    with x f32[n0,n1], y f32[m0,n1] ~ N(0,1): index transforms along the major
    dim (StableHLO Specification: pad, reverse, concatenate)."""
    g = rng(seed)
    s = Spec()
    x = s.parameter(0, "f32", [n0, n1])
    y = s.parameter(1, "f32", [m0, n1])
    z = s.constant(0.0, "f32", [])
    p = s.pad(x, z, [1, 0], [1, 0], [0, 0], "f32", [n0 + 2, n1])
    r = s.reverse(y, [0], "f32", [m0, n1])
    s.concatenate([p, r], 0, "f32", [n0 + 2 + m0, n1])
    return s, [normal_f32(g, n0 * n1), normal_f32(g, m0 * n1)], {
        "name": "pad_reverse_concat_f32", "elements": (n0 + 2 + m0) * n1,
        "bytes": 4 * (n0 * n1 + m0 * n1 + (n0 + 2 + m0) * n1)}


def pad_reverse_concat_minor_f32(n0=4096, n1=2040, m1=2048, seed=14):
    """The same transforms along the minor dim: out = concatenate([pad(x,
    low [0,4], high [0,4]), reverse(y, {1})], 1) with x f32[n0,n1], y
    f32[n0,m1] ~ N(0,1), out f32[n0, n1 + 8 + m1] (every output element's
    index map moves with the lane)."""
    g = rng(seed)
    s = Spec()
    x = s.parameter(0, "f32", [n0, n1])
    y = s.parameter(1, "f32", [n0, m1])
    z = s.constant(0.0, "f32", [])
    p = s.pad(x, z, [0, 4], [0, 4], [0, 0], "f32", [n0, n1 + 8])
    r = s.reverse(y, [1], "f32", [n0, m1])
    s.concatenate([p, r], 1, "f32", [n0, n1 + 8 + m1])
    return s, [normal_f32(g, n0 * n1), normal_f32(g, n0 * m1)], {
        "name": "pad_reverse_concat_minor_f32", "elements": n0 * (n1 + 8 + m1),
        "bytes": 4 * (n0 * n1 + n0 * m1 + n0 * (n1 + 8 + m1))}


def quantized_add_i8(r=4096, c=4096, seed=10):
    """out = add(a, b) on per-tensor quantized i8[r,c] tensors (scales 0.05 and
    0.02, zero points 3 and -7), quantized to scale 0.04, zero point 1."""
    g = rng(seed)
    s = Spec()
    a = s.parameter(0, "s8", [r, c], quant=quant_type("s8", [0.05], [3]))
    b = s.parameter(1, "s8", [r, c], quant=quant_type("s8", [0.02], [-7]))
    s.op("add", [a, b], "s8", [r, c], quant=quant_type("s8", [0.04], [1]))
    return s, [integers(g, r * c, -128, 127, np.int8), integers(g, r * c, -128, 127, np.int8)], {
        "name": "quantized_add_i8", "elements": r * c, "bytes": 3 * r * c}


def row_mean_f32(r=16384, c=4096, seed=11):
    """out f32[r] = reduce-sum over dim 1 of x f32[r,c] ~ N(0,1), divided by c:
    a reduce with an elementwise epilogue."""
    g = rng(seed)
    s = Spec()
    x = s.parameter(0, "f32", [r, c])
    m = s.reduce(x, [1], "add", 0.0, "f32", [r])
    n = s.constant(float(c), "f32", [r])
    s.binary("divide", m, n, "f32", [r])
    return s, [normal_f32(g, r * c)], {"name": "row_mean_f32", "elements": r * c, "bytes": 4 * r * c + 4 * r}


def argmax_rows_bf16(r=8192, c=8192, seed=12):
    """out s32[r] = argmax over dim 1 of x bf16[r,c] ~ N(0,1) (the variadic
    max/argmax reduce with an iota index operand)."""
    g = rng(seed)
    s = Spec()
    x = s.parameter(0, "bf16", [r, c])
    s.argmax(x, 1, [r, c])
    return s, [normal_bf16(g, r * c)], {"name": "argmax_rows_bf16", "elements": r * c, "bytes": 2 * r * c + 4 * r}


def gelu_bf16(d0=6, d1=512, d2=4096, seed=7):
    """The GELU loop fusion in bf16 (tanh form), every op rounding to bf16."""
    g = rng(seed)
    s = Spec()
    dims = [d0, d1, d2]
    x = s.parameter(0, "bf16", dims, [2, 1, 0])
    c05 = s.constant(0.5, "bf16", dims)
    c1 = s.constant(1.0, "bf16", dims)
    c2 = s.constant(0.79785, "bf16", dims)
    c3 = s.constant(0.044708, "bf16", dims)
    sq = s.binary("multiply", x, x, "bf16", dims)
    cube = s.binary("multiply", sq, x, "bf16", dims)
    m3 = s.binary("multiply", cube, c3, "bf16", dims)
    a1 = s.binary("add", x, m3, "bf16", dims)
    m2 = s.binary("multiply", a1, c2, "bf16", dims)
    th = s.unary("tanh", m2, "bf16", dims)
    a0 = s.binary("add", th, c1, "bf16", dims)
    m1 = s.binary("multiply", a0, c05, "bf16", dims)
    s.binary("multiply", x, m1, "bf16", dims, m2m=[2, 1, 0])
    n = d0 * d1 * d2
    return s, [normal_bf16(g, n)], {"name": "gelu_bf16", "elements": n, "bytes": 4 * n}
