"""Seeded random fusions, compared with the oracle.

Each case is a random graph over a rank 1-3 output space with random
minor_to_major layouts: parameters read directly, transposed, broadcast or
reversed, chains of elementwise ops that round identically on both sides
(add, subtract, multiply, maximum, minimum, negate, abs, converts between
f32 and bf16 or f16), and sometimes a reduce (add over integer-valued f32, or max/min)
followed by an elementwise epilogue.  Inputs are small integers, so every
result, sums included, is exact: the comparison is bit-exact.  Fusions the
library does not implement (a reduce whose dims are neither physically minor
nor physically major) are counted and skipped.

Five bit-exact series: any shape; tile-sized shapes biased toward the
transpose and column-reduce heroes; pad, concatenate and quantized storage;
big shapes (dims up to 16384, up to 4M elements) for the whole-workgroup
row paths, many column segments and the wide transpose tiles; and rank 4-6
spaces with size-1 dims, for layout normalisation (the pad, concatenate and
quantized series as well).  The first two also run with NaN, +-inf and +-0
in the inputs (NaN positions compare, other elements bitwise).  A sixth
series puts one exp, log or tanh among exactly rounding ops and compares
within the bound the result allows (half of it with special values in the
inputs).  A seventh series is 8-bit arithmetic for the pipelined loop:
per-tensor and per-axis dequantize of s8/u8 storage with arbitrary scales,
a bias broadcast along random dims, and a per-tensor or per-axis quantize
to s8/u8; both sides round each op once in f32 and divide by the scale, so
it is bit-exact too.

The CPU test plans and compiles every case for gfx950 (and runs the oracle on
all but the big ones); the GPU tests run them.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from harness import assert_bitexact, run_gpu

N_CASES = 192       # seeds 1000.. : any shape
N_HERO = 96         # seeds 2000.. : tile-sized shapes, a transposed read, major-dim reduces
N_WIDE = 96         # seeds 3000.. : pad, concatenate, quantized and 4-bit storage
N_BIG = 24          # seeds 4000.. : dims up to 16384, 0.2M-4M elements
N_RANK = 24         # seeds 6000.. : rank 4-6 with size-1 dims
N_WRANK = 24        # seeds 7000.. : the pad/concatenate/quantized series at rank 4-5
N_SPECIAL = 24      # seeds 8000.. : the first two series with NaN, +-inf and +-0 in the inputs
N_TRANS = 48        # seeds 5000.. : one exp, log or tanh, compared within its bound
N_Q8 = 48           # seeds 9000.. : 8-bit dequantize / bias / quantize loops
BATCH = 24


def _layout(g, rank):
    return [int(d) for d in g.permutation(rank)] if g.random() < 0.5 else None


def _values(g, dtype, n):
    v = W.integers(g, n, -8, 8, np.int64).astype(np.float32)
    if dtype == "f16":
        return v.astype(np.float16).view(np.uint16)
    return (v.view(np.uint32) >> 16).astype(np.uint16) if dtype == "bf16" else v


def _half(seed, dt):
    """A 16-bit float type becomes f16 for some seeds (drawn from a stream of
    its own, so that every other draw of the case stays as it was)."""
    return "f16" if dt == "bf16" and W.rng(seed + 7_000_000).random() < 0.4 else dt


def random_case(seed, hero_bias=False, big=False, high_rank=False):
    """(spec, params) of one random fusion.  With hero_bias the shapes are
    tile-sized, the first parameter is read transposed and reductions favour
    the physically major dims, so that the transpose and column-reduce heroes
    come up often.  With big (and hero_bias) the dims reach 16384 and the
    arrays 4M elements: whole-workgroup rows, many column segments and the
    wide transpose tiles."""
    g = W.rng(seed)
    rank = int(g.integers(2, 4)) if hero_bias else int(g.integers(1, 4))
    if high_rank:
        rank = int(g.integers(4, 7))
    if high_rank:
        sizes, cap = [1, 1, 2, 3, 4, 5, 8, 16, 17], 100_000
    elif big:
        sizes, cap = [2, 7, 64, 130, 1024, 2048, 4100, 8192, 16384], 4_000_000
    elif hero_bias:
        sizes, cap = [33, 64, 96, 130, 257], 100_000
    else:
        sizes, cap = [1, 2, 3, 5, 8, 17, 33, 64, 96, 130], 100_000
    while True:
        dims = [int(g.choice(sizes)) for _ in range(rank)]
        if math.prod(dims) <= cap and (not big or math.prod(dims) >= 200_000):
            break
    dt = _half(seed, "f32" if g.random() < 0.6 else "bf16")
    with_reduce = g.random() < 0.4
    s = W.Spec()
    params, vals = [], []
    for p in range(int(g.integers(1, 4))):
        kind = str(g.choice(["plain", "transpose", "broadcast", "reverse"]))
        if hero_bias and p == 0:
            kind = "transpose"
        if kind == "transpose" and rank < 2:
            kind = "plain"
        if kind == "plain":
            x = s.parameter(p, dt, dims, _layout(g, rank))
            pdims = dims
        elif kind == "transpose":
            perm = [int(d) for d in g.permutation(rank)]
            pdims = [0] * rank
            for d in range(rank):
                pdims[perm[d]] = dims[d]
            x = s.transpose(s.parameter(p, dt, pdims, _layout(g, rank)), perm, dt, dims)
        elif kind == "broadcast":
            k = int(g.integers(0, rank + 1))
            bd = sorted(int(d) for d in g.choice(rank, k, replace=False))
            pdims = [dims[d] if g.random() < 0.8 else 1 for d in bd]
            x = s.broadcast_in_dim(s.parameter(p, dt, pdims), bd, dt, dims)
        else:
            rd = sorted(int(d) for d in g.choice(rank, int(g.integers(1, rank + 1)), replace=False))
            pdims = dims
            x = s.reverse(s.parameter(p, dt, dims, _layout(g, rank)), rd, dt, dims)
        vals.append(x)
        params.append(_values(g, dt, math.prod(pdims)))
    binary = ["add", "subtract", "maximum", "minimum"] + ([] if with_reduce else ["multiply"])
    for _ in range(int(g.integers(1, 6))):
        if g.random() < 0.7:
            a, b = (int(i) for i in g.choice(len(vals), 2))
            vals.append(s.binary(str(g.choice(binary)), vals[a], vals[b], dt, dims))
        else:
            vals.append(s.unary(str(g.choice(["negate", "abs"])), vals[int(g.integers(len(vals)))], dt, dims))
    r = vals[-1]
    for v in vals[:-1]:  # every value reaches the root
        r = s.binary("add", r, v, dt, dims)
    cur = dt
    if g.random() < 0.3:
        cur = _half(seed + 1, "bf16") if dt == "f32" else "f32"
        r = s.convert(r, cur, dims)
    out_dims = dims
    if with_reduce:
        if hero_bias and g.random() < 0.6:  # the leading dims of the default layout
            red = list(range(int(g.integers(1, rank))))
            s.nodes[-1]["m2m"] = None
        else:
            red = sorted(int(d) for d in g.choice(rank, int(g.integers(1, rank + 1)), replace=False))
        out_dims = [dims[d] for d in range(rank) if d not in red]
        reducer = str(g.choice(["add", "max", "min"]))
        if reducer == "add" and cur != "f32":
            cur = "f32"
            r = s.convert(r, cur, dims)
        init = {"add": 0.0, "max": -np.inf, "min": np.inf}[reducer]
        r = s.reduce(r, red, reducer, init, cur, out_dims)
        if g.random() < 0.5:
            r = s.unary(str(g.choice(["negate", "abs"])), r, cur, out_dims)
    s.nodes[-1]["m2m"] = _layout(g, len(out_dims))
    return s, params


_STORAGE = {"s8": (-128, 127), "u8": (0, 255), "s4": (-8, 7), "u4": (0, 15)}


def _storage_values(g, dt, n):
    """Random storage values of n elements, packed two per byte for 4-bit."""
    if dt in ("s4", "u4"):
        return W.integers(g, (n + 1) // 2, 0, 255, np.uint8)
    lo, hi = _STORAGE[dt]
    return W.integers(g, n, lo, hi, np.int8 if dt == "s8" else np.uint8)


def random_wide_case(seed, high_rank=False):
    """(spec, params): f32 values built by pad, concatenate and per-tensor or
    per-axis dequantize (power-of-two scales, so every value is exact, and
    so is every sum whose terms stay small against their lowest bits),
    combined by exact elementwise ops, ending in a quantize to an 8- or 4-bit
    type, a reduce, or neither."""
    g = W.rng(seed)
    rank = int(g.integers(4, 6)) if high_rank else int(g.integers(1, 4))
    sizes = [1, 2, 3, 4, 6, 9, 16] if high_rank else [2, 3, 6, 9, 16, 31, 64, 100]
    while True:
        dims = [int(g.choice(sizes)) for _ in range(rank)]
        if math.prod(dims) <= 100_000:
            break
    s = W.Spec()
    params, vals = [], []
    for p in range(int(g.integers(1, 4))):
        kind = str(g.choice(["pad", "concatenate", "dequantize"]))
        if kind == "pad":
            inter = [int(g.integers(0, 2)) for _ in range(rank)]
            pd, low, high = [], [], []
            for d in range(rank):
                n = int(g.integers(1, (dims[d] - 1) // (inter[d] + 1) + 2))
                rem = dims[d] - ((n - 1) * (inter[d] + 1) + 1)
                lo = int(g.integers(0, rem + 1))
                pd.append(n), low.append(lo), high.append(rem - lo)
            x = s.parameter(len(params), "f32", pd)
            params.append(_values(g, "f32", math.prod(pd)))
            v = s.constant(float(g.integers(-4, 5)), "f32", [])
            vals.append(s.pad(x, v, low, high, inter, "f32", dims))
        elif kind == "concatenate" and max(dims) >= 2:
            d = int(np.argmax(dims))
            a = int(g.integers(1, dims[d]))
            parts = []
            for ext in (a, dims[d] - a):
                pdims = list(dims)
                pdims[d] = ext
                parts.append(s.parameter(len(params), "f32", pdims, _layout(g, rank)))
                params.append(_values(g, "f32", math.prod(pdims)))
            vals.append(s.concatenate(parts, d, "f32", dims))
        else:
            st = str(g.choice(list(_STORAGE)))
            lo, hi = _STORAGE[st]
            if g.random() < 0.5:
                q = W.quant_type(st, [float(2.0 ** -int(g.integers(0, 4)))], [int(g.integers(lo, hi + 1))])
            else:
                qd = int(g.integers(rank))
                n = dims[qd]
                q = W.quant_type(st, [float(2.0 ** -int(k)) for k in g.integers(0, 4, n)],
                                 [int(z) for z in g.integers(lo, hi + 1, n)], qdim=qd)
            x = s.parameter(len(params), st, dims, quant=q)
            params.append(_storage_values(g, st, math.prod(dims)))
            vals.append(s.op("uniform_dequantize", [x], "f32", dims))
    for _ in range(int(g.integers(0, 4))):
        a, b = (int(i) for i in g.choice(len(vals), 2))
        vals.append(s.binary(str(g.choice(["add", "subtract", "maximum", "minimum"])), vals[a], vals[b], "f32", dims))
    r = vals[-1]
    for v in vals[:-1]:
        r = s.binary("add", r, v, "f32", dims)
    end = str(g.choice(["quantize", "reduce", "none"]))
    out_dims = dims
    if end == "quantize":
        st = str(g.choice(list(_STORAGE)))
        lo, hi = _STORAGE[st]
        q = W.quant_type(st, [float(g.choice([0.3, 0.5, 1.7, 2.0]))], [int(g.integers(lo, hi + 1))])
        s.op("uniform_quantize", [r], st, dims, quant=q)
    elif end == "reduce":
        red = sorted(int(d) for d in g.choice(rank, int(g.integers(1, rank + 1)), replace=False))
        out_dims = [dims[d] for d in range(rank) if d not in red]
        reducer = str(g.choice(["add", "max", "min"]))
        init = {"add": 0.0, "max": -np.inf, "min": np.inf}[reducer]
        s.reduce(r, red, reducer, init, "f32", out_dims)
    s.nodes[-1]["m2m"] = _layout(g, len(out_dims))
    return s, params


_ZP8 = {"s8": 0, "u8": 128}  # centre of the zero points drawn


def random_q8_case(seed):
    """(spec, params): one to three s8/u8 parameters dequantized per tensor or
    per axis (scales in [0.001, 0.05], zero points near the storage centre),
    combined by add, subtract, maximum or minimum with an optional f32 bias
    broadcast along a random subset of dims, and quantized per tensor or per
    axis to s8/u8, in a random layout shared by the inputs (and usually the
    output): the fusions that take the software-pipelined loop."""
    g = W.rng(seed)
    rank = int(g.integers(1, 5))
    while True:
        if g.random() < 0.3:
            dims = [int(g.integers(1, 6)) for _ in range(rank - 1)] + [int(g.choice([16, 32, 48, 64, 4096, 8192]))]
            g.shuffle(dims)
        else:
            dims = [int(g.choice([1, 3, 7, 16, 32, 48, 64, 112, 257, 1000, 1024, 4096])) for _ in range(rank)]
        if 1 <= math.prod(dims) <= 3_000_000:
            break
    layout = _layout(g, rank)
    s = W.Spec()
    params, vals = [], []

    def qtype(st, smin, smax, spread):
        if g.random() < 0.45:
            return W.quant_type(st, [float(g.uniform(smin, smax))], [_ZP8[st] + int(g.integers(-spread, spread + 1))])
        qd = int(g.integers(rank))
        return W.quant_type(st, [float(x) for x in g.uniform(smin, smax, dims[qd])],
                            [_ZP8[st] + int(z) for z in g.integers(-spread, spread + 1, dims[qd])], qdim=qd)
    for _ in range(int(g.integers(1, 4))):
        st = str(g.choice(["s8", "u8"]))
        x = s.parameter(len(params), st, dims, layout, quant=qtype(st, 0.001, 0.05, 20))
        params.append(_storage_values(g, st, math.prod(dims)))
        vals.append(s.op("uniform_dequantize", [x], "f32", dims))
    if g.random() < 0.6:
        bd = sorted(int(d) for d in g.choice(rank, int(g.integers(0, rank + 1)), replace=False))
        bdims = [dims[d] for d in bd]
        b = s.parameter(len(params), "f32", bdims)
        params.append(W.normal_f32(g, math.prod(bdims), 0.1))
        vals.append(s.broadcast_in_dim(b, bd, "f32", dims))
    r = vals[0]
    for v in vals[1:]:
        r = s.binary(str(g.choice(["add", "subtract", "maximum", "minimum"])), r, v, "f32", dims)
    st = str(g.choice(["s8", "u8"]))
    s.op("uniform_quantize", [r], st, dims, m2m=layout if g.random() < 0.7 else None,
         quant=qtype(st, 0.005, 0.05, 10))
    return s, params


def random_trans_case(seed, specials=False):
    """(spec, params, check): one exp, log or tanh (f32 or bf16) inside a
    random fusion, between exactly rounding ops.  Its operand is exact
    (a parameter read plainly, transposed or reversed, maybe added to a
    second one; abs(.) + 1 for log); after it come an optional negate or abs,
    an optional convert, and an optional reduce.  check(got, spec, params)
    compares with the bound the result allows: 2 f32 ulp (the transcendental's
    own), 1 bf16 ulp once a bf16 rounding follows it, and for a sum the
    summation bound 2^-20 * sum|terms|."""
    g = W.rng(seed)
    rank = int(g.integers(1, 4))
    while True:
        dims = [int(g.choice([1, 2, 3, 5, 8, 17, 33, 64, 96, 130, 257])) for _ in range(rank)]
        if math.prod(dims) <= 100_000:
            break
    dt = "f32" if g.random() < 0.6 else "bf16"
    s = W.Spec()
    params, vals = [], []
    for p in range(int(g.integers(1, 3))):
        kind = str(g.choice(["plain", "transpose", "reverse"]))
        if kind == "transpose" and rank > 1:
            perm = [int(d) for d in g.permutation(rank)]
            pdims = [0] * rank
            for d in range(rank):
                pdims[perm[d]] = dims[d]
            x = s.transpose(s.parameter(p, dt, pdims, _layout(g, rank)), perm, dt, dims)
        elif kind == "reverse":
            rd = sorted(int(d) for d in g.choice(rank, int(g.integers(1, rank + 1)), replace=False))
            x = s.reverse(s.parameter(p, dt, dims, _layout(g, rank)), rd, dt, dims)
        else:
            x = s.parameter(p, dt, dims, _layout(g, rank))
        vals.append(x)
        params.append(_values(g, dt, math.prod(dims)))
    x = vals[0] if len(vals) == 1 else s.binary(str(g.choice(["add", "maximum"])), vals[0], vals[1], dt, dims)
    op = str(g.choice(["exponential", "log", "tanh"]))
    if op == "log":
        x = s.binary("add", s.unary("abs", x, dt, dims), s.constant(1.0, dt, dims), dt, dims)
    y = s.unary(op, x, dt, dims)
    if g.random() < 0.4:
        y = s.unary(str(g.choice(["negate", "abs"])), y, dt, dims)
    cur = dt
    if g.random() < 0.3:
        cur = "bf16" if dt == "f32" else "f32"
        y = s.convert(y, cur, dims)
    tol_dt = "bf16" if "bf16" in (dt, cur) else "f32"
    red = None
    out_dims = dims
    if g.random() < 0.4:
        red = sorted(int(d) for d in g.choice(rank, int(g.integers(1, rank + 1)), replace=False))
        reducer = str(g.choice(["add", "max", "min"]))
        if reducer == "add" and cur != "f32":
            cur = "f32"
            y = s.convert(y, cur, dims)
        out_dims = [dims[d] for d in range(rank) if d not in red]
        init = {"add": 0.0, "max": -np.inf, "min": np.inf}[reducer]
        s.reduce(y, red, reducer, init, cur, out_dims)
    s.nodes[-1]["m2m"] = _layout(g, len(out_dims))
    is_sum = red is not None and s.nodes[-1]["reducer"] == "add"
    if specials and not is_sum:  # a sum's bound needs finite terms
        params = _with_specials(seed, s, params)

    def check(got):
        import itertools
        if not is_sum:
            from harness import assert_ulp
            assert_ulp(got, oracle.evaluate(s.nodes, params), cur, 1 if tol_dt == "bf16" else 2)
            return
        rn = s.nodes[-1]
        pts = (np.array(list(itertools.product(*[range(d) for d in out_dims])), dtype=np.int64)
               if out_dims else np.zeros((1, 0), np.int64))
        vals_, aux = oracle.evaluate_points(s.nodes, params, pts)
        lin = oracle.linear_indices(out_dims, rn["m2m"] or oracle.default_m2m(len(out_dims)), pts) if out_dims else np.zeros(1, np.int64)
        gv = got[lin].astype(np.float64)
        bound = 2.0 ** -20 * aux[:, 0] + (2.0 ** -8 if tol_dt == "bf16" else 0.0) * aux[:, 0]
        assert np.all(np.abs(gv - aux[:, 1]) <= bound), float(np.max(np.abs(gv - aux[:, 1]) - bound))
    return s, params, check


_SPECIALS = {"f32": [np.float32(v).view(np.uint32) for v in (np.nan, np.inf, -np.inf, -0.0, 0.0)],
             "bf16": [0x7FC0, 0x7F80, 0xFF80, 0x8000, 0x0000],
             "f16": [0x7E00, 0x7C00, 0xFC00, 0x8000, 0x0000]}


def _with_specials(seed, s, params):
    """About 2% of every float parameter's elements set to NaN, +-inf or +-0
    (from a stream of their own).  IEEE arithmetic propagates them alike in
    any order (NaN positions compare, not payloads)."""
    out = []
    for k, (nd, x) in enumerate(zip([nd for nd in s.nodes if nd["op"] == "parameter"], params)):
        dt = nd["dtype"]
        if dt not in _SPECIALS or x.size == 0:
            out.append(x)
            continue
        g = W.rng(seed + 8_000_000 + k)
        x = x.copy()
        idx = g.choice(x.size, max(1, x.size // 50), replace=False)
        bits = x.view(np.uint32 if dt == "f32" else np.uint16)
        bits[idx] = np.asarray(_SPECIALS[dt], dtype=bits.dtype)[g.integers(0, 5, idx.size)]
        out.append(x)
    return out


def _make(seed, series):
    if series == "special":
        s, params = random_case(seed, seed % 2 == 1)
        return s, _with_specials(seed, s, params)
    if series in ("wide", "wrank"):
        return random_wide_case(seed, series == "wrank")
    if series == "q8":
        return random_q8_case(seed)
    return random_case(seed, series in ("hero", "big"), series == "big", series == "rank")


def _cases():
    """(seed, series) of every case."""
    return ([(1000 + k, "any") for k in range(N_CASES)] + [(2000 + k, "hero") for k in range(N_HERO)]
            + [(3000 + k, "wide") for k in range(N_WIDE)] + [(4000 + k, "big") for k in range(N_BIG)]
            + [(6000 + k, "rank") for k in range(N_RANK)] + [(7000 + k, "wrank") for k in range(N_WRANK)]
            + [(8000 + k, "special") for k in range(N_SPECIAL)] + [(9000 + k, "q8") for k in range(N_Q8)])


def test_random_fusions_plan_and_compile():
    """Every case plans and compiles (in parallel: create is thread-safe and
    releases the GIL), unsupported ones fail with HF_ERR_UNSUPPORTED only, and
    all four heroes come up."""
    import collections
    import os
    from concurrent.futures import ThreadPoolExecutor
    import compiler_hlo_amd as H
    cases = [(seed, series) + _make(seed, series) for seed, series in _cases()]

    def create(case):
        seed, series, s, params = case
        try:
            return H.Fusion(s.nodes, mode="compile").plan()["hero"]
        except H.FusionError as e:
            assert e.status == "HF_ERR_UNSUPPORTED", (seed, str(e))
            return None

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
        heroes_of = list(pool.map(create, cases))
    heroes = collections.Counter(h for h in heroes_of if h)
    for (seed, series, s, params), h in zip(cases, heroes_of):
        if h and series != "big":  # the big cases' oracle runs with their GPU test
            oracle.evaluate(s.nodes, params)
    ran = sum(1 for h in heroes_of if h)
    total = N_CASES + N_HERO + N_WIDE + N_BIG + N_RANK + N_WRANK + N_SPECIAL + N_Q8
    assert ran >= total * 2 // 3, (ran, total - ran)
    assert all(heroes[h] >= 5 for h in ("loop", "transpose", "row_reduce", "column_reduce")), heroes


def _low_bit(x: np.ndarray) -> np.ndarray:
    """Value of the lowest set bit of each finite nonzero f32 in x."""
    m, e = np.frexp(np.abs(x.astype(np.float64)))
    mi = (m * 2.0 ** 24).astype(np.int64)
    return np.ldexp((mi & -mi).astype(np.float64), e - 24)


def check_random_result(got, s, params):
    """Bit-exact against the oracle.  The one exception is an f32 sum whose
    terms do not make every partial sum exact: all terms are multiples of
    their smallest low bit q, so any partial sum below 2^24 q is exact in
    f32 and every summation order gives the oracle's rounded exact sum; an
    output whose sum of |terms| reaches 2^24 q may differ from it by at most
    (n - 1) 2^-24 sum|terms| for n terms (any order, Operation semantics,
    "Reduce": the order of a float sum is left to the implementation)."""
    root = s.nodes[-1]
    dt = root["dtype"]
    want = oracle.evaluate(s.nodes, params)
    try:
        assert_bitexact(got, want, "u8" if dt in ("s4", "u4") else dt)
        return
    except AssertionError:
        if not (root["op"] == "reduce" and root["reducer"] == "add" and dt == "f32"):
            raise
    terms = oracle.evaluate(s.nodes, params, root=root["operands"][0]).view(np.float32)
    fin = terms[np.isfinite(terms) & (terms != 0)]
    q = _low_bit(fin).min() if fin.size else np.inf
    dims = root["dims"]
    n_out = math.prod(dims)
    n_terms = terms.size // max(n_out, 1)
    idx = np.indices(dims).reshape(len(dims), -1).T if dims else np.zeros((1, 0), np.int64)
    _, aux = oracle.evaluate_points(s.nodes, params, idx)
    m2m = root.get("m2m") or list(range(len(dims) - 1, -1, -1))
    lin, stride = np.zeros(len(idx), np.int64), 1
    for d in m2m:
        lin += idx[:, d] * stride
        stride *= dims[d]
    g = got.view(np.float32)[lin].astype(np.float64)
    w = want.view(np.float32)[lin].astype(np.float64)
    bad = np.flatnonzero(~((g == w) | (np.isnan(g) & np.isnan(w))))
    total, exact = aux[bad, 0], aux[bad, 1]
    assert np.all(np.isfinite(total)) and np.all(total >= 2.0 ** 24 * q), (
        "outputs whose partial sums are all exact differ", bad[:5], g[bad[:5]], w[bad[:5]])
    assert np.all(np.abs(g[bad] - exact) <= (n_terms - 1) * 2.0 ** -24 * total), (
        "sums outside the summation bound", bad[:5], g[bad[:5]], exact[:5])


def test_sum_checker_accepts_only_what_the_order_allows():
    """check_random_result on oracle results with a planted change: a sum of
    65,536 terms in steps of 1/8 that reach 9.5 M in magnitude (its exact
    value, -7917890.625, lies between two f32 values, and a different order
    may give either) passes one ulp off but not 10^6 off; a sum whose terms
    keep every partial sum exact fails one ulp off."""
    s, params = _make(20129, "wide")
    want = oracle.evaluate(s.nodes, params)
    check_random_result(want.copy(), s, params)
    off = want.view(np.uint32).copy()
    off[0] += 1
    check_random_result(off.view(np.float32), s, params)
    far = want.copy()
    far[0] += np.float32(1e6)
    with pytest.raises(AssertionError):
        check_random_result(far, s, params)
    s, params = _make(3001, "wide")
    want = oracle.evaluate(s.nodes, params)
    check_random_result(want.copy(), s, params)
    off = want.view(np.uint32).copy()
    off[0] += 1
    with pytest.raises(AssertionError):
        check_random_result(off.view(np.float32), s, params)


@pytest.mark.gpu
@pytest.mark.parametrize("batch", range((N_CASES + N_HERO + N_WIDE + N_BIG + N_RANK + N_WRANK + N_SPECIAL + N_Q8) // BATCH))
def test_random_fusions_gpu(batch):
    import compiler_hlo_amd as H
    for seed, series in _cases()[batch * BATCH:(batch + 1) * BATCH]:
        s, params = _make(seed, series)
        try:
            H.Fusion(s.nodes, mode="plan")
        except H.FusionError:
            continue
        print("random fusion seed", seed, [nd["op"] for nd in s.nodes], flush=True)
        got, f = run_gpu(s.nodes, params)
        check_random_result(got, s, params)


def test_random_transcendental_fusions_plan_and_check_oracle():
    """Every transcendental case plans (or is HF_ERR_UNSUPPORTED), and each
    case's checker accepts the oracle's own result."""
    import compiler_hlo_amd as H
    planned = 0
    for k in range(N_TRANS):
        s, params, check = random_trans_case(5000 + k, specials=k >= BATCH)
        try:
            H.Fusion(s.nodes, mode="plan")
        except H.FusionError as e:
            assert e.status == "HF_ERR_UNSUPPORTED", (5000 + k, str(e))
            continue
        planned += 1
        check(oracle.evaluate(s.nodes, params))
    assert planned >= N_TRANS * 3 // 4


@pytest.mark.gpu
@pytest.mark.parametrize("batch", range(N_TRANS // BATCH))
def test_random_transcendental_fusions_gpu(batch):
    import compiler_hlo_amd as H
    for k in range(batch * BATCH, (batch + 1) * BATCH):
        s, params, check = random_trans_case(5000 + k, specials=k >= BATCH)  # the second batch: NaN, inf, +-0
        try:
            H.Fusion(s.nodes, mode="plan")
        except H.FusionError:
            continue
        print("random transcendental fusion seed", 5000 + k, [nd["op"] for nd in s.nodes], flush=True)
        got, _ = run_gpu(s.nodes, params)
        check(got)
