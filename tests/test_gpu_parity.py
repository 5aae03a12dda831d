"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every case draws seeded synthetic inputs (workloads), runs the fusion on the
GPU through compiler_hlo_amd (ctypes -> libhlofusion.so -> hiprtc-compiled
gfx950 kernels) and compares element by element with the oracle, to the
tolerance of the operation:
  * data movement, integer and quantized results: bit-exact;
  * f32 exp/log: within 2 ulp (ordinal distance on f32 bit patterns);
  * bf16 results of transcendentals: within 1 bf16 ulp;
  * float sums: |gpu - S| <= 1e-5 * sum|y| with S the oracle's long-double sum;
  * max/min reductions: bit-exact.
"""
import itertools

import numpy as np
import pytest

import oracle
import workloads as W
from harness import (assert_bitexact, assert_ulp, run_gpu, to_device, from_device,
                     ulp_dist_f32)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import compiler_hlo_amd  # noqa: F401  (fails loudly without the library)
    yield


def say(*a):
    print(*a, flush=True)


# --------------------------------------------------------------------------
# loop hero: per-axis dequantize + bias + requantize (bit-exact int8)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("r,c", [(37, 160), (5, 48), (3, 24), (7, 33), (1, 1), (300, 4096)])
def test_quant_small(r, c):
    say("quant", r, c)
    spec, params, _ = W.quant_dequant_bias_requant(r, c, seed=60 + r)
    got, f = run_gpu(spec.nodes, params)
    assert f.plan()["hero"] == "loop"
    want = oracle.evaluate(spec.nodes, params)
    assert_bitexact(got, want, "s8")


def test_quant_full():
    spec, params, _ = W.quant_dequant_bias_requant()
    say("quant full")
    got, f = run_gpu(spec.nodes, params, reps=2)
    want = oracle.evaluate(spec.nodes, params)
    assert_bitexact(got, want, "s8")
    clamped = np.mean((want == 127) | (want == -128))
    say("clamped fraction", clamped)


@pytest.mark.parametrize("r,c", [(1030, 4096), (4091, 4096), (4096, 4096), (257, 8192), (64, 1024),
                                 (1, 16), (5, 48)])
def test_quant_pipelined_rows(r, c):
    """The per-axis requantize on the pipelined loop (8-bit streams): row
    counts that leave the last row of some threads past the end, threads
    with no row at all (fewer rows than a workgroup's row slots), and grids
    of one to sixteen rows a thread; bit-exact."""
    spec, params, _ = W.quant_dequant_bias_requant(r, c, seed=90 + r % 7)
    got, f = run_gpu(spec.nodes, params)
    src = f.source()
    say("quant pipelined", r, c, f.plan()["grid_blocks"],
        [l for l in src.splitlines() if l.startswith(("#define HF_PIPE", "#define HF_NR"))])
    assert "#define HF_PIPE 0" not in src
    assert_bitexact(got, oracle.evaluate(spec.nodes, params), "s8")


def test_pipelined_loop_row_and_column_data():
    """Pipelined 8-bit loops whose small arrays move with the row (per-axis
    dequantize along dim 0, a bias broadcast along dim 0) and with the column
    (a per-axis quantize of the result along dim 1, with its reciprocal
    scales), plus a rank-0 parameter: the row-dependent ones are fetched
    with each row, the others once.  Bit-exact against the oracle."""
    g = W.rng(93)
    r, c = 2053, 2048
    q = W.integers(g, r * c, -128, 127, np.int8)
    s_in = W.uniform_f32(g, r, 0.001, 0.05)
    z_in = W.integers(g, r, -20, 20, np.int64)
    s_out = W.uniform_f32(g, c, 0.01, 0.04)
    z_out = W.integers(g, c, -10, 10, np.int64)
    brow = W.normal_f32(g, r, 0.1)
    k = np.array(0.03125, np.float32)
    s = W.Spec()
    p = s.parameter(0, "s8", [r, c], quant=W.quant_type("s8", s_in, z_in, qdim=0))
    b = s.parameter(1, "f32", [r])
    kk = s.parameter(2, "f32", [])
    d = s.op("uniform_dequantize", [p], "f32", [r, c])
    bb = s.broadcast_in_dim(b, [0], "f32", [r, c])
    kb = s.broadcast_in_dim(kk, [], "f32", [r, c])
    y = s.binary("add", s.binary("add", d, bb, "f32", [r, c]), kb, "f32", [r, c])
    s.op("uniform_quantize", [y], "s8", [r, c], quant=W.quant_type("s8", s_out, z_out, qdim=1))
    ps = [q, brow, k]
    got, f = run_gpu(s.nodes, ps)
    src = f.source()
    assert "#define HF_PIPE 0" not in src and f.plan()["n_partitions"] == 1
    assert_bitexact(got, oracle.evaluate(s.nodes, ps), "s8")


def test_quantized_add_pipelined_full():
    """The per-tensor quantized add of i8[4096,4096] (pipelined, sixteen rows
    a thread), whole output bit-exact."""
    spec, params, _ = W.quantized_add_i8()
    got, f = run_gpu(spec.nodes, params)
    assert "#define HF_PIPE 0" not in f.source()
    assert_bitexact(got, oracle.evaluate(spec.nodes, params), "s8")


@pytest.mark.parametrize("case", ["gelu_bf16", "s4_requantize", "pad_reverse_concat_f32", "quantized_add_3_lanes"])
def test_pipeline_forced_by_its_knob(case, monkeypatch):
    """HF_LOOP_PIPE set above zero puts any single-partition loop on the
    pipeline, whatever its types and lane width: bf16 with a tanh, si4 with
    column data, f32 index transforms, and 8-bit rows of three lanes.  A
    grid of a few workgroups gives seven rows a thread, four in flight, the
    last row past the end for some threads.  Bit-exact against the oracle."""
    monkeypatch.setenv("HF_LOOP_PIPE", "4")
    spec, params, wgs, dt = {
        "gelu_bf16": lambda: (*W.gelu_bf16(1, 2053, 512)[:2], 80, "bf16"),
        "s4_requantize": lambda: (*W.quant_dequant_bias_requant_s4(2053, 512, seed=95)[:2], 160, "u8"),
        "pad_reverse_concat_f32": lambda: (*W.pad_reverse_concat_f32(1001, 256, 1050, seed=96)[:2], 80, "f32"),
        "quantized_add_3_lanes": lambda: (*W.quantized_add_i8(2053, 24, seed=97)[:2], 4, "s8"),
    }[case]()
    monkeypatch.setenv("HF_LOOP_WGS", str(wgs))
    got, f = run_gpu(spec.nodes, params)
    src = f.source()
    say("forced pipeline", case, [l for l in src.splitlines() if l.startswith(("#define HF_PIPE", "#define HF_NR"))])
    assert "#define HF_PIPE 4" in src and "#define HF_NR 7" in src
    assert_bitexact(got, oracle.evaluate(spec.nodes, params), dt)


@pytest.mark.parametrize("r,c", [(37, 160), (5, 48), (3, 2), (300, 4096)])
def test_quant_s4_small(r, c):
    """The per-axis requantize with si4 storage in and out: bytes bit-exact."""
    say("quant s4", r, c)
    spec, params, _ = W.quant_dequant_bias_requant_s4(r, c, seed=70 + r)
    got, f = run_gpu(spec.nodes, params)
    assert f.plan()["hero"] == "loop"
    assert_bitexact(got, oracle.evaluate(spec.nodes, params), "u8")


def test_quant_s4_full():
    spec, params, _ = W.quant_dequant_bias_requant_s4()
    say("quant s4 full")
    got, f = run_gpu(spec.nodes, params, reps=2)
    want = oracle.evaluate(spec.nodes, params)
    assert_bitexact(got, want, "u8")
    lo, hi = want & 0xF, want >> 4
    say("clamped fraction", np.mean(np.isin(np.concatenate([lo, hi]), (7, 8))))


def _four_bit_cases():
    """(name, spec, params) for the 4-bit element paths of every hero."""
    g = W.rng(71)
    q = W.quant_type("s4", [0.05], [1])
    qa = W.quant_type("s4", np.linspace(0.01, 0.1, 64).astype(np.float32), np.arange(64) % 16 - 8, qdim=1)
    qu = W.quant_type("u4", [0.5], [8])
    cases = []
    s = W.Spec()
    p = s.parameter(0, "s4", [100, 64], quant=qa)
    s.op("uniform_dequantize", [p], "f32", [100, 64])
    cases.append(("dequantize s4 per-axis, 2-byte runs", s, [W.integers(g, 3200, 0, 255, np.uint8)]))
    s = W.Spec()
    p = s.parameter(0, "s4", [37, 33], quant=q)
    s.op("uniform_dequantize", [p], "f32", [37, 33])
    cases.append(("dequantize s4, odd dims, per element", s, [W.integers(g, 611, 0, 255, np.uint8)]))
    s = W.Spec()
    p = s.parameter(0, "f32", [100, 64])
    s.op("uniform_quantize", [p], "s4", [100, 64], quant=q)
    cases.append(("quantize to s4", s, [W.normal_f32(g, 6400, 0.3)]))
    s = W.Spec()
    p = s.parameter(0, "f32", [100, 6])
    s.op("uniform_quantize", [p], "u4", [100, 6], quant=qu)
    cases.append(("quantize to u4, one byte per lane", s, [W.normal_f32(g, 600, 3.0)]))
    s = W.Spec()
    a = s.parameter(0, "s4", [64, 128], quant=q)
    b = s.parameter(1, "s4", [64, 128], quant=W.quant_type("s4", [0.03], [-2]))
    s.op("add", [a, b], "s4", [64, 128], quant=W.quant_type("s4", [0.1], [0]))
    cases.append(("quantized add s4", s, [W.integers(g, 4096, 0, 255, np.uint8), W.integers(g, 4096, 0, 255, np.uint8)]))
    for dt in ("s4", "u4"):
        s = W.Spec()
        p = s.parameter(0, dt, [64, 128])
        s.convert(p, "f32", [64, 128])
        cases.append(("convert %s" % dt, s, [W.integers(g, 4096, 0, 255, np.uint8)]))
        s = W.Spec()
        s.parameter(0, dt, [64, 128])
        cases.append(("copy %s" % dt, s, [W.integers(g, 4096, 0, 255, np.uint8)]))
    s = W.Spec()
    p = s.parameter(0, "f32", [256, 512])
    t = s.transpose(p, [1, 0], "f32", [512, 256])
    s.op("uniform_quantize", [t], "s4", [512, 256], quant=q)
    cases.append(("transpose into s4 (loop)", s, [W.normal_f32(g, 256 * 512, 0.3)]))
    s = W.Spec()
    p = s.parameter(0, "s4", [200, 520], quant=q)
    d = s.op("uniform_dequantize", [p], "f32", [200, 520])
    s.transpose(d, [1, 0], "f32", [520, 200])
    cases.append(("transpose of s4 (ragged tiles)", s, [W.integers(g, 52000, 0, 255, np.uint8)]))
    s = W.Spec()
    p = s.parameter(0, "u4", [70, 4096], quant=qu)
    d = s.op("uniform_dequantize", [p], "f32", [70, 4096])
    s.reduce(d, [1], "add", 0.0, "f32", [70])
    cases.append(("row sum over u4 (exact)", s, [W.integers(g, 143360, 0, 255, np.uint8)]))
    s = W.Spec()
    p = s.parameter(0, "u4", [4100, 64], quant=qu)
    d = s.op("uniform_dequantize", [p], "f32", [4100, 64])
    s.reduce(d, [0], "max", float("-inf"), "f32", [64])
    cases.append(("column max over u4", s, [W.integers(g, 131200, 0, 255, np.uint8)]))
    s = W.Spec()
    p = s.parameter(0, "s4", [0, 64], quant=q)
    s.op("uniform_dequantize", [p], "f32", [0, 64])
    cases.append(("empty s4", s, [np.zeros(0, np.uint8)]))
    return cases


@pytest.mark.parametrize("k", range(14))
def test_four_bit_paths(k):
    """si4/ui4 reads through every hero and 4-bit writes through the loop
    hero: bit-exact against the oracle (dequantized values are small
    multiples of their scale, so the sums here are exact)."""
    name, s, params = _four_bit_cases()[k]
    say("4-bit:", name)
    got, f = run_gpu(s.nodes, params)
    say("  hero", f.plan()["hero"], "V", f.plan()["vector_elems"])
    want = oracle.evaluate(s.nodes, params)
    dt = s.nodes[-1]["dtype"]
    assert_bitexact(got, want, "u8" if dt in ("s4", "u4") else dt)


def test_quant_zero_point_and_ties():
    """Per-tensor requantize with a non-zero output zero point, on values
    placed next to the rounding ties of y / scale."""
    sc = np.float32(0.02)
    centers = ((np.arange(-130, 130) + 0.5) * 0.02).astype(np.float32).view(np.int32)
    y = np.concatenate([(centers + off).view(np.float32) for off in range(-8, 8)])
    y = y[: (y.size // 16) * 16]
    for zp in (0, 7, -20):
        s = W.Spec()
        p = s.parameter(0, "f32", [y.size])
        s.op("uniform_quantize", [p], "s8", [y.size], quant=W.quant_type("s8", [sc], [zp]))
        got, _ = run_gpu(s.nodes, [y])
        assert_bitexact(got, oracle.evaluate(s.nodes, [y]), "s8")


# --------------------------------------------------------------------------
# loop hero with a transposed read: add(log p, transpose(log p))
# --------------------------------------------------------------------------
def _log_pair_bound(x, n, got):
    s = W.Spec()
    p = s.parameter(0, "f32", [n, n], [1, 0])
    s.unary("log", p, "f32", [n, n])
    L = oracle.evaluate(s.nodes, [x]).reshape(n, n)
    g = got.reshape(n, n)
    exact = L.astype(np.float64) + L.T.astype(np.float64)
    ulp = lambda v: np.spacing(np.abs(v).astype(np.float32)).astype(np.float64)
    bound = 2 * ulp(L) + 2 * ulp(L.T) + 0.5 * ulp(g)
    assert np.all(np.abs(g.astype(np.float64) - exact) <= bound)
    assert np.array_equal(g.view(np.uint32), g.T.view(np.uint32)), "not symmetric"


@pytest.mark.parametrize("n", [64, 5, 33, 100, 128])
def test_loop_log_transpose_add(n):
    say("log-transpose-add", n)
    spec, params, _ = W.loop_log_transpose_add(n, seed=10 + n)
    got, f = run_gpu(spec.nodes, params)
    pl = f.plan()
    assert pl["hero"] == "loop" and pl["n_partitions"] == 3
    _log_pair_bound(params[0], n, got)


# --------------------------------------------------------------------------
# transpose hero
# --------------------------------------------------------------------------
@pytest.mark.parametrize("n0,n1", [(200, 300), (130, 70), (64, 64), (1, 5), (5, 1), (3, 1000), (257, 129)])
def test_transpose_exp_small(n0, n1):
    say("transpose exp", n0, n1)
    spec, params, _ = W.transpose_exp_f32(n0, n1, seed=20 + n0)
    got, f = run_gpu(spec.nodes, params)
    want = oracle.evaluate(spec.nodes, params)
    assert_ulp(got, want, "f32", 2)


@pytest.mark.parametrize("dims,perm,tile,block", [([100, 2048], [1, 0], (128, 32), 1024),
                                                  ([3, 36, 4096], [0, 2, 1], (128, 32), 1024),
                                                  ([8, 2048], [1, 0], (128, 8), 256),
                                                  ([16380, 1024], [1, 0], (128, 32), 1024),
                                                  ([65536, 256], [1, 0], (128, 32), 1024),
                                                  ([8, 4100, 256], [0, 2, 1], (128, 32), 1024),
                                                  ([2052, 8192], [1, 0], (128, 32), 1024),
                                                  ([1000, 32768], [1, 0], (128, 32), 1024),
                                                  ([1000, 1024], [1, 0], (32, 32), 256),
                                                  ([100004, 128], [1, 0], (128, 32), 1024)])
def test_transpose_narrow_tiles(dims, perm, tile, block):
    """f32 transposes whose input rows lie a power of two (>= 8 KiB) apart take
    tiles 128 wide in the load and up to 32 in the store, with 1024 threads
    when each thread then moves one vector per phase; rows of 512 B to 4 KiB
    do too when that makes 2048 workgroups or more (f32[1000,1024] would make
    256 and takes 32x32 tiles).  The tile orders run here: W fastest (4 KiB
    rows), diagonal (f32[2052,8192]), U fastest (f32[65536,256],
    f32[1000,32768]).
    Ragged U extents (100, 36, 16380, 4100, 2052, 1000, 100004) take the
    bounds-checked path; rows of 128 floats are a single W-tile.  The exp before the tile is checked against the
    oracle and bitwise against the same exp through the loop hero, transposed
    on the host."""
    say("transpose narrow tiles", dims, perm)
    n = int(np.prod(dims))
    out_dims = [dims[p] for p in perm]
    s = W.Spec()
    x = s.parameter(0, "f32", dims)
    e = s.unary("exponential", x, "f32", dims)
    s.transpose(e, perm, "f32", out_dims)
    params = [W.normal_f32(W.rng(60 + dims[0]), n)]
    got, f = run_gpu(s.nodes, params)
    p = f.plan()
    assert p["hero"] == "transpose" and (p["tile_rows"], p["tile_cols"]) == tile and p["block_threads"] == block
    assert_ulp(got, oracle.evaluate(s.nodes, params), "f32", 2)
    s2 = W.Spec()
    x2 = s2.parameter(0, "f32", dims)
    s2.unary("exponential", x2, "f32", dims)
    e2, f2 = run_gpu(s2.nodes, params)
    assert f2.plan()["hero"] == "loop"
    want = np.transpose(e2.reshape(dims), perm).ravel()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("dims", [(20, 160, 170), (3, 7, 67)])
def test_transpose3d_with_epilogue(dims):
    """The transpose emitter's 3-D example: abs(transpose(exp(x), {2,1,0}));
    abs runs on the values read back from the tile."""
    say("transpose3d exp abs", dims)
    spec, params, _ = W.transpose3d_exp_abs(*dims, seed=30 + dims[0])
    got, f = run_gpu(spec.nodes, params)
    assert f.plan()["hero"] == "transpose"
    want = oracle.evaluate(spec.nodes, params)
    assert_ulp(got, want, "f32", 2)
    assert not np.signbit(np.asarray(got, np.float32)).any()


def test_transpose_exp_full_and_loop_invariant():
    spec, params, _ = W.transpose_exp_f32()
    say("transpose exp full")
    got, f = run_gpu(spec.nodes, params, reps=2)
    assert f.plan()["hero"] == "transpose"
    want = oracle.evaluate(spec.nodes, params)
    d = assert_ulp(got, want, "f32", 2)
    say("ulp histogram", np.bincount(d.astype(np.int64)))
    # the same exp through the loop hero, transposed on the host: bitwise equal
    s = W.Spec()
    x = s.parameter(0, "f32", [4096, 4096], [1, 0])
    s.unary("exponential", x, "f32", [4096, 4096])
    e, fl = run_gpu(s.nodes, params)
    assert fl.plan()["hero"] == "loop"
    assert np.array_equal(got.reshape(4096, 4096).view(np.uint32), e.reshape(4096, 4096).T.view(np.uint32))


@pytest.mark.parametrize("b,m,n", [(3, 40, 72), (2, 130, 64), (4, 17, 9), (1, 1, 8), (5, 64, 1)])
def test_transpose_bf16_small(b, m, n):
    say("transpose bf16", b, m, n)
    spec, params, _ = W.transpose_bf16_021(b, m, n, seed=30 + m)
    got, _ = run_gpu(spec.nodes, params)
    assert_bitexact(got, oracle.evaluate(spec.nodes, params), "bf16")


@pytest.mark.parametrize("b,m,n,order", [(1, 4100, 2048, 2), (2, 1000, 16384, 0)])
def test_transpose_bf16_tile_orders(b, m, n, order):
    """bf16 transposes in the diagonal order (rows of 4 KiB, 65 U-tiles for
    32 W-tiles, the last U-tile ragged) and in U-fastest order (rows of
    32 KiB, 256 W-tiles for 16 U-tiles), bit-exact against the oracle."""
    say("transpose bf16 tile order", b, m, n, order)
    spec, params, _ = W.transpose_bf16_021(b, m, n, seed=31 + order)
    got, f = run_gpu(spec.nodes, params)
    assert f"#define HF_ORDER {order}\n" in f.source()
    assert_bitexact(got, oracle.evaluate(spec.nodes, params), "bf16")


def test_transpose_bf16_full():
    """The {0,2,1} transpose of bf16[64,512,1024] at full size: all
    33,554,432 outputs against the oracle's whole evaluation, bit-exact."""
    spec, params, _ = W.transpose_bf16_021()
    say("transpose bf16 full")
    got, f = run_gpu(spec.nodes, params, reps=2)
    assert f.plan()["hero"] == "transpose"
    assert_bitexact(got, oracle.evaluate(spec.nodes, params), "bf16")


# --------------------------------------------------------------------------
# row reduce: sum over the minor dim of convert(add(exp x, broadcast b)) in bf16
# --------------------------------------------------------------------------
def _check_sum(got, spec, params, rows_idx, threaded=False):
    pts = np.asarray(rows_idx, dtype=np.int64)
    if threaded:
        from harness import oracle_points_threaded
        vals, aux = oracle_points_threaded(spec.nodes, params, pts)
    else:
        vals, aux = oracle.evaluate_points(spec.nodes, params, pts)
    rn = spec.nodes[-1]
    lin = np.array([oracle.linear_index(rn["dims"], rn["m2m"] or oracle.default_m2m(len(rn["dims"])), p)
                    for p in pts])
    g = got[lin].astype(np.float64)
    err = np.abs(g - aux[:, 1])
    assert np.all(err <= 1e-5 * aux[:, 0]), "max err/bound %g" % np.max(err / np.maximum(aux[:, 0], 1e-300))


@pytest.mark.parametrize("d0,d2,d3", [(2, 5, 1000), (1, 3, 2048 + 8), (3, 7, 24), (2, 2, 5), (1, 1, 16384)])
def test_row_reduce_small(d0, d2, d3):
    say("row reduce", d0, d2, d3)
    spec, params, _ = W.row_reduce_exp_add_bf16(d0, d2, d3, seed=40 + d3)
    got, f = run_gpu(spec.nodes, params)
    assert f.plan()["hero"] == "row_reduce"
    _check_sum(got, spec, params, [[a, 0, c] for a in range(d0) for c in range(d2)])


def test_row_reduce_full_every_row_and_layout_invariant():
    """The row sum of exp(x) + bias over bf16[8,1,1280,16384] at full size:
    every one of the 10,240 sums within 1e-5 * sum|y| of the oracle's
    long-double sum (the oracle runs on the host's cores in parallel, a chunk
    of rows per thread)."""
    import time
    spec, params, _ = W.row_reduce_exp_add_bf16()
    say("row reduce full")
    got, f = run_gpu(spec.nodes, params, reps=2)
    rows = [[a, 0, c] for a in range(8) for c in range(1280)]
    t0 = time.time()
    _check_sum(got, spec, params, rows, threaded=True)
    say("  all %d rows checked against the oracle in %.1f s" % (len(rows), time.time() - t0))
    # {3,2,0,1} stores the same bytes (dim 1 has size 1): bitwise equal results
    spec2, params2, _ = W.row_reduce_exp_add_bf16(m2m=(3, 2, 0, 1))
    got2, _ = run_gpu(spec2.nodes, params2)
    assert np.array_equal(got.view(np.uint32), got2.view(np.uint32))


@pytest.mark.parametrize("rows", [65536, 70001])
def test_row_reduce_one_workgroup_per_row_and_past_the_cap(rows):
    """Whole-row workgroups take one row each up to 65,536 workgroups; past
    that the grid strides, so 70,001 rows leave 4,465 workgroups a second
    row.  Integer-valued f32 rows of 1028 (257 chunks over 256 threads, so
    one row a step; exact sums), bit-exact; a max over the same rows
    through the same grid."""
    say("row reduce rows", rows)
    g = W.rng(54)
    x = W.integers(g, rows * 1028, -1000, 1000, np.int64).astype(np.float32)
    for red, init in (("add", 0.0), ("max", float("-inf"))):
        s = W.Spec()
        p = s.parameter(0, "f32", [rows, 1028])
        s.reduce(p, [1], red, init, "f32", [rows])
        got, f = run_gpu(s.nodes, [x])
        assert f.plan()["hero"] == "row_reduce" and f.plan()["grid_blocks"] == 65536
        assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "f32")


@pytest.mark.parametrize("rows,cols", [(16, 1 << 20), (1, 3 * (1 << 20) + 4), (5, 100003), (3, 1 << 22)])
def test_row_reduce_split_rows(rows, cols):
    """A few long rows split over workgroups, each a segment of the row, and
    a fold kernel that combines each row's partials in order: sum, max and
    argmax of integer-valued f32 (exact, many ties and equal maxima in
    different segments), bit-exact; an odd row length (one element a lane,
    ragged last segment); a mean (the epilogue after the fold); and a second
    launch of the same handle with new values (the workspace is rewritten)."""
    say("row reduce split rows", rows, cols)
    g = W.rng(56 + rows)
    x = W.integers(g, rows * cols, -50, 50, np.int64).astype(np.float32)
    for red in ("add", "max", "argmax"):
        s = W.Spec()
        p = s.parameter(0, "f32", [rows, cols])
        if red == "argmax":
            s.argmax(p, 1, [rows, cols])
        else:
            s.reduce(p, [1], red, 0.0 if red == "add" else float("-inf"), "f32", [rows])
        got, f = run_gpu(s.nodes, [x])
        assert "#define HF_RSEG 1\n" not in f.source() and f.plan()["workspace_bytes"] > 0
        assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "s32" if red == "argmax" else "f32")
        if red == "argmax":
            x2 = x.copy()
            x2[::7] = 49.0  # new maxima, in every segment
            got2, _ = run_gpu(s.nodes, [x2], fusion=f)
            assert_bitexact(got2, oracle.evaluate(s.nodes, [x2]), "s32")
    y = W.normal_f32(g, rows * cols)
    s = W.Spec()
    p = s.parameter(0, "f32", [rows, cols])
    r = s.reduce(p, [1], "add", 0.0, "f32", [rows])
    s.binary("divide", r, s.constant(float(cols), "f32", [rows]), "f32", [rows])
    got, f = run_gpu(s.nodes, [y])
    want = np.asarray(oracle.evaluate(s.nodes, [y]), np.float64)
    bound = 1e-5 * np.abs(y.reshape(rows, cols)).astype(np.float64).sum(1) / cols + np.spacing(np.abs(want).astype(np.float32))
    assert (np.abs(np.asarray(got, np.float64) - want) <= bound).all()


def test_reduce_of_every_dim_splits_its_one_row():
    """A reduce over every dim of f32[4096,4096] (one output, one row of
    16.8 M elements): 1024 segments and the fold; integer values, exact."""
    g = W.rng(57)
    x = W.integers(g, 4096 * 4096, -8, 8, np.int64).astype(np.float32)
    s = W.Spec()
    p = s.parameter(0, "f32", [4096, 4096])
    s.reduce(p, [0, 1], "add", 0.0, "f32", [])
    got, f = run_gpu(s.nodes, [x])
    assert f.plan()["hero"] == "row_reduce" and f.plan()["grid_blocks"] >= 1024
    assert got.reshape(-1)[0] == np.float32(x.astype(np.float64).sum())


@pytest.mark.parametrize("rows,cols", [(70001, 256), (4099, 512), (37, 1020), (8, 1024)])
def test_row_reduce_one_wave_per_row(rows, cols):
    """Rows of 64 to 255 vectors take one wave each, four rows a workgroup,
    over at most 2048 workgroups (a grid stride past them; a last step with
    fewer rows than its four slots): sum, max and argmax of integer-valued
    f32 (exact, with many ties), bit-exact."""
    say("row reduce one wave per row", rows, cols)
    g = W.rng(55 + cols % 7)
    x = W.integers(g, rows * cols, -20, 20, np.int64).astype(np.float32)
    for red in ("add", "max", "argmax"):
        s = W.Spec()
        p = s.parameter(0, "f32", [rows, cols])
        if red == "argmax":
            s.argmax(p, 1, [rows, cols])
        else:
            s.reduce(p, [1], red, 0.0 if red == "add" else float("-inf"), "f32", [rows])
        got, f = run_gpu(s.nodes, [x])
        if cols // 4 < 256:
            assert f.plan()["block_threads"] == 256 and "#define HF_TPR 64" in f.source()
        assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "s32" if red == "argmax" else "f32")


@pytest.mark.parametrize("dt,rows,cols", [("f32", 7, 524292), ("bf16", 5, 1048580), ("f32", 3, 512004)])
def test_loop_long_rows(dt, rows, cols):
    """Rows of 2 MiB or more run whole-workgroup row segments (256 lanes);
    x + a broadcast bias along the row, with an odd row count and a ragged
    last segment, bit-exact against the oracle (rows of 2 MiB + 16 and
    2 MiB + 8 bytes; f32 rows of 2,048,016 bytes keep 64 lanes)."""
    say("loop long rows", dt, rows, cols)
    g = W.rng(58 + rows)
    s = W.Spec()
    x = s.parameter(0, dt, [rows, cols])
    b = s.parameter(1, dt, [cols])
    s.binary("add", x, s.broadcast_in_dim(b, [1], dt, [rows, cols]), dt, [rows, cols])
    mk = W.normal_f32 if dt == "f32" else W.normal_bf16
    params = [mk(g, rows * cols), mk(g, cols)]
    got, f = run_gpu(s.nodes, params)
    lanes = 256 if cols * (4 if dt == "f32" else 2) >= 2 << 20 else 64
    assert f.plan()["hero"] == "loop" and "#define HF_TPR %d\n" % lanes in f.source()
    assert_bitexact(got, oracle.evaluate(s.nodes, params), dt)


@pytest.mark.parametrize("rows,cols", [(262147, 64), (1048583, 16), (300001, 12)])
def test_row_reduce_many_short_rows(rows, cols):
    """Rows of fewer than 64 vectors share a wave (16, 4 and 3 vectors a
    row: 16, 64 and 64 rows a workgroup) over 2048 workgroups, each looping
    over 2 to 9 steps of rows, the last one partly empty: sum, max and argmax
    of integer-valued f32 (exact, with many ties), bit-exact."""
    say("row reduce many short rows", rows, cols)
    g = W.rng(57 + cols)
    x = W.integers(g, rows * cols, -20, 20, np.int64).astype(np.float32)
    for red in ("add", "max", "argmax"):
        s = W.Spec()
        p = s.parameter(0, "f32", [rows, cols])
        if red == "argmax":
            s.argmax(p, 1, [rows, cols])
        else:
            s.reduce(p, [1], red, 0.0 if red == "add" else float("-inf"), "f32", [rows])
        got, f = run_gpu(s.nodes, [x])
        assert f.plan()["hero"] == "row_reduce" and f.plan()["grid_blocks"] == 2048
        assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "s32" if red == "argmax" else "f32")


@pytest.mark.parametrize("d0,d2,d3", [(1, 5, 32768), (3, 3, 36864)])
def test_row_reduce_two_rows_per_step(d0, d2, d3):
    """Rows of eight or more chunks per thread, and rows of exactly one, are
    reduced two per workgroup step: odd row counts leave one row in the last
    step, and 36864 (nine chunks) leaves a partial batch of loads."""
    say("row reduce two rows per step", d0, d2, d3)
    spec, params, _ = W.row_reduce_exp_add_bf16(d0, d2, d3, seed=50 + d2)
    got, f = run_gpu(spec.nodes, params)
    assert "#define HF_RR_ROWS 2" in f.source()
    _check_sum(got, spec, params, [[a, 0, c] for a in range(d0) for c in range(d2)])
    g = W.rng(51)
    for rows, cols, red in ((37, 16384, "max"), (7, 20480, "add"), (4097, 2048, "add"), (4099, 1024, "max")):
        x = W.integers(g, rows * cols, -1000, 1000, np.int64).astype(np.float32)  # exact sums
        s = W.Spec()
        p = s.parameter(0, "f32", [rows, cols])
        s.reduce(p, [1], red, float("-inf") if red == "max" else 0.0, "f32", [rows])
        got, f = run_gpu(s.nodes, [x])
        assert "#define HF_RR_ROWS 2" in f.source()
        assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "f32")


def test_row_reduce_pipelined_option(monkeypatch):
    """The optional pipelined row path (next row's loads in flight while the
    current one is accumulated; results stored after the loop), on a grid of
    5 workgroups so that they take different, odd and even, row counts."""
    monkeypatch.setenv("HF_ROW_PIPE", "1")
    monkeypatch.setenv("HF_ROW_WGS", "5")
    spec, params, _ = W.row_reduce_exp_add_bf16(3, 7, 16384, seed=52)
    got, f = run_gpu(spec.nodes, params)
    assert "#define HF_RR_PIPE 1" in f.source() and f.plan()["grid_blocks"] == 5
    _check_sum(got, spec, params, [[a, 0, c] for a in range(3) for c in range(7)])
    g = W.rng(53)
    for rows in (23, 4, 1):
        x = W.normal_f32(g, rows * 4096)
        s = W.Spec()
        p = s.parameter(0, "f32", [rows, 4096])
        s.reduce(p, [1], "max", float("-inf"), "f32", [rows])
        got, f = run_gpu(s.nodes, [x])
        assert "#define HF_RR_PIPE 1" in f.source()
        assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "f32")


@pytest.mark.parametrize("rows", [0, 1, 2, 3, 130])
def test_row_reduce_bf16_short_rows(rows):
    """Sums of short bf16 rows (2 to 32 lanes per row, rank-0 results among
    them), integer-valued so that every order gives the same f32: bit-exact.
    A single row of 8 once came out as +0: the packed accumulate read a
    v_dot2c_f32_bf16 result too soon after the instruction."""
    g = W.rng(96 + rows)
    for cols in (4, 8, 12, 16, 24, 40, 64, 128):
        for double in (False, True):
            shape = [cols] if rows == 0 else [rows, cols]
            s = W.Spec()
            p = s.parameter(0, "bf16", shape)
            y = s.binary("add", p, p, "bf16", shape) if double else p
            c = s.convert(y, "f32", shape)
            s.reduce(c, [len(shape) - 1], "add", 0.0, "f32", shape[:-1])
            v = W.integers(g, int(np.prod(shape)), -8, 8, np.int64).astype(np.float32)
            x = (v.view(np.uint32) >> 16).astype(np.uint16)
            got, f = run_gpu(s.nodes, [x])
            assert f.plan()["hero"] == "row_reduce"
            assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "f32")


def test_f16_chain_that_crashed_the_device_compiler():
    """The f16 negate/multiply chain on a rank-5 transposed read whose kernel
    once aborted the device compiler: now bit-exact against the oracle."""
    from test_library_cpu import _f16_negate_multiply_chain
    s = _f16_negate_multiply_chain()
    v = W.integers(W.rng(97), 17 * 4 * 3 * 16, -8, 8, np.int64).astype(np.float16)
    x = v.view(np.uint16)
    got, f = run_gpu(s.nodes, [x])
    assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "f16")


def test_row_reduce_bf16_intermediates_loop():
    """The reduce operand y = add(exp x, b) itself (a bf16 loop fusion) is
    within 1 bf16 ulp of the oracle elementwise."""
    s = W.Spec()
    dims = [2, 1, 16, 512]
    x = s.parameter(0, "bf16", dims)
    b = s.parameter(1, "bf16", [512], [0])
    e = s.unary("exponential", x, "bf16", dims)
    bc = s.broadcast_in_dim(b, [3], "bf16", dims)
    s.binary("add", e, bc, "bf16", dims)
    g = W.rng(41)
    params = [W.normal_bf16(g, 2 * 16 * 512), W.normal_bf16(g, 512)]
    got, _ = run_gpu(s.nodes, params)
    d = assert_ulp(got, oracle.evaluate(s.nodes, params), "bf16", 1)
    say("1-ulp fraction", float(np.mean(d > 0)))


def test_reductions_exact_on_integers():
    """Integer-valued inputs make every summation order exact: row and column
    sums are bit-exact."""
    g = W.rng(42)
    for dims, red, m2m in (([64, 300], [1], [1, 0]), ([300, 64], [0], [1, 0]), ([33, 70], [0], [0, 1]),
                           ([5, 6, 40], [0, 1], [2, 1, 0]), ([40, 5, 6], [1, 2], [2, 1, 0])):
        x = g.integers(-4, 5, int(np.prod(dims))).astype(np.float32)
        s = W.Spec()
        p = s.parameter(0, "f32", dims, m2m)
        kept = [dims[d] for d in range(len(dims)) if d not in red]
        s.reduce(p, red, "add", 0.0, "f32", kept)
        got, f = run_gpu(s.nodes, [x])
        say("exact sum", dims, red, m2m, f.plan()["hero"])
        assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "f32")


def test_quantized_elementwise_ops():
    """Elementwise ops on per-tensor quantized i8 tensors: dequantize, the op
    on f32 values, quantize to the result type.  The arithmetic ops round
    once in f32 on both sides: bit-exact."""
    g = W.rng(61)
    n0, n1 = 96, 1000
    a = W.integers(g, n0 * n1, -128, 127, np.int8)
    b = W.integers(g, n0 * n1, -128, 127, np.int8)
    qa, qb = W.quant_type("s8", [0.05], [3]), W.quant_type("s8", [0.02], [-7])
    qo = W.quant_type("s8", [0.04], [1])
    for op in ("add", "subtract", "multiply", "maximum", "minimum"):
        s = W.Spec()
        pa = s.parameter(0, "s8", [n0, n1], quant=qa)
        pb = s.parameter(1, "s8", [n0, n1], quant=qb)
        s.op(op, [pa, pb], "s8", [n0, n1], quant=qo)
        got, _ = run_gpu(s.nodes, [a, b])
        assert_bitexact(got, oracle.evaluate(s.nodes, [a, b]), "s8")
    for op in ("negate", "abs"):
        s = W.Spec()
        pa = s.parameter(0, "s8", [n0, n1], quant=qa)
        s.op(op, [pa], "s8", [n0, n1], quant=qo)
        got, _ = run_gpu(s.nodes, [a])
        assert_bitexact(got, oracle.evaluate(s.nodes, [a]), "s8")
    # a chain: quantized add, then a quantized maximum with a third tensor
    c = W.integers(g, n0 * n1, -128, 127, np.int8)
    s = W.Spec()
    pa = s.parameter(0, "s8", [n0, n1], quant=qa)
    pb = s.parameter(1, "s8", [n0, n1], quant=qb)
    pc = s.parameter(2, "s8", [n0, n1], quant=qo)
    ad = s.op("add", [pa, pb], "s8", [n0, n1], quant=qo)
    s.op("maximum", [ad, pc], "s8", [n0, n1], quant=qa)
    got, _ = run_gpu(s.nodes, [a, b, c])
    assert_bitexact(got, oracle.evaluate(s.nodes, [a, b, c]), "s8")


def test_quantized_exp_within_one_step():
    """exp on quantized values: the f32 exp of the device may differ from the
    correctly rounded one by an ulp, which can move a quotient across a
    rounding boundary: results within one storage step, and such steps rare."""
    g = W.rng(62)
    a = W.integers(g, 200000, -128, 127, np.int8)
    qa, qo = W.quant_type("s8", [0.02], [0]), W.quant_type("s8", [0.05], [-100])
    s = W.Spec()
    pa = s.parameter(0, "s8", [200000], quant=qa)
    s.op("exponential", [pa], "s8", [200000], quant=qo)
    got, _ = run_gpu(s.nodes, [a])
    want = oracle.evaluate(s.nodes, [a])
    d = np.abs(got.astype(np.int64) - want.astype(np.int64))
    assert d.max() <= 1 and (d > 0).mean() < 1e-3


def test_every_f32_elementwise_op():
    """Each f32 elementwise op on wide-range operands (subnormal results
    included): the IEEE arithmetic and sign ops bit-exact, the
    transcendentals within 2 ulp."""
    g = W.rng(133)
    n = 1 << 18
    a = (g.standard_normal(n) * np.exp2(g.integers(-130, 60, n))).astype(np.float32)
    b = (g.standard_normal(n) * np.exp2(g.integers(-130, 60, n))).astype(np.float32)
    pos = np.abs(a) + np.float32(1e-30)
    small = (g.standard_normal(n) * 4).astype(np.float32)
    for op in ("add", "subtract", "multiply", "divide", "maximum", "minimum"):
        s = W.Spec()
        x = s.parameter(0, "f32", [n])
        y = s.parameter(1, "f32", [n])
        s.binary(op, x, y, "f32", [n])
        got, _ = run_gpu(s.nodes, [a, b])
        assert_bitexact(got, oracle.evaluate(s.nodes, [a, b]), "f32")
    for op, arr, bar in (("negate", a, 0), ("abs", a, 0), ("log", pos, 2), ("exponential", small, 2),
                         ("tanh", small, 2)):
        s = W.Spec()
        x = s.parameter(0, "f32", [n])
        s.unary(op, x, "f32", [n])
        got, _ = run_gpu(s.nodes, [arr])
        want = oracle.evaluate(s.nodes, [arr])
        if bar == 0:
            assert_bitexact(got, want, "f32")
        else:
            assert_ulp(got, want, "f32", bar)


# --------------------------------------------------------------------------
# f16 and u8 element types
# --------------------------------------------------------------------------
def test_f16_paths():
    """f16 through each hero: an elementwise loop (add, convert), a transpose
    (bit-exact), a row sum of f16 values in f32, and f16 exp within an ulp."""
    g = W.rng(131)
    n0, n1 = 300, 520
    a = (g.standard_normal(n0 * n1) * 20).astype(np.float16).view(np.uint16)
    b = (g.standard_normal(n0 * n1) * 20).astype(np.float16).view(np.uint16)
    s = W.Spec()
    pa = s.parameter(0, "f16", [n0, n1])
    pb = s.parameter(1, "f16", [n0, n1])
    ad = s.binary("add", pa, pb, "f16", [n0, n1])
    s.binary("multiply", ad, pa, "f16", [n0, n1])
    got, f = run_gpu(s.nodes, [a, b])
    assert f.plan()["hero"] == "loop"
    assert_bitexact(got, oracle.evaluate(s.nodes, [a, b]), "f16")
    s = W.Spec()
    pa = s.parameter(0, "f16", [n0, n1])
    s.transpose(pa, [1, 0], "f16", [n1, n0])
    got, f = run_gpu(s.nodes, [a])
    assert f.plan()["hero"] == "transpose"
    assert_bitexact(got, oracle.evaluate(s.nodes, [a]), "f16")
    x = W.integers(g, n0 * n1, -6, 6, np.int64).astype(np.float16).view(np.uint16)
    s = W.Spec()
    pa = s.parameter(0, "f16", [n0, n1])
    cv = s.convert(pa, "f32", [n0, n1])
    s.reduce(cv, [1], "add", 0.0, "f32", [n0])
    got, f = run_gpu(s.nodes, [x])
    assert f.plan()["hero"] == "row_reduce"
    assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "f32")
    e = (g.standard_normal(n0 * n1) * 3).astype(np.float16).view(np.uint16)
    s = W.Spec()
    pa = s.parameter(0, "f16", [n0 * n1])
    s.unary("exponential", pa, "f16", [n0 * n1])
    got, _ = run_gpu(s.nodes, [e])
    assert_ulp(got, oracle.evaluate(s.nodes, [e]), "f16", 1)


def test_u8_quantize_dequantize():
    g = W.rng(132)
    y = W.uniform_f32(g, 200000, -80.0, 80.0)
    qt = W.quant_type("u8", [0.5], [128])
    s = W.Spec()
    p = s.parameter(0, "f32", [200000])
    s.op("uniform_quantize", [p], "u8", [200000], quant=qt)
    got, _ = run_gpu(s.nodes, [y])
    assert_bitexact(got, oracle.evaluate(s.nodes, [y]), "u8")
    q = W.integers(g, 300 * 256, 0, 255, np.uint8)
    s = W.Spec()
    p = s.parameter(0, "u8", [300, 256], quant=W.quant_type("u8", list(np.linspace(0.01, 0.2, 256)),
                                                               list(range(0, 256)), qdim=1))
    s.op("uniform_dequantize", [p], "f32", [300, 256])
    got, _ = run_gpu(s.nodes, [q])
    assert_bitexact(got, oracle.evaluate(s.nodes, [q]), "f32")


# --------------------------------------------------------------------------
# variadic max/argmax
# --------------------------------------------------------------------------
def test_long_rows():
    """Rows of 2^20 elements (512 chunks per thread, fetched in batches):
    an integer-valued sum (exact in any order) and an argmax."""
    g = W.rng(112)
    x = W.integers(g, 4 << 20, -3, 3, np.int64).astype(np.float32)
    s = W.Spec()
    p = s.parameter(0, "f32", [4, 1 << 20])
    s.reduce(p, [1], "add", 0.0, "f32", [4])
    got, _ = run_gpu(s.nodes, [x])
    assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "f32")
    s = W.Spec()
    p = s.parameter(0, "f32", [4, 1 << 20])
    s.argmax(p, 1, [4, 1 << 20])
    got, _ = run_gpu(s.nodes, [x])
    assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "s32")


@pytest.mark.parametrize("dims,rdim,dtype", [([64, 3000], 1, "f32"), ([3000, 64], 0, "f32"),
                                             ([16384, 512], 0, "f32"), ([100, 40], 1, "bf16"),
                                             ([7, 5], 1, "f32"), ([10240, 2048], 1, "bf16")])
def test_argmax(dims, rdim, dtype):
    """Integer-valued data: many ties, which must go to the last index."""
    say("argmax", dims, rdim, dtype)
    g = W.rng(111 + dims[0])
    n = int(np.prod(dims))
    x = W.integers(g, n, -20, 20, np.int64).astype(np.float32)
    if dtype == "bf16":
        x = (x.view(np.uint32) >> 16).astype(np.uint16)
    s = W.Spec()
    p = s.parameter(0, dtype, dims)
    s.argmax(p, rdim, dims)
    got, f = run_gpu(s.nodes, [x])
    say("  hero", f.plan()["hero"], "workspace", f.plan()["workspace_bytes"])
    assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "s32")


def test_argmax_rows_full():
    """The argmax over the rows of bf16[8192, 8192] ~ N(0,1) at full size, in
    the launch configuration the benchmark times: all 8,192 indices
    bit-exact."""
    spec, params, _ = W.argmax_rows_bf16()
    say("argmax rows full")
    got, f = run_gpu(spec.nodes, params, reps=2)
    assert f.plan()["hero"] == "row_reduce"
    assert_bitexact(got, oracle.evaluate(spec.nodes, params), "s32")


def test_argmax_nan_and_init_ties():
    nan, ninf = np.float32("nan"), np.float32("-inf")
    rows = np.array([[1, nan, 3, nan, 3], [nan] * 5, [ninf, ninf, 2, ninf, ninf], [ninf] * 5], np.float32)
    x = np.tile(rows, (1, 200))           # rows of 1000
    for rdim, arr in ((1, x), (0, np.ascontiguousarray(x.T))):
        s = W.Spec()
        p = s.parameter(0, "f32", list(arr.shape))
        s.argmax(p, rdim, list(arr.shape))
        got, _ = run_gpu(s.nodes, [arr.ravel()])
        assert_bitexact(got, oracle.evaluate(s.nodes, [arr.ravel()]), "s32")


@pytest.mark.parametrize("index_init", [0, "n+5", -1])
@pytest.mark.parametrize("n", [5, 3, 1000, 6000])
def test_argmax_index_init_inside_and_past_the_row(n, index_init):
    """Any s32 index init (Operation semantics, "Variadic Reduce": the fold
    starts from (init_value, index init)): all-NaN rows, rows of -inf, rows
    whose maximum equals the value init (2) at several positions, rows that
    never reach it, and ordinary rows, through the row hero (short rows in
    sub-wave mode, rows of 1000) and the column hero (6000 rows: split into
    segments, so the workspace and the fold kernel carry the partials).
    Bit-exact against the oracle."""
    nan, ninf = np.float32("nan"), np.float32("-inf")
    k0 = n + 5 if index_init == "n+5" else index_init
    g = W.rng(120 + n)
    rows = [np.full(n, nan), np.full(n, ninf), np.zeros(n), g.integers(-3, 3, n, endpoint=True)]
    r = g.integers(-3, 2, n, endpoint=True).astype(np.float32)   # max 2 = the value init, ties
    rows.append(r)
    r = np.where(g.random(n) < 0.5, nan, 2.0)                    # init-valued among NaNs
    rows.append(r)
    x = np.stack([np.asarray(v, np.float32) for v in rows] * 11)  # 66 rows
    for value_init in (2.0, float("-inf")):
        for rdim, arr in ((1, x), (0, np.ascontiguousarray(x.T))):
            s = W.Spec()
            p = s.parameter(0, "f32", list(arr.shape))
            s.argmax(p, rdim, list(arr.shape), index_init=k0, init=value_init)
            got, f = run_gpu(s.nodes, [arr.ravel()])
            want = oracle.evaluate(s.nodes, [arr.ravel()])
            assert_bitexact(got, want, "s32")
            if rdim == 0 and n == 6000:
                assert f.plan()["hero"] == "column_reduce" and f.plan()["workspace_bytes"] > 0
    say("argmax index init", k0, "rows of", n, "ok")


# --------------------------------------------------------------------------
# degenerate and maximum sizes
# --------------------------------------------------------------------------
def test_empty_and_degenerate_shapes():
    """Zero-size arrays launch nothing; a reduce over a zero-length dim gives
    init for every output (row and column layouts); a reduce to a scalar."""
    import torch
    for dims in ([0, 64], [64, 0], [3, 0, 5]):
        s = W.Spec()
        p = s.parameter(0, "f32", dims)
        s.unary("exponential", p, "f32", dims)
        got, _ = run_gpu(s.nodes, [np.zeros(0, np.float32)])
        assert got.size == 0
    s = W.Spec()
    p = s.parameter(0, "f32", [0, 64])
    s.transpose(p, [1, 0], "f32", [64, 0])
    got, _ = run_gpu(s.nodes, [np.zeros(0, np.float32)])
    assert got.size == 0
    for dims, rdim, m2m in (([37, 0], 1, [1, 0]), ([37, 0], 1, [0, 1]), ([0, 37], 0, [1, 0])):
        for red, init in (("add", 1.5), ("max", -2.0)):
            s = W.Spec()
            p = s.parameter(0, "f32", dims, m2m)
            s.reduce(p, [rdim], red, init, "f32", [37])
            got, f = run_gpu(s.nodes, [np.zeros(0, np.float32)])
            say("empty reduce", m2m, red, f.plan()["hero"])
            assert np.array_equal(got, np.full(37, init, np.float32))
            assert_bitexact(got, oracle.evaluate(s.nodes, [np.zeros(0, np.float32)]), "f32")
    g = W.rng(91)
    x = W.integers(g, 3000, -8, 8, np.int64).astype(np.float32)
    s = W.Spec()
    p = s.parameter(0, "f32", [3000])
    s.reduce(p, [0], "add", 0.0, "f32", [])
    got, _ = run_gpu(s.nodes, [x])
    assert got.reshape(-1)[0] == np.float32(x.astype(np.float64).sum())
    torch.cuda.synchronize()


@pytest.mark.parametrize("kind", ["loop", "transpose", "transpose_narrow", "row_reduce", "column_reduce"])
def test_largest_arrays_below_the_size_limit(kind):
    """f32[8191, 65536] is the largest 2-D f32 array below the 2 GiB limit:
    32-bit offsets reach their maximum.  f32[8188, 65536] (output rows a
    multiple of four) takes the 32x128 transpose tiles.  Sampled outputs
    against the oracle."""
    n0, n1 = (8188 if kind == "transpose_narrow" else 8191), 65536
    say("largest arrays", kind, n0, n1)
    g = W.rng(92)
    x = W.uniform_f32(g, n0 * n1, -4.0, 4.0)
    s = W.Spec()
    p = s.parameter(0, "f32", [n0, n1])
    e = s.unary("exponential", p, "f32", [n0, n1])
    if kind.startswith("transpose"):
        s.transpose(e, [1, 0], "f32", [n1, n0])
        odims = [n1, n0]
    elif kind.endswith("reduce"):
        d = 1 if kind == "row_reduce" else 0
        s.reduce(e, [d], "add", 0.0, "f32", [n1 - d * (n1 - n0)])
    else:
        odims = [n0, n1]
    got, f = run_gpu(s.nodes, [x])
    plan = f.plan()
    assert plan["hero"] == kind.replace("_narrow", "")
    if kind == "transpose_narrow":
        assert (plan["tile_rows"], plan["tile_cols"], plan["block_threads"]) == (128, 32, 1024), plan
    if kind.endswith("reduce"):
        nout = n0 if kind == "row_reduce" else n1
        idx = np.concatenate([g.integers(0, nout, 300 if kind == "row_reduce" else 3000), [0, nout - 1]])
        _check_sum(got, s, [x], idx[:, None])
    else:
        pts = np.stack([g.integers(0, odims[0], 20000), g.integers(0, odims[1], 20000)], 1)
        pts = np.concatenate([pts, [[0, 0], [odims[0] - 1, odims[1] - 1], [odims[0] - 1, 0], [0, odims[1] - 1]]])
        want, _ = oracle.evaluate_points(s.nodes, [x], pts)
        lin = pts[:, 0] * odims[1] + pts[:, 1]
        assert_ulp(got[lin], want.astype(np.float32), "f32", 2)
    del x, got


def test_largest_four_bit_array():
    """s4[32767, 65536] requantized to u4 after a per-tensor dequantize: 2^31 -
    65536 elements, the most below the 2^31 element limit, so nibble indices
    and byte offsets both reach their maximum (the f32 values between, 8 GiB,
    never reach memory).  Sampled outputs, bit-exact."""
    n0, n1 = 32767, 65536
    say("largest four-bit array", n0, n1)
    g = W.rng(93)
    q = np.frombuffer(bytearray(g.bytes(n0 * n1 // 2)), np.uint8)
    s = W.Spec()
    p = s.parameter(0, "s4", [n0, n1], quant=W.quant_type("s4", [0.25], [-1]))
    d = s.op("uniform_dequantize", [p], "f32", [n0, n1])
    s.op("uniform_quantize", [d], "u4", [n0, n1], quant=W.quant_type("u4", [0.5], [7]))
    got, f = run_gpu(s.nodes, [q])
    assert f.plan()["hero"] == "loop"
    assert got.dtype == np.uint8 and got.size == n0 * n1 // 2
    pts = np.stack([g.integers(0, n0, 20000), g.integers(0, n1, 20000)], 1)
    pts = np.concatenate([pts, [[0, 0], [n0 - 1, n1 - 1], [n0 - 1, n1 - 2], [0, 1]]])
    want, _ = oracle.evaluate_points(s.nodes, [q], pts)
    lin = pts[:, 0] * n1 + pts[:, 1]
    nib = (got[lin // 2] >> (4 * (lin % 2))) & 15
    assert np.array_equal(nib.astype(np.float64), want)
    del q, got


def test_largest_pipelined_loop():
    """The per-axis requantize of s8[32767, 65536] (2^31 - 65536 bytes in and
    out) on the pipelined loop: byte offsets reach their maximum, and the
    last of a thread's sixteen rows lies past the end for one row slot.
    Sampled outputs, bit-exact."""
    n0, n1 = 32767, 65536
    say("largest pipelined loop", n0, n1)
    g = W.rng(94)
    q = np.frombuffer(bytearray(g.bytes(n0 * n1)), np.int8)
    scales = W.uniform_f32(g, n1, 0.001, 0.05)
    zps = W.integers(g, n1, -20, 20, np.int64)
    bias = W.normal_f32(g, n1, 0.1)
    s = W.Spec()
    p = s.parameter(0, "s8", [n0, n1], quant=W.quant_type("s8", scales, zps, qdim=1))
    b = s.parameter(1, "f32", [n1])
    d = s.op("uniform_dequantize", [p], "f32", [n0, n1])
    y = s.binary("add", d, s.broadcast_in_dim(b, [1], "f32", [n0, n1]), "f32", [n0, n1])
    s.op("uniform_quantize", [y], "s8", [n0, n1], quant=W.quant_type("s8", [0.02], [0]))
    got, f = run_gpu(s.nodes, [q, bias])
    src = f.source()
    assert f.plan()["hero"] == "loop" and "#define HF_PIPE 0" not in src
    assert "#define HF_NR 16" in src
    pts = np.stack([g.integers(0, n0, 20000), g.integers(0, n1, 20000)], 1)
    pts = np.concatenate([pts, [[0, 0], [n0 - 1, n1 - 1], [n0 - 1, 0], [0, n1 - 1]]])
    want, _ = oracle.evaluate_points(s.nodes, [q, bias], pts)
    lin = pts[:, 0] * n1 + pts[:, 1]
    assert np.array_equal(got[lin].astype(np.float64), want)
    del q, got


# --------------------------------------------------------------------------
# index transforms: reverse, iota, pad, concatenate
# --------------------------------------------------------------------------
def test_index_transforms_small_bitexact():
    g = W.rng(81)
    cases = 0
    for shape in [(5, 7), (3, 1, 6), (2, 3, 4)]:
        r = len(shape)
        x = W.normal_f32(g, int(np.prod(shape)))
        for dims in [(r - 1,), (0,), tuple(range(r))]:
            s = W.Spec()
            p = s.parameter(0, "f32", list(shape))
            s.reverse(p, dims, "f32", list(shape))
            got, _ = run_gpu(s.nodes, [x])
            assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "f32")
            cases += 1
        for d in range(r):
            for dt in ("f32", "s32", "bf16"):
                s = W.Spec()
                s.iota(d, dt, list(shape))
                got, _ = run_gpu(s.nodes, [])
                assert_bitexact(got, oracle.evaluate(s.nodes, []), dt)
                cases += 1
            other = list(shape)
            other[d] = 3
            y = W.normal_f32(g, int(np.prod(other)))
            out = list(shape)
            out[d] = 2 * shape[d] + 3
            s = W.Spec()
            pa = s.parameter(0, "f32", list(shape))
            pb = s.parameter(1, "f32", other)
            s.concatenate([pa, pb, pa], d, "f32", out)
            got, _ = run_gpu(s.nodes, [x, y])
            assert_bitexact(got, oracle.evaluate(s.nodes, [x, y]), "f32")
            cases += 1
        for lo, hi, it in [([1] * r, [2] * r, [0] * r), ([-1] + [0] * (r - 1), [0] * (r - 1) + [-1], [1] * r),
                           ([2] * r, [-1] * r, [2] * r)]:
            out = [n + l + max(n - 1, 0) * i + h for n, l, h, i in zip(shape, lo, hi, it)]
            if min(out) < 1:
                continue
            s = W.Spec()
            p = s.parameter(0, "f32", list(shape))
            v = s.parameter(1, "f32", [])
            s.pad(p, v, lo, hi, it, "f32", out)
            pv = np.array(-3.25, np.float32)
            got, _ = run_gpu(s.nodes, [x, pv])
            assert_bitexact(got, oracle.evaluate(s.nodes, [x, pv]), "f32")
            cases += 1
    say("index-transform cases:", cases)


def test_index_transforms_composed():
    """pad (negative edge, interior), reverse along the minor dim, plus iota,
    then concatenated with a padded second input: every element is a data
    movement or one f32 add, so the result is bit-exact."""
    g = W.rng(82)
    n0, n1, m1 = 1000, 1500, 77
    x = W.normal_f32(g, n0 * n1)
    y = W.normal_f32(g, n0 * m1)
    o0, o1 = 2 + n0 + (n0 - 1) + 1, -1 + n1 + 3
    s = W.Spec()
    px = s.parameter(0, "f32", [n0, n1])
    py = s.parameter(1, "f32", [n0, m1])
    pv = s.constant(-1.0, "f32", [])
    p = s.pad(px, pv, [2, -1], [1, 3], [1, 0], "f32", [o0, o1])
    rv = s.reverse(p, [1], "f32", [o0, o1])
    io = s.iota(0, "f32", [o0, o1])
    a = s.binary("add", rv, io, "f32", [o0, o1])
    yy = s.pad(py, pv, [0, 0], [o0 - n0, 0], [0, 0], "f32", [o0, m1])
    s.concatenate([a, yy], 1, "f32", [o0, o1 + m1])
    got, f = run_gpu(s.nodes, [x, y])
    assert f.plan()["hero"] == "loop"
    assert_bitexact(got, oracle.evaluate(s.nodes, [x, y]), "f32")


def test_index_transforms_on_major_dims_vectorize():
    """pad, reverse and concatenate along the major dim leave the lane dim
    alone: the loop keeps 128-bit lanes, and a reverse inside a transpose's
    prologue keeps the transpose hero.  Bit-exact."""
    spec, params, _ = W.pad_reverse_concat_f32(300, 520, 77)
    got, f = run_gpu(spec.nodes, params)
    assert f.plan()["hero"] == "loop" and f.plan()["vector_elems"] == 4
    assert_bitexact(got, oracle.evaluate(spec.nodes, params), "f32")
    spec, params, _ = W.pad_reverse_concat_f32()
    got, f = run_gpu(spec.nodes, params)
    g = W.rng(83)
    pts = np.stack([g.integers(0, 6146, 20000), g.integers(0, 4096, 20000)], 1)
    pts = np.concatenate([pts, [[0, 0], [1, 5], [4096, 7], [4097, 4095], [4098, 0], [6145, 4095]]])
    want, _ = oracle.evaluate_points(spec.nodes, params, pts)
    assert_bitexact(got[pts[:, 0] * 4096 + pts[:, 1]], want.astype(np.float32), "f32")
    s = W.Spec()
    x = s.parameter(0, "f32", [1000, 1536])
    r = s.reverse(x, [0], "f32", [1000, 1536])
    s.transpose(r, [1, 0], "f32", [1536, 1000])
    xs = W.normal_f32(g, 1000 * 1536)
    got, f = run_gpu(s.nodes, [xs])
    assert f.plan()["hero"] == "transpose"
    assert_bitexact(got, oracle.evaluate(s.nodes, [xs]), "f32")


def test_pad_reverse_concat_minor_full():
    """pad, reverse and concatenate along the minor dim (one element a lane,
    eight rows a thread, loads guarded by the selects): small ragged shapes
    and the benchmark's f32[4096, 2040 + 8 + 2048], whole output bit-exact."""
    for dims in ((3, 5, 7), (37, 100, 64), (4096, 2040, 2048)):
        say("pad reverse concat minor", dims)
        spec, params, _ = W.pad_reverse_concat_minor_f32(*dims, seed=84 + dims[0] % 5)
        got, f = run_gpu(spec.nodes, params)
        assert f.plan()["hero"] == "loop"
        assert_bitexact(got, oracle.evaluate(spec.nodes, params), "f32")


# --------------------------------------------------------------------------
# elementwise epilogues after a reduce
# --------------------------------------------------------------------------
def test_reduce_epilogue_mean():
    """mean = reduce-sum / N: the division runs once per output, after the
    reduce (an elementwise epilogue)."""
    rows, n = 96, 3000
    g = W.rng(41)
    x = W.normal_f32(g, rows * n)
    s = W.Spec()
    p = s.parameter(0, "f32", [rows, n])
    r = s.reduce(p, [1], "add", 0.0, "f32", [rows])
    c = s.constant(float(n), "f32", [rows])
    s.binary("divide", r, c, "f32", [rows])
    got, f = run_gpu(s.nodes, [x])
    assert f.plan()["hero"] == "row_reduce"
    want = np.asarray(oracle.evaluate(s.nodes, [x]), np.float64)
    bound = 1e-5 * np.abs(x.reshape(rows, n)).astype(np.float64).sum(1) / n + np.spacing(np.abs(want).astype(np.float32))
    assert (np.abs(np.asarray(got, np.float64) - want) <= bound).all()


def test_row_mean_full():
    """The row mean of f32[16384, 4096] at full size, in the launch
    configuration the benchmark times: every row within the summation bound
    plus the division's rounding."""
    spec, params, _ = W.row_mean_f32()
    say("row mean full")
    got, f = run_gpu(spec.nodes, params, reps=2)
    assert f.plan()["hero"] == "row_reduce"
    x = params[0].reshape(16384, 4096)
    want = np.asarray(oracle.evaluate(spec.nodes, params), np.float64)
    bound = 1e-5 * np.abs(x).astype(np.float64).sum(1) / 4096 + np.spacing(np.abs(want).astype(np.float32))
    assert (np.abs(np.asarray(got, np.float64) - want) <= bound).all()


def test_reduce_epilogue_exact_cases():
    """Epilogues whose results are unique: a column max through the segment
    fold, then negate and convert to bf16; a max plus a per-output bias; an
    integer-valued sum then per-tensor quantize."""
    g = W.rng(42)
    # column max (segments + fold kernel), negate, convert to bf16
    r_, c_ = 4096, 96
    x = W.uniform_f32(g, r_ * c_, -100.0, 100.0)
    s = W.Spec()
    p = s.parameter(0, "f32", [r_, c_])
    m = s.reduce(p, [0], "max", float("-inf"), "f32", [c_])
    ng = s.unary("negate", m, "f32", [c_])
    s.convert(ng, "bf16", [c_])
    got, f = run_gpu(s.nodes, [x])
    assert f.plan()["hero"] == "column_reduce" and f.plan()["workspace_bytes"] > 0
    assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "bf16")
    # row max plus a bias parameter of the output's shape
    x = W.uniform_f32(g, 300 * 700, -100.0, 100.0)
    bias = W.normal_f32(g, 300)
    s = W.Spec()
    p = s.parameter(0, "f32", [300, 700])
    b = s.parameter(1, "f32", [300])
    m = s.reduce(p, [1], "max", float("-inf"), "f32", [300])
    s.binary("add", m, b, "f32", [300])
    got, _ = run_gpu(s.nodes, [x, bias])
    assert_bitexact(got, oracle.evaluate(s.nodes, [x, bias]), "f32")
    # integer-valued sum (exact in any order), then quantize to i8
    x = W.integers(g, 200 * 1000, -4, 4, np.int64).astype(np.float32)
    s = W.Spec()
    p = s.parameter(0, "f32", [200, 1000])
    r = s.reduce(p, [1], "add", 0.0, "f32", [200])
    s.op("uniform_quantize", [r], "s8", [200], quant=W.quant_type("s8", [0.5], [3]))
    got, _ = run_gpu(s.nodes, [x])
    assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "s8")


# --------------------------------------------------------------------------
# column reduce (max) and its column-major twin
# --------------------------------------------------------------------------
@pytest.mark.parametrize("r,c", [(100, 48), (1000, 4096), (7, 3), (513, 260), (16384, 40)])
def test_column_reduce_small(r, c):
    say("column reduce", r, c)
    spec, params, _ = W.column_reduce_max_f32(r, c, seed=50 + c)
    got, f = run_gpu(spec.nodes, params)
    assert f.plan()["hero"] in ("column_reduce", "row_reduce")
    assert_bitexact(got, oracle.evaluate(spec.nodes, params), "f32")


def test_column_reduce_full_both_layouts():
    spec, params, _ = W.column_reduce_max_f32()
    say("column reduce full")
    got, f = run_gpu(spec.nodes, params, reps=3)  # repeated launches, each with its own workspace
    assert f.plan()["hero"] == "column_reduce"
    want = params[0].reshape(16384, 4096).max(axis=0)
    assert_bitexact(got, want, "f32")
    assert_bitexact(got, oracle.evaluate(spec.nodes, params), "f32")
    spec_c, _, _ = W.column_reduce_max_f32(m2m=(0, 1))
    colmajor = np.ascontiguousarray(params[0].reshape(16384, 4096).T).ravel()
    got_c, fc = run_gpu(spec_c.nodes, [colmajor])
    assert fc.plan()["hero"] == "row_reduce"
    assert np.array_equal(got.view(np.uint32), got_c.view(np.uint32))
    assert_bitexact(got_c, oracle.evaluate(spec_c.nodes, [colmajor]), "f32")


@pytest.mark.parametrize("dims,red,m2m", [([3, 50, 40], [1], None), ([2, 3, 1000, 64], [2], None),
                                          ([5, 7, 9], [2], [0, 2, 1]), ([4, 6, 5, 32], [1, 2], None),
                                          ([8, 4096, 512], [1], None), ([3, 130, 7], [1], None)])
def test_column_reduce_batched(dims, red, m2m):
    """Reduced dims that form one physically contiguous block with kept dims
    on both sides: a column reduce over the kept dims flattened in physical
    order, the major kept dims acting as a batch.  Sum of integers (exact in
    any order) and max, bit-exact against the oracle."""
    say("column reduce batched", dims, red, m2m)
    g = W.rng(98)
    n = int(np.prod(dims))
    out = [d for k, d in enumerate(dims) if k not in red]
    for reducer, init in (("add", 0.0), ("max", float("-inf"))):
        s = W.Spec()
        p = s.parameter(0, "f32", dims, m2m)
        s.reduce(p, red, reducer, init, "f32", out)
        x = (W.integers(g, n, -8, 8, np.int64).astype(np.float32) if reducer == "add"
             else W.normal_f32(g, n))
        got, f = run_gpu(s.nodes, [x])
        assert f.plan()["hero"] == "column_reduce", f.plan()
        assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "f32")


@pytest.mark.parametrize("hero", ["row_reduce", "column_reduce"])
def test_reduce_special_values(hero):
    """max, min and add reductions over data with NaN, signed zeros and
    infinities, through the row hero (rows of 16384: two rows per step) and
    the column hero (many segments: the specials cross the fold kernel).
    IEEE maximum/minimum propagate NaN and order -0 < +0; +inf + -inf is NaN.
    Integer-valued data keeps the sums exact: bit-exact against the oracle."""
    g = W.rng(95)
    n_red, n_keep = 16384, 64
    x = W.integers(g, n_red * n_keep, -100, 100, np.int64).astype(np.float32).reshape(n_keep, n_red)
    nan, inf = np.float32("nan"), np.float32("inf")
    x[0, 777] = nan                      # one NaN in the middle
    x[1] = np.where(np.arange(n_red) % 2, -0.0, 0.0)
    x[2] = -0.0                          # all -0
    x[3] = -inf
    x[4, 5], x[4, 9000] = inf, -inf      # inf - inf
    x[5, -1] = nan                       # NaN last
    x[6] = nan
    x[7, 0] = nan                        # NaN first
    x[8, 123] = inf
    arr = x if hero == "row_reduce" else np.ascontiguousarray(x.T)   # [keep, red] or [red, keep]
    dims = list(arr.shape)
    rdim = 1 if hero == "row_reduce" else 0
    for red, init in (("max", -np.inf), ("min", np.inf), ("add", 0.0)):
        say("reduce specials", hero, red)
        s = W.Spec()
        p = s.parameter(0, "f32", dims)
        s.reduce(p, [rdim], red, float(init), "f32", [n_keep])
        got, f = run_gpu(s.nodes, [arr.ravel()])
        assert f.plan()["hero"] == hero
        assert_bitexact(got, oracle.evaluate(s.nodes, [arr.ravel()]), "f32")
        if red == "max":
            assert np.isnan(got[[0, 5, 6, 7]]).all() and got[8] == inf and got[3] == -inf
            assert got[1] == 0 and not np.signbit(got[1]) and np.signbit(got[2])
        if red == "add":
            assert np.isnan(got[4]) and got[8] == inf


# --------------------------------------------------------------------------
# launches recorded into a HIP graph
# --------------------------------------------------------------------------
def _concurrency_cases():
    makers = [lambda: W.transpose_exp_f32(512, 768, seed=71),
              lambda: W.row_reduce_exp_add_bf16(2, 16, 4096, seed=72),
              lambda: W.column_reduce_max_f32(2048, 1024, seed=73),
              lambda: W.quant_dequant_bias_requant(300, 4096, seed=74)]
    return [mk() for mk in makers]


def test_concurrent_launches_of_one_handle_from_threads_on_streams():
    """ONE handle per hero (a loop, a transpose, a row reduce and a column
    reduce whose launch needs a workspace), shared by four host threads, each
    with its own stream (default priority), its own result buffers and its own
    workspace, launching 20 rounds at once.  Every output equals the
    single-stream result bitwise, and the oracle where exact."""
    import threading
    import torch
    import compiler_hlo_amd as H
    from harness import from_device, to_device
    cases = _concurrency_cases()
    fs = [H.Fusion(spec.nodes) for spec, _, _ in cases]
    assert fs[2].plan()["hero"] == "column_reduce" and fs[2].workspace_bytes > 0
    ref = []
    for (spec, params, _), f in zip(cases, fs):
        got, _ = run_gpu(spec.nodes, params, fusion=f)
        ref.append(got)
    assert_bitexact(ref[2], oracle.evaluate(cases[2][0].nodes, cases[2][1]), "f32")
    assert_bitexact(ref[3], oracle.evaluate(cases[3][0].nodes, cases[3][1]), "s8")
    outs, errors = {}, []

    def worker(t):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                devs = [[to_device(p) for p in params] for _, params, _ in cases]
                wss = [torch.empty(max(1, f.workspace_bytes), dtype=torch.uint8, device="cuda") for f in fs]
                res = [f(*d, stream=stream, workspace=w) for f, d, w in zip(fs, devs, wss)]
                for _ in range(19):
                    for f, d, r, w in zip(fs, devs, res, wss):
                        f(*d, out=r, stream=stream, workspace=w)
            stream.synchronize()
            outs[t] = [from_device(r, spec.nodes[-1]["dtype"]) for r, (spec, _, _) in zip(res, cases)]
        except Exception as e:  # reported by the main thread
            errors.append((t, repr(e)))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not errors, errors
    assert sorted(outs) == [0, 1, 2, 3]
    for t in range(4):
        for k in range(4):
            assert np.array_equal(outs[t][k].view(np.uint8), ref[k].view(np.uint8)), (t, k)


def test_one_handle_on_four_streams_from_one_thread():
    """One column-reduce handle launched round-robin on four streams from one
    thread, so that its launches overlap on the device: each stream has its
    own input, result and workspace.  Every result equals the oracle's."""
    import torch
    import compiler_hlo_amd as H
    from harness import from_device, to_device
    seeds = [301, 302, 303, 304]
    specs = [W.column_reduce_max_f32(4096, 2048, seed=s) for s in seeds]
    f = H.Fusion(specs[0][0].nodes)
    assert f.plan()["hero"] == "column_reduce" and f.workspace_bytes > 0
    streams = [torch.cuda.Stream() for _ in seeds]
    ins, outs, wss = [], [], []
    for (spec, params, _), st in zip(specs, streams):
        with torch.cuda.stream(st):
            ins.append([to_device(p) for p in params])
            outs.append(torch.empty(2048, dtype=torch.float32, device="cuda"))
            wss.append(torch.empty(f.workspace_bytes, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    for _ in range(25):
        for st, i, o, w in zip(streams, ins, outs, wss):
            f(*i, out=o, stream=st, workspace=w)
    torch.cuda.synchronize()
    for (spec, params, _), o in zip(specs, outs):
        assert_bitexact(from_device(o, "f32"), oracle.evaluate(spec.nodes, params), "f32")


def test_destroy_right_after_an_async_launch():
    """Destroying a handle while its launch may still run waits for the
    device first: the output is complete and correct afterwards."""
    import torch
    import compiler_hlo_amd as H
    from harness import from_device, to_device
    spec, params, _ = W.column_reduce_max_f32(8192, 4096, seed=305)
    x = to_device(params[0])
    torch.cuda.synchronize()
    f = H.Fusion(spec.nodes)
    out = f(x)
    f.close()
    torch.cuda.synchronize()
    assert_bitexact(from_device(out, "f32"), oracle.evaluate(spec.nodes, params), "f32")
    out2 = H.Fusion(spec.nodes)(x)  # the temporary handle is destroyed at once
    torch.cuda.synchronize()
    assert np.array_equal(from_device(out2, "f32").view(np.uint32), from_device(out, "f32").view(np.uint32))


@pytest.mark.parametrize("k", range(3))
def test_launch_in_hip_graph(k):
    """A launch recorded into a HIP graph (torch.cuda.graph) and replayed with
    new inputs copied in, with an eager launch of the same handle between
    replays: every replay equals the eager result bitwise.  The column
    reduce's launch holds two kernels and a workspace."""
    import torch
    import compiler_hlo_amd as H
    make = [lambda seed: W.transpose_bf16_021(4, 64, 128, seed=seed),
            lambda seed: W.row_reduce_exp_add_bf16(2, 8, 4096, seed=seed),
            lambda seed: W.column_reduce_max_f32(4096, 512, seed=seed)][k]
    spec, p0, _ = make(90)
    say("graph", spec.nodes[-1]["op"], [nd["dims"] for nd in spec.nodes if nd["op"] == "parameter"])
    f = H.Fusion(spec.nodes)
    if k == 2:
        assert f.plan()["hero"] == "column_reduce" and f.plan()["workspace_bytes"] > 0
    static_in = [to_device(p) for p in p0]
    static_out = f(*static_in)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        f(*static_in, out=static_out)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        f(*static_in, out=static_out)
    dt = spec.nodes[-1]["dtype"]
    for seed in (91, 92, 93):
        _, pk, _ = make(seed)
        for t, p in zip(static_in, pk):
            t.copy_(to_device(p))
        static_out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        got = from_device(static_out, dt)
        want, _ = run_gpu(spec.nodes, pk, fusion=f)
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), seed
    del graph


# --------------------------------------------------------------------------
# special values and exhaustive bf16 exp
# --------------------------------------------------------------------------
def test_special_values_max_min_exp_log():
    vals = [float("nan"), -0.0, 0.0, float("-inf"), float("inf"), 1.5, -2.0, 1e-40]
    a = np.array([v for v in vals for _ in vals] * 2, np.float32)
    b = np.array([w for _ in vals for w in vals] * 2, np.float32)
    n = a.size
    for op in ("maximum", "minimum"):
        s = W.Spec()
        x = s.parameter(0, "f32", [n])
        y = s.parameter(1, "f32", [n])
        s.binary(op, x, y, "f32", [n])
        got, _ = run_gpu(s.nodes, [a, b])
        assert_bitexact(got, oracle.evaluate(s.nodes, [a, b]), "f32")
    x = np.array([1.0, 0.0, -0.0, -1.0, np.inf, np.nan, 1e-45, 3.4e38, -np.inf, 88.7, -103.0, 0.5] * 4,
                 np.float32)
    for op in ("log", "exponential"):
        s = W.Spec()
        p = s.parameter(0, "f32", [x.size])
        s.unary(op, p, "f32", [x.size])
        got, _ = run_gpu(s.nodes, [x])
        assert_ulp(got, oracle.evaluate(s.nodes, [x]), "f32", 2)


def test_exp_bf16_exhaustive():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    s = W.Spec()
    p = s.parameter(0, "bf16", [65536])
    s.unary("exponential", p, "bf16", [65536])
    got, _ = run_gpu(s.nodes, [allbits])
    d = assert_ulp(got, oracle.evaluate(s.nodes, [allbits]), "bf16", 1)
    off = int((d > 0).sum())
    say("bf16 exp: %d of 65536 inputs 1 ulp off" % off)
    # measured: 2 inputs; more would move the bf16 exp + bias row sums and the
    # bf16 exp fusions
    assert off <= 2, off


def test_tanh_bf16_exhaustive():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    s = W.Spec()
    p = s.parameter(0, "bf16", [65536])
    s.unary("tanh", p, "bf16", [65536])
    got, _ = run_gpu(s.nodes, [allbits])
    # correctly rounded on every input: the bit-exact GELU rests on it
    assert_bitexact(got, oracle.evaluate(s.nodes, [allbits]), "bf16")


@pytest.mark.parametrize("dt,op", [("bf16", "log"), ("f16", "exponential"), ("f16", "tanh"), ("f16", "log")])
def test_16_bit_transcendentals_exhaustive(dt, op):
    """Every 16-bit input of the 16-bit transcendentals not covered above:
    within one ulp of the oracle's correctly rounded value (the f32 result of
    the device function rounds once more to the 16-bit type), NaN where the
    oracle has NaN, and no more inputs one ulp off than measured."""
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    s = W.Spec()
    p = s.parameter(0, dt, [65536])
    s.unary(op, p, dt, [65536])
    got, _ = run_gpu(s.nodes, [allbits])
    d = assert_ulp(got, oracle.evaluate(s.nodes, [allbits]), dt, 1)
    off = int((d > 0).sum())
    say("%s %s: %d of 65536 inputs 1 ulp off" % (dt, op, off))
    # measured: bf16 log 0, f16 exp 2, f16 tanh 0 (correctly rounded), f16 log 4
    assert off <= {("bf16", "log"): 0, ("f16", "exponential"): 2, ("f16", "tanh"): 0, ("f16", "log"): 4}[dt, op]


def test_tanh_f32_sample():
    """f32 tanh (tanhf) on 2^20 inputs of every magnitude from 2^-12 to 8 and
    the special values: within 2 ulp of the oracle's correctly rounded value."""
    g = W.rng(44)
    x = (g.standard_normal(1 << 20) * np.exp2(g.integers(-12, 4, 1 << 20))).astype(np.float32)
    x[:8] = [0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, -20.0, 20.0]
    s = W.Spec()
    p = s.parameter(0, "f32", [x.size])
    s.unary("tanh", p, "f32", [x.size])
    got, _ = run_gpu(s.nodes, [x])
    d = assert_ulp(got, oracle.evaluate(s.nodes, [x]), "f32", 2)
    say("tanh ulp histogram", np.bincount(d.astype(np.int64)))


def test_exp_log_f32_sample():
    g = W.rng(43)
    for op, x in (("exponential", g.uniform(-103, 89, 1 << 20).astype(np.float32)),
                  ("log", np.exp2(g.uniform(-149, 128, 1 << 20)).astype(np.float32))):
        s = W.Spec()
        p = s.parameter(0, "f32", [x.size])
        s.unary(op, p, "f32", [x.size])
        got, _ = run_gpu(s.nodes, [x])
        d = assert_ulp(got, oracle.evaluate(s.nodes, [x]), "f32", 2)
        say(op, "ulp histogram", np.bincount(d.astype(np.int64)))


# --------------------------------------------------------------------------
# brute force over tiny shapes: transposes, broadcasts, layouts, reduces
# --------------------------------------------------------------------------
def _rand_perm_cases(seed, count):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(count):
        rank = int(rng.integers(2, 5))
        dims = [int(v) for v in rng.integers(1, 4, rank)]
        perm = [int(v) for v in rng.permutation(rank)]
        m_in = [int(v) for v in rng.permutation(rank)]
        m_out = [int(v) for v in rng.permutation(rank)]
        dt = ["f32", "bf16"][int(rng.integers(0, 2))]
        cases.append((dims, perm, m_in, m_out, dt))
    return cases


def test_brute_force_transpose_layouts():
    for dims, perm, m_in, m_out, dt in _rand_perm_cases(44, 60):
        n = int(np.prod(dims))
        x = (np.arange(n, dtype=np.uint32) * 2654435761 % 65521).astype(np.float32)
        if dt == "bf16":
            x = (x.view(np.uint32) >> 16).astype(np.uint16)
        s = W.Spec()
        p = s.parameter(0, dt, dims, m_in)
        s.transpose(p, perm, dt, [dims[q] for q in perm], m2m=m_out)
        got, _ = run_gpu(s.nodes, [x])
        assert_bitexact(got, oracle.evaluate(s.nodes, [x]), dt)


def test_brute_force_broadcast():
    rng = np.random.default_rng(45)
    for _ in range(40):
        rank = int(rng.integers(1, 4))
        out_dims = [int(v) for v in rng.integers(1, 5, rank)]
        k = int(rng.integers(0, rank + 1))
        bd = sorted(int(v) for v in rng.choice(rank, k, replace=False))
        if rng.integers(0, 2):
            bd = bd[::-1]
        od = [out_dims[d] if rng.integers(0, 3) else 1 for d in bd]
        x = rng.standard_normal(max(1, int(np.prod(od)))).astype(np.float32)[: int(np.prod(od))]
        m_out = [int(v) for v in rng.permutation(rank)]
        s = W.Spec()
        p = s.parameter(0, "f32", od)
        b = s.broadcast_in_dim(p, bd, "f32", out_dims)
        y = s.parameter(1, "f32", out_dims, m_out)
        s.binary("add", b, y, "f32", out_dims, m2m=m_out)
        yy = rng.standard_normal(int(np.prod(out_dims))).astype(np.float32)
        got, _ = run_gpu(s.nodes, [x, yy])
        assert_bitexact(got, oracle.evaluate(s.nodes, [x, yy]), "f32")


def test_brute_force_reduce():
    import compiler_hlo_amd as H
    rng = np.random.default_rng(46)
    done = 0
    for _ in range(50):
        rank = int(rng.integers(1, 4))
        dims = [int(v) for v in rng.integers(1, 6, rank)]
        k = int(rng.integers(1, rank + 1))
        red = sorted(int(v) for v in rng.choice(rank, k, replace=False))
        m2m = [int(v) for v in rng.permutation(rank)]
        op = ["add", "max", "min"][int(rng.integers(0, 3))]
        init = {"add": 0.0, "max": float("-inf"), "min": float("inf")}[op]
        x = rng.integers(-8, 9, int(np.prod(dims))).astype(np.float32)
        s = W.Spec()
        p = s.parameter(0, "f32", dims, m2m)
        s.reduce(p, red, op, init, "f32", [dims[d] for d in range(rank) if d not in red])
        try:
            got, _ = run_gpu(s.nodes, [x])
        except H.FusionError as e:
            assert e.status == "HF_ERR_UNSUPPORTED", str(e)
            continue
        assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "f32")
        done += 1
    assert done >= 30


def test_reshape_bitcast_and_general():
    g = W.rng(47)
    x = g.standard_normal(24 * 16).astype(np.float32)
    for out_dims in ([24, 16], [4, 6, 16], [1, 384], [6, 64], [16, 24]):
        s = W.Spec()
        p = s.parameter(0, "f32", [24, 16])
        e = s.unary("exponential", p, "f32", [24, 16])
        s.reshape(e, "f32", out_dims)
        got, _ = run_gpu(s.nodes, [x])
        assert_ulp(got, oracle.evaluate(s.nodes, [x]), "f32", 2)


# --------------------------------------------------------------------------
# GELU (bf16, tanh form)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [(2, 8, 64), (6, 512, 4096)])
def test_gelu_bf16(shape):
    say("gelu", shape)
    spec, params, _ = W.gelu_bf16(*shape)
    got, f = run_gpu(spec.nodes, params)
    assert f.plan()["hero"] == "loop"
    # bit-exact: a product of two bf16 values is exact in f32, a sum of two
    # bf16 values rounded to f32 and then to bf16 is the single bf16 rounding,
    # and the bf16 tanh is correctly rounded on every input (exhaustive test)
    assert_bitexact(got, oracle.evaluate(spec.nodes, params), "bf16")


# --------------------------------------------------------------------------
# launch-time argument checks (host side, before any kernel runs)
# --------------------------------------------------------------------------
def test_launch_argument_errors():
    import torch
    import compiler_hlo_amd as H
    spec, params, _ = W.transpose_exp_f32(64, 64)
    f = H.Fusion(spec.nodes)
    x = to_device(params[0])
    out = torch.empty(64 * 64, dtype=torch.float32, device="cuda")
    with pytest.raises(H.FusionError) as e:
        f.launch_ptrs([], out.data_ptr())
    assert e.value.status == "HF_ERR_INVALID"
    with pytest.raises(H.FusionError) as e:
        f.launch_ptrs([x.data_ptr() + 4], out.data_ptr())
    assert e.value.status == "HF_ERR_INVALID"
    with pytest.raises(H.FusionError) as e:
        f.launch_ptrs([x.data_ptr()], x.data_ptr())
    assert e.value.status == "HF_ERR_INVALID" and "overlaps" in e.value.message
    # a plan that needs a workspace: missing, misaligned or overlapping
    cspec, cparams, _ = W.column_reduce_max_f32(4096, 512, seed=7)
    cf = H.Fusion(cspec.nodes)
    nws = cf.workspace_bytes
    assert nws > 0
    cx = to_device(cparams[0])
    cout = torch.empty(512, dtype=torch.float32, device="cuda")
    ws = torch.empty(nws + 64, dtype=torch.uint8, device="cuda")
    with pytest.raises(H.FusionError) as e:
        cf.launch_ptrs([cx.data_ptr()], cout.data_ptr(), 0, 0)
    assert e.value.status == "HF_ERR_INVALID" and "workspace" in e.value.message
    with pytest.raises(H.FusionError) as e:
        cf.launch_ptrs([cx.data_ptr()], cout.data_ptr(), 0, ws.data_ptr() + 4)
    assert e.value.status == "HF_ERR_INVALID" and "workspace" in e.value.message
    with pytest.raises(H.FusionError) as e:
        cf.launch_ptrs([cx.data_ptr()], cout.data_ptr(), 0, cx.data_ptr())
    assert e.value.status == "HF_ERR_INVALID" and "overlaps" in e.value.message
    with pytest.raises(ValueError):
        cf(cx, workspace=torch.empty(nws - 16, dtype=torch.uint8, device="cuda"))
    cf.launch_ptrs([cx.data_ptr()], cout.data_ptr(), torch.cuda.current_stream().cuda_stream, ws.data_ptr())
    torch.cuda.synchronize()
    assert_bitexact(from_device(cout, "f32"), oracle.evaluate(cspec.nodes, cparams), "f32")
    # pinned host memory is not device memory (the GPU could read it, so the
    # launch would not fault even if it were let through)
    h = torch.empty(64 * 64, dtype=torch.float32).pin_memory()
    with pytest.raises(H.FusionError) as e:
        f.launch_ptrs([h.data_ptr()], out.data_ptr())
    assert e.value.status == "HF_ERR_INVALID" and "device memory" in e.value.message
    # the binding checks tensors before anything reaches the library
    with pytest.raises(ValueError):
        f(x.cpu())
    with pytest.raises(ValueError):
        f(x, out=torch.empty(100, dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        f(x, out=torch.empty(64 * 64, dtype=torch.int32, device="cuda"))
    f(x, out=out)
    torch.cuda.synchronize()
    assert from_device(out, "f32").size == 4096
