"""Host-side tests of the C-ABI library (no GPU): exports, layout mapper,
descriptor validation, planning decisions, code generation and compilation
for gfx950, and the arithmetic claims the kernels rely on."""
import itertools
import os
import re
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import compiler_hlo_amd as H
import oracle
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def plan_of(spec):
    return H.Fusion(spec.nodes, mode="plan").plan()


# --------------------------------------------------------------------------
# exports
# --------------------------------------------------------------------------
def test_exports_every_declared_function():
    text = open(os.path.join(ROOT, "include", "hlofusion.h")).read()
    declared = set(re.findall(r"\b(hf_[a-z_]+)\s*\(", text))
    declared = {d for d in declared if not d.startswith("hf_fusion_desc")}
    assert {"hf_fusion_create", "hf_fusion_launch", "hf_fusion_destroy"} <= declared
    lib = H.library()
    for name in sorted(declared):
        assert hasattr(lib, name), name
    assert lib.hf_abi_version() == H.ABI_VERSION == 4


C_CLIENT = r"""
#include "hlofusion.h"
#include <stdio.h>
#include <string.h>

static hf_type f32_2d(int64_t r, int64_t c) {
  hf_type t;
  memset(&t, 0, sizeof t);
  t.dtype = HF_F32;
  t.rank = 2;
  t.dims[0] = r;
  t.dims[1] = c;
  return t;
}

int main(void) {
  hf_node n[3];
  hf_fusion_desc d;
  hf_fusion *f = NULL;
  hf_plan_info info;
  hf_status st;
  memset(n, 0, sizeof n);
  n[0].op = HF_PARAMETER;
  n[0].type = f32_2d(4096, 4096);
  n[0].parameter_number = 0;
  n[1].op = HF_EXP;
  n[1].n_operands = 1;
  n[1].operands[0] = 0;
  n[1].type = f32_2d(4096, 4096);
  n[2].op = HF_TRANSPOSE;
  n[2].n_operands = 1;
  n[2].operands[0] = 1;
  n[2].type = f32_2d(4096, 4096);
  n[2].n_attr = 2;
  n[2].attr[0] = 1;
  n[2].attr[1] = 0;
  d.abi_version = HF_ABI_VERSION;
  d.n_nodes = 3;
  d.nodes = n;
  d.root = 2;
  d.n_params = 1;
  st = hf_fusion_create(&d, HF_CREATE_PLAN_ONLY, &f);
  if (st != HF_OK) {
    printf("create failed: %s\n", hf_last_error());
    return 1;
  }
  if (hf_fusion_plan(f, &info) != HF_OK) return 2;
  printf("hero %d bytes %lld\n", (int)info.hero, (long long)info.algorithmic_bytes);
  hf_fusion_destroy(f);
  n[2].attr[1] = 1; /* not a permutation */
  f = NULL;
  st = hf_fusion_create(&d, HF_CREATE_PLAN_ONLY, &f);
  printf("invalid %d %s null %d\n", (int)st, hf_last_error(), f == NULL);
  printf("abi %d\n", (int)hf_abi_version());
  return 0;
}
"""


def test_header_is_c99_and_plans_from_c(tmp_path):
    """include/hlofusion.h compiles as strict C99 with every warning an error,
    and a C program plans a fusion and sees a validation error through it."""
    src = tmp_path / "client.c"
    src.write_text(C_CLIENT)
    exe = tmp_path / "client"
    libdir = os.path.join(ROOT, "compiler_hlo_amd")
    subprocess.check_call(["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
                           "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                           "-L", libdir, "-lhlofusion", "-Wl,-rpath," + libdir])
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    lines = out.stdout.splitlines()
    assert lines[0] == "hero 1 bytes 134217728"
    assert lines[1].startswith("invalid 1 ") and "permutation" in lines[1] and lines[1].endswith("null 1")
    assert lines[2] == "abi 4"


def test_missing_library_fails_loudly(tmp_path):
    """Without libhlofusion.so the package refuses to import: no fallback."""
    pkg = tmp_path / "compiler_hlo_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "compiler_hlo_amd", "__init__.py"), pkg / "__init__.py")
    r = subprocess.run(["python", "-c", "import compiler_hlo_amd"], cwd=tmp_path,
                       capture_output=True, text=True)
    assert r.returncode != 0 and "libhlofusion.so is missing" in r.stderr


# --------------------------------------------------------------------------
# layout mapper (Shapes and layout, "Array indexing")
# --------------------------------------------------------------------------
def test_linear_index_matches_oracle_all_small_shapes():
    for rank in range(1, 5):
        for dims in itertools.product([1, 2, 3], repeat=rank):
            idx = list(itertools.product(*[range(d) for d in dims]))
            for m2m in itertools.permutations(range(rank)):
                got = [H.linear_index(list(dims), list(m2m), list(i)) for i in idx]
                want = oracle.linear_indices(list(dims), list(m2m), np.array(idx)).tolist()
                assert got == want


def test_linear_index_rejects_bad_input():
    assert H.linear_index([2, 3], [0, 0], [0, 0]) == -1
    assert H.linear_index([2, 3], [1, 0], [2, 0]) == -1


# --------------------------------------------------------------------------
# validation: each broken constraint gives HF_ERR_INVALID with the node named
# --------------------------------------------------------------------------
def _status(nodes, **kw):
    try:
        H.Fusion(nodes, mode="plan", **kw)
    except H.FusionError as e:
        return e.status, e.message
    return "HF_OK", ""


def test_validation_errors():
    s = W.Spec()
    p = s.parameter(0, "f32", [2, 3])
    s.transpose(p, [0, 0], "f32", [2, 3])
    st, msg = _status(s.nodes)
    assert st == "HF_ERR_INVALID" and "node 1 (transpose)" in msg and "permutation" in msg

    s = W.Spec()
    p = s.parameter(0, "f32", [2, 3], m2m=[0, 0])
    st, msg = _status(s.nodes)
    assert st == "HF_ERR_INVALID" and "minor_to_major" in msg

    s = W.Spec()
    a = s.parameter(0, "f32", [2, 3])
    b = s.parameter(1, "f32", [3, 2])
    s.binary("add", a, b, "f32", [2, 3])
    assert _status(s.nodes)[0] == "HF_ERR_INVALID"

    s = W.Spec()
    a = s.parameter(0, "f32", [3])
    s.broadcast_in_dim(a, [1], "f32", [3, 4])
    st, msg = _status(s.nodes)
    assert st == "HF_ERR_INVALID" and "(C5)" in msg

    s = W.Spec()
    a = s.parameter(0, "f32", [3])
    s.broadcast_in_dim(a, [0, 1], "f32", [3, 3])
    assert "(C2)" in _status(s.nodes)[1]

    s = W.Spec()
    a = s.parameter(0, "f32", [4, 5])
    s.reduce(a, [1, 1], "add", 0.0, "f32", [4])
    assert "(C5)" in _status(s.nodes)[1]

    s = W.Spec()
    a = s.parameter(0, "f32", [4, 5])
    s.reduce(a, [1], "add", 0.0, "f32", [5])
    assert "(C7)" in _status(s.nodes)[1]

    # quantization constraints
    s = W.Spec()
    s.parameter(0, "s8", [4, 3], quant=W.quant_type("s8", [0.1, -0.2, 0.3], [0, 0, 0], qdim=1))
    assert "(C6)" in _status(s.nodes)[1]
    s = W.Spec()
    s.parameter(0, "s8", [4, 3], quant=W.quant_type("s8", [0.1, 0.2], [0, 0], qdim=1))
    assert "(C13)" in _status(s.nodes)[1]
    s = W.Spec()
    s.parameter(0, "s8", [4, 3], quant=W.quant_type("s8", [0.1], [300]))
    assert "(C8)" in _status(s.nodes)[1]
    s = W.Spec()
    s.parameter(0, "s8", [4, 3], quant=W.quant_type("s8", [float("inf")], [0]))
    assert "(C7)" in _status(s.nodes)[1]

    # parameter numbering and operand order
    s = W.Spec()
    s.parameter(0, "f32", [2])
    s.parameter(0, "f32", [2])
    assert _status(s.nodes, n_params=1)[0] == "HF_ERR_INVALID"
    nodes = [{"op": "log", "operands": [1], "dtype": "f32", "dims": [2]},
             {"op": "parameter", "param": 0, "dtype": "f32", "dims": [2]}]
    assert _status(nodes, root=0)[0] == "HF_ERR_INVALID"


def test_unsupported_is_distinguished():
    # only elementwise ops may follow the reduce hero
    s = W.Spec()
    p = s.parameter(0, "f32", [4, 5])
    r = s.reduce(p, [1], "add", 0.0, "f32", [4])
    s.broadcast_in_dim(r, [0], "f32", [4, 3])
    st, msg = _status(s.nodes)
    assert st == "HF_ERR_UNSUPPORTED" and "only elementwise ops may follow the reduce" in msg
    # one reduce per fusion
    s = W.Spec()
    p = s.parameter(0, "f32", [4, 5])
    r = s.reduce(p, [1], "add", 0.0, "f32", [4])
    r2 = s.reduce(p, [1], "max", float("-inf"), "f32", [4])
    s.binary("add", r, r2, "f32", [4])
    st, msg = _status(s.nodes)
    assert st == "HF_ERR_UNSUPPORTED" and "at most one reduce" in msg


def test_quantized_elementwise_validation_and_expansion():
    qa, qb = W.quant_type("s8", [0.5], [1]), W.quant_type("s8", [0.25], [0])
    # per-tensor quantized add: dequantize both, add in f32, quantize
    s = W.Spec()
    a = s.parameter(0, "s8", [16, 64], quant=qa)
    b = s.parameter(1, "s8", [16, 64], quant=qb)
    s.op("add", [a, b], "s8", [16, 64], quant=W.quant_type("s8", [0.3], [-2]))
    assert _status(s.nodes) == ("HF_OK", "")
    assert plan_of(s)["hero"] == "loop"
    # quantized and non-quantized operands mixed
    s = W.Spec()
    a = s.parameter(0, "s8", [16], quant=qa)
    b = s.parameter(1, "f32", [16])
    s.op("add", [a, b], "s8", [16], quant=qa)
    st, msg = _status(s.nodes)
    assert st == "HF_ERR_INVALID" and "baseline" in msg
    # per-axis operands are not allowed for the elementwise ops
    s = W.Spec()
    a = s.parameter(0, "s8", [2, 3], quant=W.quant_type("s8", [0.1, 0.2, 0.3], [0, 0, 0], qdim=1))
    s.op("negate", [a], "s8", [2, 3], quant=W.quant_type("s8", [0.1, 0.2, 0.3], [0, 0, 0], qdim=1))
    st, msg = _status(s.nodes)
    assert st == "HF_ERR_INVALID" and "per-tensor" in msg
    # storage ranges differ
    s = W.Spec()
    a = s.parameter(0, "s8", [16], quant=qa)
    s.op("abs", [a], "s8", [16], quant=W.quant_type("s8", [0.5], [1], storage_min=-100, storage_max=100))
    st, msg = _status(s.nodes)
    assert st == "HF_ERR_INVALID" and "storage" in msg


def test_four_bit_types_validation_and_plans():
    """si4/ui4: default storage ranges [-8, 7] and [0, 15]; byte counts pack
    two elements per byte; a 4-bit result is written by the loop hero only,
    with an even run per lane along an even physically minor dim."""
    q = W.quant_type("s4", [0.05], [1])
    s = W.Spec()
    p = s.parameter(0, "f32", [100, 64])
    s.op("uniform_quantize", [p], "s4", [100, 64], quant=q)
    pl = plan_of(s)
    assert pl["hero"] == "loop" and pl["vector_elems"] % 2 == 0
    assert pl["algorithmic_bytes"] == 100 * 64 * 4 + 100 * 64 // 2
    # an odd minor dim, a reduce result and an iota cannot be 4-bit
    s = W.Spec()
    p = s.parameter(0, "f32", [100, 63])
    s.op("uniform_quantize", [p], "s4", [100, 63], quant=q)
    st, msg = _status(s.nodes)
    assert st == "HF_ERR_UNSUPPORTED" and "even" in msg
    s = W.Spec()
    p = s.parameter(0, "f32", [64, 64])
    r = s.reduce(p, [1], "add", 0.0, "f32", [64])
    s.op("uniform_quantize", [r], "s4", [64], quant=q)
    st, msg = _status(s.nodes)
    assert st == "HF_ERR_UNSUPPORTED" and "4-bit" in msg
    s = W.Spec()
    s.iota(0, "u4", [16])
    assert _status(s.nodes)[0] == "HF_ERR_UNSUPPORTED"
    # storage range and zero points inside [-8, 7] / [0, 15]
    for dt, zp, lo, hi, ok in (("s4", -8, None, None, True), ("s4", 8, None, None, False),
                               ("u4", 15, None, None, True), ("u4", -1, None, None, False),
                               ("s4", 0, -9, 7, False), ("u4", 0, 0, 16, False), ("s4", 2, -2, 5, True)):
        s = W.Spec()
        p = s.parameter(0, dt, [8, 32], quant=W.quant_type(dt, [0.5], [zp], storage_min=lo, storage_max=hi))
        s.op("uniform_dequantize", [p], "f32", [8, 32])
        assert (_status(s.nodes)[0] == "HF_OK") == ok, (dt, zp, lo, hi)
    # 4-bit inputs are read by every hero; a transpose into 4-bit takes the loop
    s = W.Spec()
    p = s.parameter(0, "u4", [64, 4096], quant=W.quant_type("u4", [0.5], [8]))
    d = s.op("uniform_dequantize", [p], "f32", [64, 4096])
    s.reduce(d, [1], "add", 0.0, "f32", [64])
    assert plan_of(s)["hero"] == "row_reduce"
    s = W.Spec()
    p = s.parameter(0, "s4", [256, 512], quant=q)
    d = s.op("uniform_dequantize", [p], "f32", [256, 512])
    s.transpose(d, [1, 0], "f32", [512, 256])
    assert plan_of(s)["hero"] == "transpose"
    s = W.Spec()
    p = s.parameter(0, "f32", [256, 512])
    t = s.transpose(p, [1, 0], "f32", [512, 256])
    s.op("uniform_quantize", [t], "s4", [512, 256], quant=q)
    assert plan_of(s)["hero"] == "loop"


def test_argmax_validation():
    s = W.Spec()
    p = s.parameter(0, "f32", [8, 9])
    s.argmax(p, 1, [8, 9])
    assert _status(s.nodes) == ("HF_OK", "")
    # indices that are not an iota along the reduced dim
    s = W.Spec()
    p = s.parameter(0, "f32", [8, 9])
    k = s.parameter(1, "s32", [8, 9])
    s.op("reduce", [p, k], "s32", [8], dimensions=[1], reducer="argmax", init=float("-inf"), index_init=-1)
    st, msg = _status(s.nodes)
    assert st == "HF_ERR_UNSUPPORTED" and "iota" in msg
    s = W.Spec()
    p = s.parameter(0, "f32", [8, 9])
    k = s.iota(0, "s32", [8, 9])
    s.op("reduce", [p, k], "s32", [8], dimensions=[1], reducer="argmax", init=float("-inf"), index_init=-1)
    assert _status(s.nodes)[0] == "HF_ERR_UNSUPPORTED"
    # the result must be s32
    s = W.Spec()
    p = s.parameter(0, "f32", [8, 9])
    k = s.iota(1, "s32", [8, 9])
    s.op("reduce", [p, k], "f32", [8], dimensions=[1], reducer="argmax", init=float("-inf"), index_init=-1)
    st, msg = _status(s.nodes)
    assert st == "HF_ERR_INVALID" and "s32" in msg


def test_size_limit():
    ok = W.Spec()
    p = ok.parameter(0, "f32", [8191, 65536])
    ok.unary("exponential", p, "f32", [8191, 65536])
    assert _status(ok.nodes) == ("HF_OK", "")
    big = W.Spec()
    p = big.parameter(0, "f32", [8192, 65536])
    big.unary("exponential", p, "f32", [8192, 65536])
    st, msg = _status(big.nodes)
    assert st == "HF_ERR_UNSUPPORTED" and "2 GiB" in msg and "node 0" in msg
    # the byte limit holds for the arrays in memory only: an f32 value of
    # 2 GiB or more between a bf16 parameter and a bf16 result is fine
    mid = W.Spec()
    p = mid.parameter(0, "bf16", [8192, 65536])
    c = mid.convert(p, "f32", [8192, 65536])
    mid.convert(mid.unary("exponential", c, "f32", [8192, 65536]), "bf16", [8192, 65536])
    assert _status(mid.nodes) == ("HF_OK", "")
    big_param = W.Spec()
    p = big_param.parameter(0, "f32", [8192, 65536])
    big_param.convert(p, "bf16", [8192, 65536])
    st, msg = _status(big_param.nodes)
    assert st == "HF_ERR_UNSUPPORTED" and "2 GiB" in msg and "node 0" in msg
    big_root = W.Spec()
    p = big_root.parameter(0, "bf16", [8192, 65536])
    big_root.convert(p, "f32", [8192, 65536])
    st, msg = _status(big_root.nodes)
    assert st == "HF_ERR_UNSUPPORTED" and "2 GiB" in msg and "node 1" in msg
    # the element limit holds for every value
    for n0, ok_want in ((32767, True), (32768, False)):
        q = W.Spec()
        p = q.parameter(0, "s4", [n0, 65536], quant=W.quant_type("s4", [0.25], [-1]))
        d = q.op("uniform_dequantize", [p], "f32", [n0, 65536])
        q.op("uniform_quantize", [d], "u4", [n0, 65536], quant=W.quant_type("u4", [0.5], [7]))
        st, msg = _status(q.nodes)
        assert (st == "HF_OK") == ok_want and (ok_want or "2^31 elements" in msg), (n0, st, msg)


def test_index_transform_validation():
    def st(build):
        s = W.Spec()
        build(s)
        return _status(s.nodes)
    def rev(s):
        p = s.parameter(0, "f32", [3, 4])
        s.reverse(p, [1, 1], "f32", [3, 4])
    assert st(rev)[0] == "HF_ERR_INVALID" and "is_unique" in st(rev)[1]
    def iota(s):
        s.iota(2, "f32", [3, 4])
    assert st(iota)[0] == "HF_ERR_INVALID" and "iota_dimension" in st(iota)[1]
    def pad_shape(s):
        p = s.parameter(0, "f32", [2, 3])
        v = s.constant(0.0, "f32", [])
        s.pad(p, v, [0, 1], [2, 1], [1, 2], "f32", [5, 8])
    assert st(pad_shape)[0] == "HF_ERR_INVALID" and "(C4)" in st(pad_shape)[1]
    def pad_interior(s):
        p = s.parameter(0, "f32", [2, 3])
        v = s.constant(0.0, "f32", [])
        s.pad(p, v, [0, 0], [0, 0], [-1, 0], "f32", [1, 3])
    assert st(pad_interior)[0] == "HF_ERR_INVALID" and "(C3)" in st(pad_interior)[1]
    def pad_value_rank(s):
        p = s.parameter(0, "f32", [2, 3])
        v = s.parameter(1, "f32", [1])
        s.pad(p, v, [0, 0], [0, 0], [0, 0], "f32", [2, 3])
    assert st(pad_value_rank)[0] == "HF_ERR_INVALID" and "0-dimensional" in st(pad_value_rank)[1]
    def cat(s):
        a = s.parameter(0, "f32", [3, 2])
        b = s.parameter(1, "f32", [2, 3])
        s.concatenate([a, b], 0, "f32", [5, 2])
    assert st(cat)[0] == "HF_ERR_INVALID" and "(C2)" in st(cat)[1]
    def ok(s):
        a = s.parameter(0, "f32", [3, 2])
        b = s.parameter(1, "f32", [1, 2])
        c = s.concatenate([a, b, a], 0, "f32", [7, 2])
        r = s.reverse(c, [0], "f32", [7, 2])
        v = s.constant(0.5, "f32", [])
        s.pad(r, v, [1, -1], [0, 2], [0, 1], "f32", [8, 4])
    assert st(ok) == ("HF_OK", "")


def test_slice_validation():
    """slice (start/limit/strides) and dynamic_slice (StableHLO Specification,
    "dynamic_slice", C1-C5) constraints; integer constants only as start
    indices."""
    def st(build):
        s = W.Spec()
        build(s)
        return _status(s.nodes)
    def sl(start, limit, strides, out):
        def b(s):
            p = s.parameter(0, "f32", [6, 8])
            s.slice(p, start, limit, strides, "f32", out)
        return st(b)
    assert sl([1, 2], [5, 8], [1, 3], [4, 2]) == ("HF_OK", "")
    assert sl([0, 0], [6, 8], [4, 5], [2, 2]) == ("HF_OK", "")
    assert sl([3, 0], [2, 8], [1, 1], [0, 8])[0] == "HF_ERR_INVALID"          # start > limit
    assert sl([0, 0], [7, 8], [1, 1], [7, 8])[0] == "HF_ERR_INVALID"          # limit > dim
    assert sl([0, 0], [6, 8], [0, 1], [6, 8])[0] == "HF_ERR_INVALID"          # stride 0
    assert "ceil" in sl([0, 0], [6, 8], [4, 3], [2, 2])[1]                    # 8/3 -> 3 columns
    def ds(sizes, out, start_dtypes=("s32", "s32"), nstarts=2, const=False):
        def b(s):
            p = s.parameter(0, "f32", [6, 8])
            if const:
                starts = [s.constant(1, start_dtypes[k], []) for k in range(nstarts)]
            else:
                starts = [s.parameter(1 + k, start_dtypes[k], []) for k in range(nstarts)]
            s.dynamic_slice(p, starts, sizes, "f32")
            s.nodes[-1]["dims"] = list(out)
        return st(b)
    assert ds([2, 3], [2, 3]) == ("HF_OK", "")
    assert ds([2, 3], [2, 3], ("u8", "u8")) == ("HF_OK", "")
    assert ds([2, 3], [2, 3], const=True) == ("HF_OK", "")
    assert "(C2)" in ds([2, 3], [2, 3], nstarts=1)[1]
    assert "(C3)" in ds([2, 3], [2, 3], ("s32", "s8"))[1]
    assert "(C4)" in ds([7, 3], [7, 3])[1]
    assert "(C5)" in ds([2, 3], [3, 2])[1]
    assert "(I2)" in ds([2, 3], [2, 3], ("f32", "f32"))[1]
    def int_const_elsewhere(s):
        p = s.parameter(0, "f32", [4])
        c = s.constant(2, "s32", [4])
        s.binary("add", p, p, "f32", [4])
        s.nodes.append(s.nodes[c])
    assert st(int_const_elsewhere)[0] == "HF_ERR_UNSUPPORTED"
    def computed_start(s):
        p = s.parameter(0, "f32", [6, 8])
        a = s.parameter(1, "s32", [])
        b = s.convert(s.parameter(2, "f32", []), "f32", [])
        s.dynamic_slice(p, [a, a], [2, 2], "f32")
        s.nodes[-1]["operands"][2] = b
    assert st(computed_start)[0] == "HF_ERR_INVALID"


def test_loop_pipeline_choice():
    """The loop's software pipeline goes to single-partition fusions of 8-bit
    streams with 16 elements a lane: the per-axis requantize (six rows in
    flight, sixteen rows a thread, 256 workgroups) and the quantized add (four
    in flight); GELU, the si4 requantize and log(x) + transpose(log(x)) keep
    the plain loop.  In the pipelined source the column data load into their
    own struct (hf_I_), pinned after the first row, and the compute takes
    it."""
    def macros(spec):
        src = H.Fusion(spec.nodes, mode="compile").source()
        return {k: int(v) for k, v in re.findall(r"#define (HF_PIPE|HF_NR|HF_RSTEP) (\d+)", src)}, src
    m, src = macros(W.quant_dequant_bias_requant()[0])
    assert (m["HF_PIPE"], m["HF_NR"], m["HF_RSTEP"]) == (6, 16, 256)
    assert plan_of(W.quant_dequant_bias_requant()[0])["grid_blocks"] == 256
    assert "struct hf_I_" in src and "hf_loop_inv_pin(I)" in src and 'asm volatile("" : "+v"' in src
    m, _ = macros(W.quantized_add_i8()[0])
    assert (m["HF_PIPE"], m["HF_NR"]) == (4, 16)
    for mk in (W.gelu_bf16, W.quant_dequant_bias_requant_s4, W.loop_log_transpose_add):
        m, src = macros(mk()[0])
        assert m["HF_PIPE"] == 0 and "struct hf_I_" not in src, mk.__name__
    # a row count that leaves some threads one row short: 16 rows at most
    m, _ = macros(W.quant_dequant_bias_requant(4091, 4096)[0])
    assert (m["HF_NR"], m["HF_RSTEP"]) == (16, 256) and 15 * 256 < 4091


def test_loop_rows_per_thread_choice():
    """A loop that holds small arrays in registers over its rows: four rows a
    thread for per-axis quantization data (the s4 requantize: 4096
    workgroups), two for a broadcast f32 bias and one for a bf16 one, which
    leaves x + bias with the grid of the plain elementwise loop (f32: half
    of it)."""
    def bias(dt, bdim):
        s = W.Spec()
        x = s.parameter(0, dt, [4096, 4096])
        b = s.parameter(1, dt, [4096])
        s.binary("add", x, s.broadcast_in_dim(b, [bdim], dt, [4096, 4096]), dt, [4096, 4096])
        return s

    def neg(dt):
        s = W.Spec()
        s.unary("negate", s.parameter(0, dt, [4096, 4096]), dt, [4096, 4096])
        return s
    assert plan_of(neg("f32"))["grid_blocks"] == 16384 and plan_of(neg("bf16"))["grid_blocks"] == 8192
    for bdim in (0, 1):
        assert plan_of(bias("f32", bdim))["grid_blocks"] == 8192
        assert plan_of(bias("bf16", bdim))["grid_blocks"] == 8192
    assert plan_of(W.quant_dequant_bias_requant_s4()[0])["grid_blocks"] == 4096
    # rows of 2 MiB or more: whole-workgroup row segments (256 lanes)
    for dt, rows, cols, lanes in (("f32", 16, 1 << 20, 256), ("f32", 64, 1 << 18, 64),
                                  ("bf16", 16, 1 << 20, 256), ("bf16", 32, 1 << 19, 64)):
        s = W.Spec()
        s.unary("negate", s.parameter(0, dt, [rows, cols]), dt, [rows, cols])
        assert "#define HF_TPR %d\n" % lanes in H.Fusion(s.nodes, mode="compile").source()


def test_lane_moving_maps_keep_vector_lanes_and_guard_their_loads():
    """concatenate(pad(x), reverse(y)) along the minor dim of f32[4096,4096]:
    the index maps move with the lane, yet the loop keeps 4-wide lanes and
    reads each lane's element on its own (index at lane base + l); every
    load whose index holds a pad or concatenate clamp is issued only where
    each clamp is the identity, and fills zeros elsewhere."""
    spec = W.pad_reverse_concat_minor_f32()[0]
    f = H.Fusion(spec.nodes, mode="compile")
    p, src = f.plan(), f.source()
    assert p["hero"] == "loop" and p["vector_elems"] == 4
    lanes = [ln.strip() for ln in src.splitlines() if ln.strip().startswith("for (int l = 0; l < 4; ++l) R.")]
    assert len(lanes) == 2, lanes
    for ln in lanes:
        assert "(i1 + l)" in ln and "? A.p" in ln and ln.endswith(": 0;"), ln
    # y is read only where the concatenate's clamp on it is the identity
    assert "((i1 + l) - 2048) >= (0) && ((i1 + l) - 2048) <= (2047)" in lanes[1]


def test_slice_plans():
    """A slice keeps 128-bit lanes when its start along the minor dim is a
    multiple of the vector width and counts only the elements it reads; a
    dynamic start along the minor dim reads one element per lane."""
    s = W.Spec()
    p = s.parameter(0, "f32", [64, 256])
    s.slice(p, [3, 8], [40, 200], [1, 1], "f32", [37, 192])
    pl = plan_of(s)
    assert pl["hero"] == "loop" and pl["vector_elems"] == 4
    assert pl["algorithmic_bytes"] == 2 * 37 * 192 * 4
    s = W.Spec()
    p = s.parameter(0, "f32", [64, 256])
    s.slice(p, [3, 6], [40, 198], [1, 1], "f32", [37, 192])
    assert plan_of(s)["vector_elems"] == 2
    s = W.Spec()
    p = s.parameter(0, "bf16", [64, 256])
    a, b = s.parameter(1, "s32", []), s.parameter(2, "s32", [])
    s.dynamic_slice(p, [a, b], [16, 128], "bf16")
    pl = plan_of(s)
    assert pl["algorithmic_bytes"] == 2 * 16 * 128 * 2 + 8
    src = H.Fusion(s.nodes, mode="compile").source()
    assert "hf_clampi((int)hf_a_p1[0], 0, 48)" in src and "hf_clampi((int)hf_a_p2[0], 0, 128)" in src
    # a start along a dim sliced whole is 0 whatever the parameter holds
    s = W.Spec()
    p = s.parameter(0, "f32", [64, 256])
    a, b = s.parameter(1, "s32", []), s.parameter(2, "s32", [])
    s.dynamic_slice(p, [a, b], [16, 256], "f32")
    src = H.Fusion(s.nodes, mode="compile").source()
    assert "hf_a_p2[0]" not in src and "hf_raw_ld<16, true>" in src
    # the transposed read of a slice still picks the transpose hero
    s = W.Spec()
    p = s.parameter(0, "f32", [512, 512])
    q = s.slice(p, [0, 64], [512, 448], [1, 1], "f32", [512, 384])
    s.transpose(q, [1, 0], "f32", [384, 512])
    assert plan_of(s)["hero"] == "transpose"


def test_reduce_epilogue_is_planned_as_a_second_context():
    s = W.Spec()
    p = s.parameter(0, "f32", [64, 300])
    b = s.parameter(1, "f32", [64])
    r = s.reduce(p, [1], "add", 0.0, "f32", [64])
    e = s.unary("exponential", r, "f32", [64])
    s.binary("add", e, b, "f32", [64])
    pl = plan_of(s)
    assert pl["hero"] == "row_reduce"
    assert pl["n_partitions"] == 1  # the epilogue (exp, add); the reduce input is a bare parameter
    assert pl["algorithmic_bytes"] == 4 * 64 * 300 + 4 * 64 + 4 * 64


# --------------------------------------------------------------------------
# planning decisions
# --------------------------------------------------------------------------
def test_partitioning_of_log_transpose_add():
    """param -> log -> {transpose, add}: the pages' partitioner makes three
    one-instruction functions (XLA:GPU Emitters, "Partitioning")."""
    spec, _, _ = W.loop_log_transpose_add(64)
    p = plan_of(spec)
    assert p["hero"] == "loop" and p["n_partitions"] == 3
    # the same graph with exp in front of log: exp has one user and joins log
    s = W.Spec()
    x = s.parameter(0, "f32", [8, 8], [1, 0])
    e = s.unary("exponential", x, "f32", [8, 8])
    l = s.unary("log", e, "f32", [8, 8])
    t = s.transpose(l, [1, 0], "f32", [8, 8])
    s.binary("add", l, t, "f32", [8, 8])
    assert plan_of(s)["n_partitions"] == 3
    # a node read twice at the same index stays in its user's function
    s = W.Spec()
    x = s.parameter(0, "f32", [8, 8])
    l = s.unary("log", x, "f32", [8, 8])
    s.binary("multiply", l, l, "f32", [8, 8])
    assert plan_of(s)["n_partitions"] == 1


def test_hero_classification():
    cases = [
        (W.transpose_exp_f32(64, 96), "transpose"),
        (W.transpose_bf16_021(2, 64, 96), "transpose"),
        (W.row_reduce_exp_add_bf16(2, 4, 512), "row_reduce"),
        (W.row_reduce_exp_add_bf16(2, 4, 512, m2m=(3, 2, 0, 1)), "row_reduce"),
        (W.column_reduce_max_f32(256, 64), "column_reduce"),
        (W.column_reduce_max_f32(256, 64, m2m=(0, 1)), "row_reduce"),
        (W.quant_dequant_bias_requant(16, 64), "loop"),
        (W.gelu_bf16(2, 4, 64), "loop"),
        (W.transpose3d_exp_abs(), "transpose"),
    ]
    for (spec, _, meta), hero in cases:
        assert plan_of(spec)["hero"] == hero, meta["name"]
    # the pages' 3-D example: exp is read into the tile, abs runs after it
    assert plan_of(W.transpose3d_exp_abs()[0])["n_partitions"] == 2
    # a transpose that is the identity in memory is a plain loop
    s = W.Spec()
    x = s.parameter(0, "f32", [64, 32], [0, 1])
    s.transpose(x, [1, 0], "f32", [32, 64], m2m=[1, 0])
    assert plan_of(s)["hero"] == "loop"
    # a layout change without a transpose op is still a transpose in memory
    s = W.Spec()
    x = s.parameter(0, "f32", [64, 32], [1, 0])
    s.unary("exponential", x, "f32", [64, 32], m2m=[0, 1])
    assert plan_of(s)["hero"] == "transpose"


def test_algorithmic_bytes_of_the_workloads():
    expect = {
        "loop_log_transpose_add": 32768, "transpose_exp_f32": 134217728,
        "transpose_bf16_021": 134217728, "row_reduce_exp_add_bf16": 335618048,
        "column_reduce_max_f32": 268451840, "quant_dequant_bias_requant": 33591296,
    }
    for make in (W.loop_log_transpose_add, W.transpose_exp_f32, W.transpose_bf16_021,
                 W.row_reduce_exp_add_bf16, W.column_reduce_max_f32, W.quant_dequant_bias_requant):
        spec, _, meta = make()
        assert plan_of(spec)["algorithmic_bytes"] == expect[meta["name"]], meta["name"]


def test_transpose_tile_arithmetic_of_the_pages_example():
    """The pages' transpose example (20x160x170 -> 170x160x20 with 32-wide tiles
    over the two swapped dims, one batch index per block) has 960 blocks.  Our
    tiling merges the output's middle dim (160, physically between the
    output's minor dim and the transposed one) into the tile's U index, which
    runs over 160 x 20 = 3200 contiguous outputs: with the same 32x32 tiles
    (chosen by itself for a grid this small) that is 100 x 6 = 600 blocks,
    with no padding of the 20-long rows up to 32."""
    ntiles = -(-20 // 32) * 160 * -(-170 // 32)
    assert ntiles == 960
    s = W.Spec()
    x = s.parameter(0, "f32", [20, 160, 170])
    e = s.unary("exponential", x, "f32", [20, 160, 170])
    s.transpose(e, [2, 1, 0], "f32", [170, 160, 20])
    p = plan_of(s)
    assert p["hero"] == "transpose" and (p["tile_rows"], p["tile_cols"]) == (32, 32)
    assert p["cols"] == 3200 and p["grid_blocks"] == -(-3200 // 32) * -(-170 // 32) == 600


# (dtype, input dims, permutation) -> (TU, TW, threads, tile order)
# order: 0 U-tiles fastest, 1 W-tiles fastest, 2 diagonal, 3 XCD-contiguous
TRANSPOSE_GEOMETRY = [
    ("f32", [4096, 4096], [1, 0], (32, 128, 1024, 2)),     # 16 KiB rows: narrow, diagonal
    ("f32", [1024, 16384], [1, 0], (32, 128, 1024, 0)),    # 128 W-tiles, 32 U-tiles: U fastest
    ("f32", [2048, 16384], [1, 0], (32, 128, 1024, 2)),    # 128 W-tiles, 64 U-tiles: diagonal
    ("f32", [16384, 1024], [1, 0], (32, 128, 1024, 1)),    # narrow on 4 KiB rows: W fastest
    ("f32", [65536, 256], [1, 0], (32, 128, 1024, 0)),     # narrow on 1 KiB rows
    ("f32", [32768, 512], [1, 0], (32, 128, 1024, 0)),
    ("f32", [4096, 8, 256], [0, 2, 1], (8, 64, 256, 0)),   # U extent 8: no narrow tile
    ("f32", [4096, 1024], [1, 0], (64, 64, 512, 2)),       # narrow would make 1024 WGs
    ("f32", [4160, 4160], [1, 0], (64, 64, 512, 2)),       # not a power of two
    ("f32", [20, 160, 170], [2, 1, 0], (32, 32, 512, 3)),  # rows of 680 B; small grid
    ("bf16", [16384, 2048], [1, 0], (64, 64, 512, 2)),     # 4 KiB rows: diagonal
    ("bf16", [64, 512, 1024], [0, 2, 1], (64, 64, 512, 0)),  # 2 KiB rows
    ("bf16", [2048, 16384], [1, 0], (64, 64, 512, 0)),     # 256 W-tiles, 32 U-tiles
]


@pytest.mark.parametrize("dt,dims,perm,want", TRANSPOSE_GEOMETRY,
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, list) else str(v))
def test_transpose_geometry_choice(dt, dims, perm, want):
    """Tile shape, threads and tile order as measured best: the narrow
    32x128 tile for 4-byte types with power-of-two rows (of 512 B to 4 KiB
    only when it makes 2048 workgroups or more over U extents of 32 or
    more), the diagonal order from
    4 KiB rows while the U-tiles number at least half the W-tiles, U fastest
    otherwise, W fastest for the narrow tile on 4 KiB rows, and the
    XCD-contiguous order for rows that are not whole 128-byte lines."""
    s = W.Spec()
    x = s.parameter(0, dt, dims)
    e = s.unary("exponential", x, dt, dims)
    s.transpose(e, perm, dt, [dims[p] for p in perm])
    src = H.Fusion(s.nodes, mode="compile").source()
    m = {k: int(v) for k, v in re.findall(r"#define (HF_TU|HF_TW|HF_BLOCK|HF_ORDER) (\d+)", src)}
    assert (m["HF_TU"], m["HF_TW"], m["HF_BLOCK"], m["HF_ORDER"]) == want


@pytest.mark.parametrize("dims,grid,block", [([65536, 256], 2048, 256), ([262144, 64], 2048, 256),
                                             ([1048576, 16], 2048, 256), ([300, 256], 75, 256),
                                             ([16384, 1024], 8192, 256), ([8192, 2048], 4096, 512),
                                             ([4096, 4096], 4096, 512), ([10240, 4096], 10240, 512),
                                             ([2048, 16384], 1024, 512)])
def test_row_reduce_grid_choice(dims, grid, block):
    """Row reduces: whole-row workgroups one per row step (up to 65,536),
    two rows a step where each thread holds one chunk of a row or eight and
    more, one row otherwise; rows of fewer than 256 vectors share workgroups
    of 256 threads, which loop over the rows in a grid of at most 2048 (one
    round of 32 waves on each of the 256 CUs)."""
    s = W.Spec()
    p = s.parameter(0, "f32", dims)
    s.reduce(p, [1], "add", 0.0, "f32", [dims[0]])
    pl = plan_of(s)
    assert pl["hero"] == "row_reduce" and (pl["grid_blocks"], pl["block_threads"]) == (grid, block)


@pytest.mark.parametrize("dims,grid,rows_per_seg,cols_per_wg", [
    ([16384, 4096], 4096, 128, 128),   # 32 column lanes of 4; 128 segments of 128 rows
    ([4096, 4096], 1024, 128, 128),    # segments of at least 128 rows
    ([16384, 1024], 2048, 128, 64),    # 2048 columns or fewer: 16 column lanes
    ([65536, 256], 1024, 256, 64),     # at most 256 segments
    ([262144, 64], 256, 1024, 64),
    ([1048576, 16], 256, 4096, 16),    # 4 column lanes cover the 16 columns
    ([100, 4096], 32, 100, 128),       # one segment: no workspace, no fold
])
def test_column_reduce_geometry_choice(dims, grid, rows_per_seg, cols_per_wg):
    """Column reduces: workgroups of 128 columns (32 lanes of four) or, for
    2048 columns or fewer, of 64; the rows split into at most 256 segments
    of at least 128 rows, toward 4096 workgroups; a workspace of one partial
    per segment and column only when there are two segments or more."""
    s = W.Spec()
    p = s.parameter(0, "f32", dims)
    s.reduce(p, [0], "max", float("-inf"), "f32", [dims[1]])
    pl = plan_of(s)
    assert pl["hero"] == "column_reduce"
    assert (pl["grid_blocks"], pl["tile_rows"], pl["tile_cols"]) == (grid, rows_per_seg, cols_per_wg)
    segs = -(-dims[0] // rows_per_seg)
    assert pl["workspace_bytes"] == (segs * dims[1] * 4 if segs > 1 else 0)


@pytest.mark.parametrize("dims,red,segs,grid,ws", [
    ([16, 1048576], "add", 64, 1024, 16 * 64 * 4),
    ([1, 16777216], "add", 1024, 1024, 1024 * 4),    # one row: 1024 segments
    ([64, 65536], "add", 4, 256, 64 * 4 * 4),        # segments of one batch of loads at least
    ([4, 262144], "argmax", 32, 128, 4 * 32 * 8),    # values and indices
    ([2048, 4096], "add", 1, 2048, 0),               # enough rows: no split
])
def test_row_reduce_split_choice(dims, red, segs, grid, ws):
    """A few long rows split into segments toward 2048 workgroups, each
    segment at least eight chunks a thread; the workspace holds a partial
    per row and segment (with its index for argmax), folded by one
    workgroup per row."""
    s = W.Spec()
    p = s.parameter(0, "f32", dims)
    if red == "argmax":
        s.argmax(p, 1, dims)
    else:
        s.reduce(p, [1], "add", 0.0, "f32", [dims[0]])
    f = H.Fusion(s.nodes, mode="compile")
    pl, src = f.plan(), f.source()
    assert "#define HF_RSEG %d\n" % segs in src
    assert (pl["grid_blocks"], pl["workspace_bytes"]) == (grid, ws)


# --------------------------------------------------------------------------
# code generation and compilation for gfx950
# --------------------------------------------------------------------------
WORKLOADS = [W.loop_log_transpose_add, W.transpose_exp_f32, W.transpose_bf16_021,
             W.row_reduce_exp_add_bf16, W.column_reduce_max_f32, W.quant_dequant_bias_requant,
             W.gelu_bf16, W.quant_dequant_bias_requant_s4]


@pytest.mark.parametrize("make", WORKLOADS, ids=lambda m: m.__name__)
def test_workload_compiles_for_gfx950(make):
    spec, _, _ = make()
    f = H.Fusion(spec.nodes, mode="compile")
    src = f.source()
    assert "HF_KERNEL_NAME" in src and "__builtin_amdgcn" in src


@pytest.mark.skipif(shutil.which("/opt/rocm/bin/hipcc") is None, reason="needs hipcc")
@pytest.mark.parametrize("make", [W.quant_dequant_bias_requant, W.row_reduce_exp_add_bf16,
                                  W.transpose_exp_f32], ids=lambda m: m.__name__)
def test_no_packed_fp32_and_no_scratch(make):
    """The generated kernels, compiled with the library's flags, contain no
    packed-FP32 instructions and use no scratch memory."""
    spec, _, _ = make()
    src = H.Fusion(spec.nodes, mode="compile").source()
    with tempfile.TemporaryDirectory() as d:
        hip = os.path.join(d, "k.hip")
        co = os.path.join(d, "k.co")
        open(hip, "w").write(src)
        subprocess.check_call(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17",
                               "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang",
                               "-packed-fp32-ops", "--cuda-device-only", "--no-gpu-bundle-output",
                               "-include", "hip/hip_runtime.h", "-c", "-x", "hip", hip, "-o", co],
                              stderr=subprocess.DEVNULL)
        dis = subprocess.check_output(["/opt/rocm/llvm/bin/llvm-objdump", "-d", "--mcpu=gfx950", co]).decode()
        notes = subprocess.check_output(["/opt/rocm/llvm/bin/llvm-readelf", "--notes", co]).decode()
    assert not re.search(r"v_pk_(fma|mul|add)_f32", dis)
    assert re.search(r"\.private_segment_fixed_size:\s+0\b", notes)


def test_generated_code_is_deterministic():
    spec, _, _ = W.quant_dequant_bias_requant(64, 128)
    a = H.Fusion(spec.nodes, mode="compile").source()
    b = H.Fusion(spec.nodes, mode="compile").source()
    assert a == b


# --------------------------------------------------------------------------
# arithmetic claims the kernels rely on (checked on the host with numpy)
# --------------------------------------------------------------------------
def test_reciprocal_double_quotient_equals_ieee_f32_division():
    """fl32(fl64(y * fl64(1/s))) == fl32(y / s) (IEEE) for f32 y and s: the
    quantize kernels divide this way.  Random scales and values, and values
    placed next to every rounding midpoint of the quotient."""
    g = W.rng(70)
    for _ in range(40):
        s = np.float32(np.exp(g.uniform(np.log(1e-4), np.log(10.0))))
        y = (g.standard_normal(200000) * g.uniform(0.01, 10)).astype(np.float32)
        got = (y.astype(np.float64) * (1.0 / np.float64(s))).astype(np.float32)
        want = y / s
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
        # quotients next to f32 midpoints: y = fl32(m * s) around midpoints m
        q = (g.standard_normal(50000) * 100).astype(np.float32)
        m = (q.astype(np.float64) + np.spacing(q).astype(np.float64) / 2)
        yy = (m * np.float64(s)).astype(np.float32)
        for off in (-1, 0, 1):
            y2 = (yy.view(np.int32) + off).view(np.float32)
            got = (y2.astype(np.float64) * (1.0 / np.float64(s))).astype(np.float32)
            assert np.array_equal(got.view(np.uint32), (y2 / s).view(np.uint32))


def test_code_object_cache_dir_under_concurrent_creates(tmp_path, monkeypatch):
    """HF_CACHE_DIR: eight threads compile the same three fusions at once.
    Each distinct source leaves exactly one code object and no temporary
    file; a fresh process then creates the same fusions from the directory."""
    import os
    import subprocess
    import sys
    from concurrent.futures import ThreadPoolExecutor
    monkeypatch.setenv("HF_CACHE_DIR", str(tmp_path))
    specs = []
    for n in (1000, 1001, 1002):   # sizes that no other test compiles in this process
        s = W.Spec()
        p = s.parameter(0, "f32", [n])
        s.unary("exponential", p, "f32", [n])
        specs.append(s)
    with ThreadPoolExecutor(max_workers=8) as pool:
        plans = list(pool.map(lambda k: H.Fusion(specs[k % 3].nodes, mode="compile").plan()["hero"], range(24)))
    assert plans == ["loop"] * 24
    files = sorted(os.listdir(tmp_path))
    assert len(files) == 3 and all(f.endswith(".co") for f in files), files
    code = ("import sys; sys.path.insert(0, %r); import compiler_hlo_amd as H, workloads as W\n"
            "for n in (1000, 1001, 1002):\n"
            "    s = W.Spec(); p = s.parameter(0, 'f32', [n]); s.unary('exponential', p, 'f32', [n])\n"
            "    assert H.Fusion(s.nodes, mode='compile').plan()['hero'] == 'loop'\n"
            "print('ok')\n") % ROOT
    stamps = {f: os.stat(tmp_path / f).st_mtime_ns for f in files}
    env = dict(os.environ, HF_CACHE_DIR=str(tmp_path))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stderr[-2000:]
    # read from the directory, not compiled and written again
    assert {f: os.stat(tmp_path / f).st_mtime_ns for f in os.listdir(tmp_path)} == stamps


def _f16_negate_multiply_chain():
    """An f16 chain (negate, subtract, multiply, adds) on a rank-5 transposed
    read: with SLP vectorization on, the device compiler aborted on it
    ("Cannot select" of an i32 -> v2f32 bitcast) under -packed-fp32-ops."""
    dims_in, dims = [17, 4, 3, 16, 1], [16, 3, 4, 17, 1]
    s = W.Spec()
    p = s.parameter(0, "f16", dims_in)
    t = s.transpose(p, [3, 2, 1, 0, 4], "f16", dims)
    n = s.unary("negate", t, "f16", dims)
    d = s.binary("subtract", t, n, "f16", dims)
    m = s.binary("multiply", d, n, "f16", dims)
    a = s.binary("add", m, t, "f16", dims)
    b = s.binary("add", a, n, "f16", dims)
    s.binary("add", b, d, "f16", dims, m2m=[0, 3, 4, 2, 1])
    return s


def test_f16_chain_that_crashed_the_device_compiler_compiles():
    f = H.Fusion(_f16_negate_multiply_chain().nodes, mode="compile")
    assert f.plan()["hero"] == "loop"
