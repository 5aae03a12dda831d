"""Python binding of the CPU oracle (``hlo_oracle.c``).

TEST INFRASTRUCTURE ONLY.  The tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use this module to compute the expected
result of a fusion; the product package ``compiler_hlo_amd`` never imports it
and shares no code with it.

A fusion is given in the neutral node-list form (a list of dicts, the last
node is the root unless ``root`` says otherwise)::

    {"op": "parameter", "param": 0, "dtype": "f32", "dims": [64, 64], "m2m": [1, 0]}
    {"op": "log", "operands": [0], "dtype": "f32", "dims": [64, 64]}
    {"op": "transpose", "operands": [1], "dtype": "f32", "dims": [64, 64],
     "permutation": [1, 0]}
    ...

Every node states its own result type, as HLO text does.  Parameters and the
root carry a ``minor_to_major`` layout (``m2m``); when it is missing the
default layout [rank-1, ..., 0] applies (Shapes and layout, "Default
minor-to-major ordering").  Buffers are flat numpy arrays in physical order.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hlo_oracle.c")
_LIB = os.path.join(_HERE, "libhlo_oracle.so")

MAX_RANK = 8
MAX_OPERANDS = 9
MAX_ATTR = 24
DTYPES = {"f32": 0, "bf16": 1, "f16": 2, "s8": 3, "s32": 4, "u8": 5, "s4": 6, "u4": 7}
# Host buffers: one element per item, except s4/u4, which are packed two per
# byte (see storage_size).
NP_STORAGE = {"f32": np.float32, "bf16": np.uint16, "f16": np.uint16, "s8": np.int8,
              "s32": np.int32, "u8": np.uint8, "s4": np.uint8, "u4": np.uint8}


def storage_size(dtype: str, n: int) -> int:
    """Items of NP_STORAGE[dtype] that hold n elements: s4/u4 take one byte
    per two elements (the last byte half used when n is odd)."""
    return (n + 1) // 2 if dtype in ("s4", "u4") else n
OPS = {
    "parameter": 0, "constant": 1, "log": 2, "exponential": 3, "tanh": 4,
    "add": 5, "subtract": 6, "multiply": 7, "divide": 8, "maximum": 9,
    "minimum": 10, "negate": 11, "abs": 12, "convert": 13,
    "broadcast_in_dim": 14, "reshape": 15, "transpose": 16,
    "uniform_dequantize": 17, "uniform_quantize": 18, "reduce": 19, "dot": 20,
    "reverse": 21, "iota": 22, "pad": 23, "concatenate": 24, "slice": 25,
    "dynamic_slice": 26,
}
REDUCERS = {"add": 0, "max": 1, "min": 2, "argmax": 3}


def build(force: bool = False) -> str:
    """Compile the oracle with gcc: single-threaded, no FMA contraction, no fast-math."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
            "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unused-parameter",
            "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class OrType(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("rank", ctypes.c_int32),
        ("dims", ctypes.c_int64 * MAX_RANK), ("m2m", ctypes.c_int32 * MAX_RANK),
        ("quantized", ctypes.c_int32), ("qdim", ctypes.c_int32), ("nq", ctypes.c_int64),
        ("scales", ctypes.POINTER(ctypes.c_double)),
        ("zero_points", ctypes.POINTER(ctypes.c_int64)),
        ("storage_min", ctypes.c_int64), ("storage_max", ctypes.c_int64),
    ]


class OrNode(ctypes.Structure):
    _fields_ = [
        ("op", ctypes.c_int32), ("n_operands", ctypes.c_int32),
        ("operands", ctypes.c_int32 * MAX_OPERANDS), ("type", OrType),
        ("param_index", ctypes.c_int32), ("constant", ctypes.c_double),
        ("n_attr", ctypes.c_int32), ("attr", ctypes.c_int64 * MAX_ATTR),
        ("reducer", ctypes.c_int32), ("init", ctypes.c_double),
    ]


_lib_handle = None


def lib():
    global _lib_handle
    if _lib_handle is None:
        h = ctypes.CDLL(build())
        h.or_last_error.restype = ctypes.c_char_p
        h.or_linear_index.restype = ctypes.c_int64
        h.or_linear_index.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_int64),
                                      ctypes.POINTER(ctypes.c_int32),
                                      ctypes.POINTER(ctypes.c_int64)]
        h.or_round_format_d.restype = ctypes.c_double
        h.or_round_format_d.argtypes = [ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        h.or_eval.restype = ctypes.c_int
        h.or_eval_points.restype = ctypes.c_int
        _lib_handle = h
    return _lib_handle


def default_m2m(rank: int) -> list[int]:
    return list(range(rank - 1, -1, -1))


def _storage_bounds(dtype: str) -> tuple[int, int]:
    return {"s8": (-128, 127), "u8": (0, 255), "s4": (-8, 7), "u4": (0, 15),
            "s32": (-(2 ** 31), 2 ** 31 - 1)}[dtype]


class _Graph:
    """ctypes image of a node list; keeps the quantization arrays alive."""

    def __init__(self, nodes: list[dict], root: int | None = None):
        self.n = len(nodes)
        self.root = self.n - 1 if root is None else root
        self.arr = (OrNode * self.n)()
        self._keep = []
        for i, nd in enumerate(nodes):
            c = self.arr[i]
            c.op = OPS[nd["op"]]
            ops = list(nd.get("operands", []))
            c.n_operands = len(ops)
            for k, o in enumerate(ops):
                c.operands[k] = o
            dims = list(nd["dims"])
            c.type.dtype = DTYPES[nd["dtype"]]
            c.type.rank = len(dims)
            m2m = nd.get("m2m")
            if m2m is None:
                m2m = default_m2m(len(dims))
            for d in range(len(dims)):
                c.type.dims[d] = dims[d]
                c.type.m2m[d] = m2m[d]
            q = nd.get("quant")
            c.type.qdim = -1
            if q is not None:
                c.type.quantized = 1
                qd = q.get("qdim")
                c.type.qdim = -1 if qd is None else qd
                sc = np.ascontiguousarray(np.asarray(q["scales"], dtype=np.float32).astype(np.float64))
                zp = np.ascontiguousarray(np.asarray(q["zero_points"], dtype=np.int64))
                self._keep += [sc, zp]
                c.type.nq = sc.size
                c.type.scales = sc.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
                c.type.zero_points = zp.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
                lo, hi = _storage_bounds(nd["dtype"])
                c.type.storage_min = q.get("storage_min", lo)
                c.type.storage_max = q.get("storage_max", hi)
            c.param_index = nd.get("param", -1)
            c.constant = float(nd.get("value", nd.get("index_init", 0.0)))
            if nd["op"] == "pad":
                attr = list(nd["edge_padding_low"]) + list(nd["edge_padding_high"]) + list(nd["interior_padding"])
            elif nd["op"] == "iota":
                attr = [nd["iota_dimension"]]
            elif nd["op"] == "concatenate":
                attr = [nd["dimension"]]
            elif nd["op"] == "slice":
                attr = list(nd["start_indices"]) + list(nd["limit_indices"]) + list(nd["strides"])
            elif nd["op"] == "dynamic_slice":
                attr = list(nd["slice_sizes"])
            else:
                attr = nd.get("permutation", nd.get("broadcast_dimensions", nd.get("dimensions", [])))
            c.n_attr = len(attr)
            for k, a in enumerate(attr):
                c.attr[k] = a
            c.reducer = REDUCERS[nd.get("reducer", "add")]
            c.init = float(nd.get("init", 0.0))
        self.root_node = nodes[self.root]

    def param_ptrs(self, params):
        bufs = [np.ascontiguousarray(p) for p in params]
        self._keep += bufs
        arr = (ctypes.c_void_p * max(1, len(bufs)))()
        for i, b in enumerate(bufs):
            arr[i] = b.ctypes.data
        return arr, len(bufs)


def _check(rc):
    if rc != 0:
        raise RuntimeError("oracle: %s (rc=%d)" % (lib().or_last_error().decode(), rc))


def evaluate(nodes: list[dict], params: list[np.ndarray], root: int | None = None) -> np.ndarray:
    """Whole root, encoded in the root's layout: flat array of its storage type."""
    g = _Graph(nodes, root)
    rn = g.root_node
    n = int(np.prod(rn["dims"], dtype=np.int64))
    out = np.zeros(storage_size(rn["dtype"], n), dtype=NP_STORAGE[rn["dtype"]])
    pp, npar = g.param_ptrs(params)
    _check(lib().or_eval(g.arr, g.n, g.root, pp, npar, ctypes.c_void_p(out.ctypes.data)))
    return out


def evaluate_points(nodes: list[dict], params: list[np.ndarray], points,
                    root: int | None = None):
    """Root value at logical indices ``points`` (n x rank).

    Returns (values, aux): values as float64 (exact for every supported type);
    aux[:, 0] = sum of |operand| and aux[:, 1] = the unrounded accumulator
    when the root is a reduce (zeros otherwise).
    """
    g = _Graph(nodes, root)
    pts = np.ascontiguousarray(np.asarray(points, dtype=np.int64))
    n = pts.shape[0]
    vals = np.zeros(n, dtype=np.float64)
    aux = np.zeros((n, 2), dtype=np.float64)
    pp, npar = g.param_ptrs(params)
    _check(lib().or_eval_points(g.arr, g.n, g.root, pp, npar, ctypes.c_int64(n),
                                ctypes.c_void_p(pts.ctypes.data),
                                ctypes.c_void_p(vals.ctypes.data),
                                ctypes.c_void_p(aux.ctypes.data)))
    return vals, aux


def linear_index(dims, m2m, idx) -> int:
    r = len(dims)
    d = (ctypes.c_int64 * MAX_RANK)(*dims)
    m = (ctypes.c_int32 * MAX_RANK)(*m2m)
    i = (ctypes.c_int64 * MAX_RANK)(*idx)
    return lib().or_linear_index(r, d, m, i)


def linear_indices(dims, m2m, idx: np.ndarray) -> np.ndarray:
    """Vectorised linear_index over an (n x rank) index array."""
    r = len(dims)
    d = (ctypes.c_int64 * MAX_RANK)(*dims)
    m = (ctypes.c_int32 * MAX_RANK)(*m2m)
    pts = np.ascontiguousarray(np.asarray(idx, dtype=np.int64).reshape(-1, r))
    out = np.zeros(pts.shape[0], dtype=np.int64)
    lib().or_linear_indices(ctypes.c_int32(r), d, m, ctypes.c_int64(pts.shape[0]),
                            ctypes.c_void_p(pts.ctypes.data), ctypes.c_void_p(out.ctypes.data))
    return out


def round_format(v: float, p: int, emin: int, emax: int) -> float:
    """Round to a binary format with p significand bits (RNE, subnormals, overflow to inf)."""
    return lib().or_round_format_d(v, p, emin, emax)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
