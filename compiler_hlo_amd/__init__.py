"""Python binding of the hero-fusion C ABI (include/hlofusion.h).

Argument marshalling only: every step of a fusion runs in the library's
generated HIP kernels.  PyTorch provides device memory and streams.  The
shared library must have been built in-tree (``python
compiler_hlo_amd/build.py`` or ``__graft_entry__.build()``); importing this
package without it raises ImportError -- there is no fallback path.

A fusion is given as a list of node dicts (the last node is the root unless
``root`` is passed), each stating its own result type the way HLO text does::

    {"op": "parameter", "param": 0, "dtype": "f32", "dims": [64, 64], "m2m": [1, 0]}
    {"op": "log", "operands": [0], "dtype": "f32", "dims": [64, 64]}
    {"op": "transpose", "operands": [1], "dtype": "f32", "dims": [64, 64],
     "permutation": [1, 0]}
    {"op": "reduce", "operands": [k], "dtype": "f32", "dims": [...],
     "dimensions": [1], "reducer": "add", "init": 0.0}

Quantized types carry ``"quant": {"qdim": 1 or None, "scales": [...],
"zero_points": [...], "storage_min": ..., "storage_max": ...}`` with the
storage type in ``dtype``.  Parameter and result buffers are flat tensors in
physical (minor_to_major) order.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libhlofusion.so")

ABI_VERSION = 4
MAX_RANK = 8
MAX_OPERANDS = 9
MAX_ATTR = 3 * MAX_RANK
DTYPES = {"f32": 0, "bf16": 1, "f16": 2, "s8": 3, "u8": 4, "s32": 5, "s4": 6, "u4": 7}
DTYPE_BITS = {"f32": 32, "bf16": 16, "f16": 16, "s8": 8, "u8": 8, "s32": 32, "s4": 4, "u4": 4}


def storage_bytes(dtype: str, n: int) -> int:
    """Bytes of an array of n elements; s4/u4 pack two elements per byte (the
    even linear index in the low half), so n elements take ceil(n / 2)."""
    return (n * DTYPE_BITS[dtype] + 7) // 8
OPS = {
    "parameter": 0, "constant": 1, "add": 2, "subtract": 3, "multiply": 4,
    "divide": 5, "maximum": 6, "minimum": 7, "log": 8, "exponential": 9,
    "tanh": 10, "negate": 11, "abs": 12, "convert": 13, "broadcast_in_dim": 14,
    "reshape": 15, "transpose": 16, "uniform_dequantize": 17,
    "uniform_quantize": 18, "reduce": 19, "reverse": 20, "iota": 21, "pad": 22,
    "concatenate": 23, "slice": 24, "dynamic_slice": 25,
}
REDUCERS = {"add": 0, "max": 1, "min": 2, "argmax": 3}
HEROES = {0: "loop", 1: "transpose", 2: "row_reduce", 3: "column_reduce"}
STATUS = {0: "HF_OK", 1: "HF_ERR_INVALID", 2: "HF_ERR_UNSUPPORTED", 3: "HF_ERR_COMPILE",
          4: "HF_ERR_HIP", 5: "HF_ERR_NOMEM"}
PLAN_ONLY = 1
COMPILE_ONLY = 2


class HfQuant(ctypes.Structure):
    _fields_ = [("quantization_dimension", ctypes.c_int32), ("n", ctypes.c_int32),
                ("scales", ctypes.POINTER(ctypes.c_float)),
                ("zero_points", ctypes.POINTER(ctypes.c_int32)),
                ("has_storage_range", ctypes.c_int32),
                ("storage_min", ctypes.c_int32), ("storage_max", ctypes.c_int32)]


class HfType(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("dims", ctypes.c_int64 * MAX_RANK), ("has_layout", ctypes.c_int32),
                ("minor_to_major", ctypes.c_int32 * MAX_RANK),
                ("quant", ctypes.POINTER(HfQuant))]


class HfNode(ctypes.Structure):
    _fields_ = [("op", ctypes.c_int32), ("n_operands", ctypes.c_int32),
                ("operands", ctypes.c_int32 * MAX_OPERANDS), ("type", HfType),
                ("parameter_number", ctypes.c_int32), ("constant", ctypes.c_double),
                ("n_attr", ctypes.c_int32), ("attr", ctypes.c_int64 * MAX_ATTR),
                ("reducer", ctypes.c_int32), ("init_value", ctypes.c_double)]


class HfFusionDesc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("n_nodes", ctypes.c_int32),
                ("nodes", ctypes.POINTER(HfNode)), ("root", ctypes.c_int32),
                ("n_params", ctypes.c_int32)]


class HfPlanInfo(ctypes.Structure):
    _fields_ = [("hero", ctypes.c_int32), ("n_partitions", ctypes.c_int32),
                ("vector_elems", ctypes.c_int32), ("block_threads", ctypes.c_int32),
                ("grid_blocks", ctypes.c_int64), ("lds_bytes", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_int64), ("algorithmic_bytes", ctypes.c_int64),
                ("elements", ctypes.c_int64), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("tile_rows", ctypes.c_int32), ("tile_cols", ctypes.c_int32)]


def node_attr(nd: dict) -> list:
    """The attribute list of a node dict, in the order hf_node.attr holds it."""
    if nd["op"] == "pad":
        return list(nd["edge_padding_low"]) + list(nd["edge_padding_high"]) + list(nd["interior_padding"])
    if nd["op"] == "iota":
        return [int(nd["iota_dimension"])]
    if nd["op"] == "concatenate":
        return [int(nd["dimension"])]
    if nd["op"] == "slice":
        return list(nd["start_indices"]) + list(nd["limit_indices"]) + list(nd["strides"])
    if nd["op"] == "dynamic_slice":
        return list(nd["slice_sizes"])
    return list(nd.get("permutation", nd.get("broadcast_dimensions", nd.get("dimensions", []))))


EXPORTS = ["hf_fusion_create", "hf_fusion_plan", "hf_fusion_source", "hf_fusion_launch",
           "hf_fusion_launch_noalloc", "hf_fusion_destroy", "hf_last_error", "hf_abi_version",
           "hf_linear_index"]
SCRATCH_BYTES = 16 << 20  # HF_SCRATCH_BYTES: the no-allocation launch's scratch memory per GPU


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            "compiler_hlo_amd: %s is missing; build it with `python compiler_hlo_amd/build.py` "
            "(there is no fallback implementation)" % _LIB_PATH)
    # PyTorch ships its own HIP runtime under the same soname as the system's.
    # Loaded first, it serves this library too; loaded after the system one,
    # the process would hold two HIP runtimes, and whichever initialises
    # second finds no device.  So torch is imported before the library.
    import torch  # noqa: F401
    lib = ctypes.CDLL(_LIB_PATH)
    lib.hf_fusion_create.restype = ctypes.c_int
    lib.hf_fusion_create.argtypes = [ctypes.POINTER(HfFusionDesc), ctypes.c_uint32,
                                     ctypes.POINTER(ctypes.c_void_p)]
    lib.hf_fusion_plan.restype = ctypes.c_int
    lib.hf_fusion_plan.argtypes = [ctypes.c_void_p, ctypes.POINTER(HfPlanInfo)]
    lib.hf_fusion_source.restype = ctypes.c_int
    lib.hf_fusion_source.argtypes = [ctypes.c_void_p, ctypes.c_char_p, ctypes.c_size_t,
                                     ctypes.POINTER(ctypes.c_size_t)]
    lib.hf_fusion_launch.restype = ctypes.c_int
    lib.hf_fusion_launch.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p),
                                     ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p]
    lib.hf_fusion_launch_noalloc.restype = ctypes.c_int
    lib.hf_fusion_launch_noalloc.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p),
                                             ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.hf_fusion_destroy.restype = ctypes.c_int
    lib.hf_fusion_destroy.argtypes = [ctypes.c_void_p]
    lib.hf_last_error.restype = ctypes.c_char_p
    lib.hf_abi_version.restype = ctypes.c_int32
    lib.hf_linear_index.restype = ctypes.c_int64
    lib.hf_linear_index.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_int64),
                                    ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)]
    return lib


_lib = _load()


def library():
    """The loaded ctypes handle of libhlofusion.so."""
    return _lib


class FusionError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS.get(status, status), message))
        self.status = STATUS.get(status, status)
        self.message = message


def _check(rc: int):
    if rc != 0:
        raise FusionError(rc, _lib.hf_last_error().decode(errors="replace"))


def linear_index(dims, m2m, index) -> int:
    r = len(dims)
    return _lib.hf_linear_index(r, (ctypes.c_int64 * MAX_RANK)(*dims),
                                (ctypes.c_int32 * MAX_RANK)(*m2m),
                                (ctypes.c_int64 * MAX_RANK)(*index))


class PreparedLaunch:
    """hf_fusion_launch with its argument array built once (see
    Fusion.prepare); it keeps the fusion alive."""

    def __init__(self, fusion, param_ptrs, out_ptr: int, workspace: int = 0):
        self._fusion = fusion
        self._n = len(param_ptrs)
        self._arr = (ctypes.c_void_p * max(1, self._n))(*param_ptrs)
        self._out = ctypes.c_void_p(out_ptr)
        self._ws = ctypes.c_void_p(workspace)
        self._launch = _lib.hf_fusion_launch

    def __call__(self, stream: int = 0):
        rc = self._launch(self._fusion._h, self._arr, self._n, self._out, self._ws, stream)
        if rc:
            _check(rc)


class Fusion:
    """One compiled fusion.  ``mode`` is "load" (default: compile and load on
    the current GPU), "compile" (generate and compile only; no GPU) or "plan"
    (validate and plan only)."""

    def __init__(self, nodes: list[dict], root: int | None = None, mode: str = "load",
                 n_params: int | None = None):
        self.nodes = nodes
        self.root = len(nodes) - 1 if root is None else root
        if n_params is None:
            n_params = 1 + max([nd.get("param", -1) for nd in nodes if nd["op"] == "parameter"],
                               default=-1)
        self.n_params = n_params
        self._keep = []
        arr = (HfNode * len(nodes))()
        for i, nd in enumerate(nodes):
            self._fill(arr[i], nd)
        desc = HfFusionDesc(ABI_VERSION, len(nodes), arr, self.root, n_params)
        self._arr = arr
        flags = {"load": 0, "compile": COMPILE_ONLY, "plan": PLAN_ONLY}[mode]
        h = ctypes.c_void_p()
        _check(_lib.hf_fusion_create(ctypes.byref(desc), flags, ctypes.byref(h)))
        self._h = h
        self.mode = mode
        rn = nodes[self.root]
        self.out_dtype = rn["dtype"]
        self.out_numel = int(np.prod(rn["dims"], dtype=np.int64))
        self._param_nodes = {nd["param"]: nd for nd in nodes if nd["op"] == "parameter"}

    def _fill(self, c: HfNode, nd: dict):
        c.op = OPS[nd["op"]]
        ops = list(nd.get("operands", []))
        c.n_operands = len(ops)
        for k, o in enumerate(ops):
            c.operands[k] = o
        dims = list(nd["dims"])
        c.type.dtype = DTYPES[nd["dtype"]]
        c.type.rank = len(dims)
        for d, v in enumerate(dims):
            c.type.dims[d] = v
        m2m = nd.get("m2m")
        if m2m is not None:
            c.type.has_layout = 1
            for k, v in enumerate(m2m):
                c.type.minor_to_major[k] = v
        q = nd.get("quant")
        if q is not None:
            sc = np.ascontiguousarray(np.asarray(q["scales"], dtype=np.float32))
            zp = np.ascontiguousarray(np.asarray(q["zero_points"], dtype=np.int32))
            hq = HfQuant()
            qd = q.get("qdim")
            hq.quantization_dimension = -1 if qd is None else int(qd)
            hq.n = sc.size
            hq.scales = sc.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
            hq.zero_points = zp.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
            if "storage_min" in q or "storage_max" in q:
                hq.has_storage_range = 1
                lo, hi = {"s8": (-128, 127), "u8": (0, 255)}.get(nd["dtype"], (0, 0))
                hq.storage_min = int(q.get("storage_min", lo))
                hq.storage_max = int(q.get("storage_max", hi))
            self._keep += [sc, zp, hq]
            c.type.quant = ctypes.pointer(hq)
        c.parameter_number = nd.get("param", -1)
        c.constant = float(nd.get("value", nd.get("index_init", 0.0)))
        attr = node_attr(nd)
        c.n_attr = len(attr)
        for k, a in enumerate(attr):
            c.attr[k] = a
        c.reducer = REDUCERS[nd.get("reducer", "add")]
        c.init_value = float(nd.get("init", 0.0))

    def plan(self) -> dict:
        info = HfPlanInfo()
        _check(_lib.hf_fusion_plan(self._h, ctypes.byref(info)))
        d = {f: getattr(info, f) for f, _ in HfPlanInfo._fields_}
        d["hero"] = HEROES[d["hero"]]
        return d

    def source(self) -> str:
        n = ctypes.c_size_t()
        _check(_lib.hf_fusion_source(self._h, None, 0, ctypes.byref(n)))
        buf = ctypes.create_string_buffer(n.value + 1)
        _check(_lib.hf_fusion_source(self._h, buf, n.value + 1, ctypes.byref(n)))
        return buf.value.decode()

    @property
    def workspace_bytes(self) -> int:
        """Scratch bytes a launch needs (0 for most plans)."""
        return self.plan()["workspace_bytes"]

    def launch_ptrs(self, param_ptrs, out_ptr: int, stream: int = 0, workspace: int = 0):
        """Launch with raw device pointers (ints) on a raw hipStream_t;
        `workspace` is a device pointer of workspace_bytes bytes (0 when none
        is needed)."""
        arr = (ctypes.c_void_p * max(1, len(param_ptrs)))(*param_ptrs)
        _check(_lib.hf_fusion_launch(self._h, arr, len(param_ptrs), ctypes.c_void_p(out_ptr),
                                     ctypes.c_void_p(workspace), ctypes.c_void_p(stream)))

    def prepare(self, param_ptrs, out_ptr: int, workspace: int = 0):
        """A launch with fixed buffers, marshalled once: calling the returned
        object with a raw hipStream_t launches it (hf_fusion_launch) without
        rebuilding the ctypes argument array each time."""
        return PreparedLaunch(self, param_ptrs, out_ptr, workspace)

    def launch_noalloc_ptrs(self, param_ptrs, out_ptr: int, stream: int = 0):
        """hf_fusion_launch_noalloc: launch with raw device pointers, the
        library's per-GPU scratch memory standing in for the workspace (no
        allocation anywhere; overlapping calls on one GPU race on it)."""
        arr = (ctypes.c_void_p * max(1, len(param_ptrs)))(*param_ptrs)
        _check(_lib.hf_fusion_launch_noalloc(self._h, arr, len(param_ptrs), ctypes.c_void_p(out_ptr),
                                             ctypes.c_void_p(stream)))

    def __call__(self, *params, out=None, stream=None, workspace=None):
        """Run on torch tensors (flat, physical order, on the GPU); returns the
        result tensor (allocated with torch.empty if `out` is None).  A plan
        that needs a workspace takes `workspace` (a uint8 GPU tensor of at
        least workspace_bytes) or, when it is None, a fresh one from torch's
        allocator on the launch stream, which the allocator reuses only after
        this launch on that stream."""
        import torch
        if len(params) != self.n_params:
            raise ValueError("expected %d parameters, got %d" % (self.n_params, len(params)))
        for k, p in enumerate(params):
            nd = self._param_nodes.get(k)
            if nd is None:
                continue
            want = storage_bytes(nd["dtype"], int(np.prod(nd["dims"], dtype=np.int64)))
            if not p.is_contiguous() or p.numel() * p.element_size() != want:
                raise ValueError("parameter %d must be a dense buffer of %d bytes" % (k, want))
            if not p.is_cuda:
                raise ValueError("parameter %d must be a GPU tensor" % k)
        # s4/u4 results are bytes, two elements each
        tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16,
               "s8": torch.int8, "u8": torch.uint8, "s32": torch.int32,
               "s4": torch.uint8, "u4": torch.uint8}[self.out_dtype]
        n_out = storage_bytes(self.out_dtype, self.out_numel) if self.out_dtype in ("s4", "u4") else self.out_numel
        if out is None:
            dev = params[0].device if params else torch.device("cuda")
            out = torch.empty(n_out, dtype=tdt, device=dev)
        elif (not out.is_cuda or not out.is_contiguous() or out.dtype != tdt
              or out.numel() != n_out):
            raise ValueError("out must be a dense GPU tensor of %d %s items" % (n_out, tdt))
        if stream is None:
            stream = torch.cuda.current_stream()
        ws_ptr = 0
        nws = self._ws_bytes()
        if nws:
            if workspace is None:
                with torch.cuda.stream(stream):
                    workspace = torch.empty(nws, dtype=torch.uint8, device=out.device)
            elif not workspace.is_cuda or not workspace.is_contiguous() or workspace.numel() * workspace.element_size() < nws:
                raise ValueError("workspace must be a dense GPU tensor of at least %d bytes" % nws)
            ws_ptr = workspace.data_ptr()
        self.launch_ptrs([p.data_ptr() for p in params], out.data_ptr(), stream.cuda_stream, ws_ptr)
        return out

    def _ws_bytes(self) -> int:
        if not hasattr(self, "_nws"):
            self._nws = self.workspace_bytes
        return self._nws

    def close(self):
        """Destroy the handle (waits for the device first).  Raises
        FusionError if the library could not release it (the handle then
        stays open)."""
        if getattr(self, "_h", None):
            _check(_lib.hf_fusion_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
