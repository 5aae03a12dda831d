"""Descriptor mutation: valid fusion descriptors with one to three fields
set to random, often out-of-range, values, handed to hf_fusion_create.
Every call must return OK, INVALID or UNSUPPORTED; a descriptor that plans
must also generate and compile.  Pointers are never mutated (the C ABI takes
them as the caller's promise), and every count is backed by memory: the node
array holds HF_MAX_NODES entries and each quantization type 64 more scales
and zero points than it declares (a mutated count grows by at most 6)."""
import ctypes
import types

import numpy as np

import compiler_hlo_amd as H

MAX_NODES = 256
QN = 64
DIMS = [-1, 0, 1, 2, 3, 7, 64, 4096, 1 << 31, 1 << 40, 1 << 62]


def marshal(nodes, root, n_params):
    """(desc, keepalive) with spare capacity behind every count."""
    keep = []
    arr = (H.HfNode * MAX_NODES)()
    filler = types.SimpleNamespace(_keep=keep)
    for i, nd in enumerate(nodes):
        H.Fusion._fill(filler, arr[i], nd)
        if nd.get("quant") is not None:
            hq = arr[i].type.quant.contents
            sc = np.ones(hq.n + QN, np.float32)
            zp = np.zeros(hq.n + QN, np.int32)
            sc[:hq.n] = np.ctypeslib.as_array(hq.scales, (hq.n,))
            zp[:hq.n] = np.ctypeslib.as_array(hq.zero_points, (hq.n,))
            keep += [sc, zp]
            hq.scales = sc.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
            hq.zero_points = zp.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    desc = H.HfFusionDesc(H.ABI_VERSION, len(nodes), arr, root, n_params)
    return desc, (arr, keep)


def mutate(g, desc, n):
    """Set one random field of the descriptor or of one of its first n nodes."""
    arr = desc.nodes
    k = int(g.integers(0, 40))
    if k == 0:
        desc.n_nodes = int(g.integers(0, min(n + 3, MAX_NODES) + 1))
        return
    if k == 1:
        desc.root = int(g.integers(-1, n + 2))
        return
    if k == 2:
        desc.n_params = int(g.integers(-1, 18))
        return
    nd = arr[int(g.integers(0, n))]
    t = nd.type
    f = int(g.integers(0, 19))
    if f == 0:
        nd.op = int(g.integers(-2, 40))
    elif f == 1:
        nd.n_operands = int(g.integers(-1, 10))
    elif f == 2:
        nd.operands[int(g.integers(0, 8))] = int(g.integers(-2, n + 3))
    elif f == 3:
        t.dtype = int(g.integers(-1, 11))
    elif f == 4:
        t.rank = int(g.integers(-1, 10))
    elif f == 5:
        t.dims[int(g.integers(0, 8))] = int(g.choice(DIMS))
    elif f == 6:
        t.has_layout = int(g.integers(0, 3))
    elif f == 7:
        t.minor_to_major[int(g.integers(0, 8))] = int(g.integers(-1, 10))
    elif f == 8:
        nd.parameter_number = int(g.integers(-1, 18))
    elif f == 9:
        nd.constant = float(g.choice([np.nan, np.inf, -np.inf, -0.0, 1e300, 3.5]))
    elif f == 10:
        nd.n_attr = int(g.integers(-1, 26))
    elif f == 11:
        nd.attr[int(g.integers(0, 24))] = int(g.choice([-3, -1, 0, 1, 2, 3, 5, 9, 1 << 40]))
    elif f == 12:
        nd.reducer = int(g.integers(-1, 7))
    elif f == 13:
        nd.init_value = float(g.choice([np.nan, np.inf, -np.inf, -0.0, 0.0, 1.0]))
    elif t.quant:
        q = t.quant.contents
        if f == 14:
            q.quantization_dimension = int(g.integers(-2, 10))
        elif f == 15:
            q.n = int(g.integers(-1, max(q.n, 0) + 3))
        elif f == 16:
            q.has_storage_range = int(g.integers(0, 3))
            q.storage_min, q.storage_max = (int(v) for v in g.integers(-300, 300, 2))
        elif f == 17:
            q.scales[int(g.integers(0, max(q.n, 1)))] = float(g.choice([0.0, -1.0, np.nan, np.inf, 1e-40, 3e38]))
        else:
            q.zero_points[int(g.integers(0, max(q.n, 1)))] = int(g.integers(-300, 300))


def run(bases, count, seed, compile_every=50):
    """Mutate and create `count` times; returns (status counts, compiled)."""
    g = np.random.default_rng(seed)
    lib = H.library()
    counts = {}
    compiled = 0
    for it in range(count):
        nodes, root, n_params = bases[it % len(bases)]
        desc, keep = marshal(nodes, root, n_params)
        for _ in range(int(g.integers(1, 4))):
            mutate(g, desc, len(nodes))
        h = ctypes.c_void_p()
        rc = lib.hf_fusion_create(ctypes.byref(desc), H.PLAN_ONLY, ctypes.byref(h))
        assert rc in (0, 1, 2), (it, rc, lib.hf_last_error())
        counts[rc] = counts.get(rc, 0) + 1
        if rc == 0:
            lib.hf_fusion_destroy(h)
            if it % compile_every == 0:
                h2 = ctypes.c_void_p()
                rc2 = lib.hf_fusion_create(ctypes.byref(desc), H.COMPILE_ONLY, ctypes.byref(h2))
                assert rc2 == 0, (it, rc2, lib.hf_last_error())
                lib.hf_fusion_destroy(h2)
                compiled += 1
        del keep
    return counts, compiled
