"""hf_fusion_launch_noalloc, the launch that allocates nothing: its output
equals hf_fusion_launch's (with a caller workspace) bit for bit, on two
calls in a row, the second with a smaller input, through the C ABI.  The
column reduces and the row reduces of a few long rows below are split into
segments, so their launches use the library's scratch memory; a loop needs
none.  A plan whose workspace exceeds the scratch memory is rejected."""
import numpy as np
import pytest

import oracle
import workloads as W
from harness import assert_bitexact, from_device, to_device

pytestmark = pytest.mark.gpu


def _both(spec, params):
    """(noalloc result, launch-with-workspace result) of one fusion."""
    import torch
    import compiler_hlo_amd as H
    f = H.Fusion(spec.nodes)
    dev = [to_device(p) for p in params]
    stream = torch.cuda.current_stream()
    rn = spec.nodes[-1]
    ref = f(*dev)                        # hf_fusion_launch, workspace from torch
    out = torch.empty_like(ref)
    out.fill_(float("nan") if out.is_floating_point() else -1)
    torch.cuda.synchronize()
    f.launch_noalloc_ptrs([d.data_ptr() for d in dev], out.data_ptr(), stream.cuda_stream)
    torch.cuda.synchronize()
    return from_device(out, rn["dtype"]), from_device(ref, rn["dtype"]), f


def test_noalloc_matches_launch_on_two_calls_second_smaller():
    import torch
    print("noalloc: column reduce f32[8192,4096] max", flush=True)
    spec, params, _ = W.column_reduce_max_f32(8192, 4096, seed=501)
    got, ref, f = _both(spec, params)
    assert f.workspace_bytes > 0
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert_bitexact(got, oracle.evaluate(spec.nodes, params), "f32")
    print("noalloc: column reduce f32[2048,1024] max (smaller)", flush=True)
    spec2, params2, _ = W.column_reduce_max_f32(2048, 1024, seed=502)
    got2, ref2, f2 = _both(spec2, params2)
    assert 0 < f2.workspace_bytes < f.workspace_bytes
    assert np.array_equal(got2.view(np.uint32), ref2.view(np.uint32))
    assert_bitexact(got2, oracle.evaluate(spec2.nodes, params2), "f32")
    torch.cuda.synchronize()


def test_noalloc_sum_and_argmax_and_no_workspace():
    """A column sum (integer-valued, exact in any order), a column argmax
    (value and index partials in the scratch) and a loop that needs no
    workspace."""
    g = W.rng(503)
    s = W.Spec()
    p = s.parameter(0, "f32", [6000, 700])
    s.reduce(p, [0], "add", 0.0, "f32", [700])
    x = g.integers(-4, 4, 6000 * 700, endpoint=True).astype(np.float32)
    got, ref, f = _both(s, [x])
    assert f.plan()["hero"] == "column_reduce" and f.workspace_bytes > 0
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "f32")
    s = W.Spec()
    p = s.parameter(0, "f32", [5000, 300])
    s.argmax(p, 0, [5000, 300])
    x = W.normal_f32(g, 5000 * 300)
    got, ref, f = _both(s, [x])
    assert f.plan()["hero"] == "column_reduce" and f.workspace_bytes > 0
    assert np.array_equal(got, ref)
    assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "s32")
    spec, params, _ = W.quant_dequant_bias_requant(300, 4096, seed=504)
    got, ref, f = _both(spec, params)
    assert f.workspace_bytes == 0
    assert np.array_equal(got, ref)


def test_noalloc_split_rows():
    """Row reduces of a few long rows, split into segments whose partials
    (for argmax, values and indices) go to the scratch: an integer-valued
    sum of f32[16,1048576] (exact in any order), then the argmax of the
    smaller f32[4,262144]."""
    g = W.rng(505)
    print("noalloc: row sum f32[16,1048576] split", flush=True)
    s = W.Spec()
    p = s.parameter(0, "f32", [16, 1048576])
    s.reduce(p, [1], "add", 0.0, "f32", [16])
    x = g.integers(-4, 4, 16 * 1048576, endpoint=True).astype(np.float32)
    got, ref, f = _both(s, [x])
    assert f.plan()["hero"] == "row_reduce" and f.workspace_bytes > 0
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "f32")
    print("noalloc: row argmax f32[4,262144] split", flush=True)
    s = W.Spec()
    p = s.parameter(0, "f32", [4, 262144])
    s.argmax(p, 1, [4, 262144])
    x = W.normal_f32(g, 4 * 262144)
    got, ref, f = _both(s, [x])
    assert f.plan()["hero"] == "row_reduce" and f.workspace_bytes > 0
    assert np.array_equal(got, ref)
    assert_bitexact(got, oracle.evaluate(s.nodes, [x]), "s32")


def test_noalloc_rejects_a_workspace_beyond_the_scratch(monkeypatch):
    import torch
    import compiler_hlo_amd as H
    monkeypatch.setenv("HF_COL_WGS", "1000000")  # many segments: a large workspace
    s = W.Spec()
    p = s.parameter(0, "f32", [65536, 2048])
    s.reduce(p, [0], "max", float("-inf"), "f32", [2048])
    f = H.Fusion(s.nodes)
    assert f.workspace_bytes > H.SCRATCH_BYTES
    x = torch.zeros(65536 * 2048, dtype=torch.float32, device="cuda")
    out = torch.empty(2048, dtype=torch.float32, device="cuda")
    with pytest.raises(H.FusionError) as e:
        f.launch_noalloc_ptrs([x.data_ptr()], out.data_ptr())
    assert e.value.status == "HF_ERR_UNSUPPORTED" and "scratch" in e.value.message
