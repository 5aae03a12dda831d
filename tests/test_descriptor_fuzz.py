"""hf_fusion_create on mutated descriptors (CPU): valid fusions with one to
three fields set to random, mostly out-of-range, values.  Every call returns
HF_OK, HF_ERR_INVALID or HF_ERR_UNSUPPORTED -- never a crash -- and every
descriptor that plans also generates and compiles.  Larger runs of the same
mutator were clean under AddressSanitizer and UBSan."""
import bench as B
import descfuzz as D
import test_random_fusions as T


def _bases():
    out = []
    nodes_list = [mk(**kw)[0].nodes for mk, kw, _ in B.workload_makers().values()]
    nodes_list += [T._make(seed, series)[0].nodes for seed, series in T._cases()[::16]]
    for nodes in nodes_list:
        n_params = 1 + max([nd.get("param", -1) for nd in nodes if nd["op"] == "parameter"], default=-1)
        out.append((nodes, len(nodes) - 1, n_params))
    return out


def test_mutated_descriptors_never_crash():
    counts, compiled = D.run(_bases(), 3000, seed=7, compile_every=300)
    assert set(counts) <= {0, 1, 2}
    assert counts.get(0, 0) > 500 and counts.get(1, 0) > 500, counts
    assert compiled >= 3


def test_reduce_with_missing_operands_is_invalid():
    """The mutation that once crashed create: a reduce node with no operands
    (its operand type was read before the count was checked)."""
    import compiler_hlo_amd as H
    import pytest
    import workloads as W
    s = W.Spec()
    p = s.parameter(0, "f32", [4, 8])
    s.reduce(p, [1], "add", 0.0, "f32", [4])
    s.nodes[1]["operands"] = []
    with pytest.raises(H.FusionError) as e:
        H.Fusion(s.nodes, mode="plan")
    assert e.value.status == "HF_ERR_INVALID" and "operand" in str(e.value)
