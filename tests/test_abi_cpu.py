"""CPU-only checks of the C-ABI library: it loads, exports every entry point
include/tra.h declares, plans without a GPU, rejects every invalid argument
with its documented status, and its chooser agrees with the oracle's cost
model and dynamic programme.  No compute kernel is launched here.
"""
import json
import os
import re

import pytest

import tensor_relational_algebra_amd as tra
from oracle import chooser
from tensor_relational_algebra_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")

# No skip when the library is absent: it is built here (host compile and a gfx950
# cross-compile, no GPU needed), and a failed build fails every test below.
if not os.path.exists(_binding.LIB_PATH):
    from tensor_relational_algebra_amd import build as _tra_build
    _tra_build.build()


def _declared():
    txt = open(os.path.join(ROOT, "include", "tra.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(tra_[a-z_]+)\s*\(", txt)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert "tra_plan" in names and "tra_execute" in names and "tra_repartition" in names
    L = tra.lib()
    for n in names:
        assert hasattr(L, n), f"{n} declared in tra.h but not exported"


def test_canonical_labels_and_operand_form():
    assert tra.tra_canonical_labels("ij,jk->ik") == "ikj"
    assert tra.tra_canonical_labels("abef,cfed->abcd") == "abcdef"
    assert tra.tra_canonical_labels("shd,ahd->sa") == "sahd"
    assert tra.tra_canonical_labels("hst->hs") == "hst"
    # the page's per-operand matmul vector [d_i, d_j(X), d_j(Y), d_k]
    assert tra.tra_d_from_operand_form("ij,jk->ik", [4, 1, 1, 4]) == [4, 4, 1]
    assert tra.tra_d_from_operand_form("ij,jk->ik", [1, 4, 4, 1]) == [1, 1, 4]
    with pytest.raises(tra.TraError) as e:
        tra.tra_d_from_operand_form("ij,jk->ik", [1, 2, 4, 1])
    assert e.value.code == -5


def test_plan_task_structure_matches_the_worked_examples():
    g = json.load(open(os.path.join(GOLDEN, "matmul_partition_examples.json")))
    for c in g["cases"]:
        d = tra.tra_d_from_operand_form("ij,jk->ik", c["d4"])
        p = tra.tra_plan("ij,jk->ik", [256, 256, 256], d, "mul", "sum", "i32", "i32")
        assert (p.info.n_tasks, p.info.n_groups, p.info.n_agg) == (c["N"], c["G"], c["n_agg"])
        assert p.info.z_elems == 65536


def test_kernel_family_choice():
    p = tra.tra_plan("ij,jk->ik", {"i": 16384, "j": 8192, "k": 8192}, {"i": 16, "j": 4, "k": 4},
                     "mul", "sum", "bf16", "f32")
    assert p.kernel == "mfma_bf16" and p.info.workspace_bytes == 0
    p = tra.tra_plan("abef,cfed->abcd", dict(a=64, b=64, c=64, d=64, e=32, f=32),
                     dict(a=2, b=2, c=2, d=2, e=4, f=4), "mul", "sum", "bf16", "f32")
    assert p.kernel == "mfma_bf16" and p.info.n_tasks == 256 and p.info.n_agg == 16
    p = tra.tra_plan("ij,jk->ik", {"i": 8192, "j": 256, "k": 8192}, {"i": 16, "j": 1, "k": 16},
                     "sqdiff", "sum", "f32", "f32")
    assert p.kernel == "valu_tile"
    p = tra.tra_plan("ij,jk->ik", {"i": 8192, "j": 256, "k": 8192}, {"i": 16, "j": 1, "k": 16},
                     "add", "max", "i32", "i32")
    # int32 max-plus: the packed 16-bit variant, with 256 range-check flag words
    # in the workspace
    assert p.kernel == "valu_tile" and p.info.tile == 1 and p.info.workspace_bytes == 1024
    p = tra.tra_plan("ij,jk->ik", {"i": 256, "j": 1024, "k": 256}, {"i": 1, "j": 1, "k": 1}, "add", "min", "i32",
                     "i32")
    assert p.info.tile == 1 and p.info.agg_split > 1
    assert p.info.workspace_bytes == p.info.agg_split * 65536 * 4 + 1024
    for idt, join, agg in (("f32", "add", "max"), ("f32", "sqdiff", "sum"), ("i32", "mul", "sum")):
        p = tra.tra_plan("ij,jk->ik", [256, 256, 256], [1, 1, 1], join, agg, idt, idt)
        assert p.kernel == "valu_tile" and p.info.tile == 0
    p = tra.tra_plan("hst->hs", {"h": 32, "s": 4096, "t": 4096}, {"h": 32, "s": 8, "t": 1},
                     "ident", "lse", "f32", "f32")
    assert p.kernel == "rowreduce"
    p = tra.tra_plan("hst,hs->hst", {"h": 32, "s": 4096, "t": 4096}, {"h": 32, "s": 8, "t": 1},
                     "exp_sub", "none", "f32", "bf16")
    assert p.kernel == "elemwise"
    # small partitioned matmul: one output tile per group, so the contracted
    # range is split over workgroups with a workspace
    p = tra.tra_plan("ij,jk->ik", [256, 256, 256], [1, 1, 4], "mul", "sum", "f32", "f32")
    assert p.kernel == "valu_tile" and p.info.agg_split > 1
    assert p.info.workspace_bytes == p.info.agg_split * 65536 * 4


@pytest.mark.parametrize("args,code", [
    (("ij,jk-ik", [2, 2, 2], [1, 1, 1]), -2),                      # no arrow
    (("ij,jk,kl->il", [2, 2, 2, 2], [1, 1, 1, 1]), -2),            # three operands
    (("i1,jk->ik", [2, 2, 2], [1, 1, 1]), -2),                     # non-letter label
    (("ii,jk->ik", [2, 2, 2], [1, 1, 1]), -3),                     # repeated label
    (("ij,jk->iq", [2, 2, 2], [1, 1, 1]), -3),                     # output label in no operand
    (("ij,jk->ik", [2, 2], [1, 1]), -5),                           # wrong label count
    (("ij,jk->ik", [4, 4, 4], [3, 1, 1]), -4),                     # d does not divide
    (("ij,jk->ik", [4, 4, 4], [0, 1, 1]), -4),                     # d < 1
    (("ij,jk->ik", [4, -1, 4], [1, 1, 1]), -4),                    # extent < 0
    (("ij,jk->ik", [4, 0, 4], [1, 2, 1]), -4),                     # a zero extent takes d = 1
])
def test_plan_validation_errors(args, code):
    spec, b, d = args
    with pytest.raises(tra.TraError) as e:
        tra.tra_plan(spec, b, d)
    assert e.value.code == code
    assert tra.lib().tra_last_error().decode()


def test_plan_op_and_dtype_errors():
    b, d = [8, 8, 8], [1, 1, 1]
    cases = [
        (dict(join="mul", agg="none"), -7),                          # contracted labels, no aggregate
        (dict(join="ident", agg="sum"), -7),                         # ident with two operands
        (dict(join="exp_sub", agg="sum", in_dtype="i32", out_dtype="i32"), -6),
        (dict(join="mul", agg="lse", in_dtype="i32", out_dtype="i32"), -6),
        (dict(join="mul", agg="sum", in_dtype="i32", out_dtype="f32"), -6),
        (dict(join="mul", agg="sum", in_dtype="i32", out_dtype="i32", post_scale=2.0), -7),
    ]
    for kw, code in cases:
        with pytest.raises(tra.TraError) as e:
            tra.tra_plan("ij,jk->ik", b, d, **kw)
        assert e.value.code == code, kw
    with pytest.raises(tra.TraError) as e:
        tra.tra_plan("ij->i", [4, 4], [1, 1], "mul", "sum")        # binary join, one operand
    assert e.value.code == -7
    with pytest.raises(tra.TraError) as e:
        tra.tra_plan("ij,jk->ik", [65536, 65536, 2], [1, 1, 1])    # 2^32 elements
    assert e.value.code == -12


def test_execute_and_repartition_host_errors():
    import ctypes
    L = tra.lib()
    p = tra.tra_plan("ij,jk->ik", [256, 256, 256], [1, 1, 4], "mul", "sum", "f32", "f32")
    assert L.tra_execute(None, 16, 16, 16, None, 0, None) == -1
    assert L.tra_execute(p.handle, None, 16, 16, None, 0, None) == -1
    assert L.tra_execute(p.handle, 17, 16, 16, None, 0, None) == -9           # misaligned
    assert L.tra_execute(p.handle, 16, 16, 16, None, 0, None) == -8           # workspace missing
    assert L.tra_execute(p.handle, 16, 16, 16, 16, 8, None) == -8             # workspace too small
    I64, I32 = ctypes.c_int64, ctypes.c_int32
    b = (I64 * 2)(8, 8)
    d1 = (I32 * 2)(1, 1)
    d3 = (I32 * 2)(3, 1)
    assert L.tra_repartition(b, 2, d1, d3, 0, 16, 32, None) == -4            # 3 does not divide 8
    assert L.tra_repartition(b, 0, d1, d1, 0, 16, 32, None) == -5            # rank 0
    assert L.tra_repartition(b, 2, d1, d1, 7, 16, 32, None) == -6            # bad dtype
    assert L.tra_repartition(b, 2, d1, d1, 0, 18, 32, None) == -9            # misaligned
    assert L.tra_repartition(b, 2, None, d1, 0, 16, 32, None) == -1
    b6 = (I64 * 1)(6)
    d2 = (I32 * 1)(2)
    d3b = (I32 * 1)(3)
    assert L.tra_repartition(b6, 1, d2, d3b, 0, 16, 32, None) == -4          # blocks 3 and 2 do not nest


def test_cost_matches_hand_worked_values():
    g = json.load(open(os.path.join(GOLDEN, "chooser_costs.json")))
    for c in g["cases"]:
        assert tra.tra_cost(c["spec"], c["bounds"], c["d"]) == c["cost"], c["_work"]


def test_probe_argument_errors():
    L = tra.lib()
    for distinct in (0, 1):
        assert L.tra_probe_mfma_loop(0, 1, distinct, 0x1000, None) == -7
        assert L.tra_probe_mfma_loop(1, 0, distinct, 0x1000, None) == -7
        assert L.tra_probe_mfma_loop(1, 1, distinct, None, None) == -1


def test_softmax_node_cost_matches_hand_worked_values():
    """The library's chooser on one softmax node, at a P that leaves exactly one
    admissible d (every element its own block), returns the hand-worked cost of
    that d; at full size its minimum (d_t = 1) is the hand-worked cost of a
    d_t = 1 case."""
    g = json.load(open(os.path.join(GOLDEN, "chooser_costs.json")))
    only = [c for c in g["softmax_cases"] if all(c["d"][k] == c["bounds"][k] for k in "hst")]
    assert len(only) >= 2
    for c in only:
        b = c["bounds"]
        desc = f"Attn softmax hst->hst h={b['h']},s={b['s']},t={b['t']} @S in=f32 out=bf16"
        ds, cost = tra.tra_choose(desc, b["h"] * b["s"] * b["t"])
        assert ds == [[b["h"], b["s"], b["t"]]]
        assert cost == c["cost"], c["_work"]
    full = [c for c in g["softmax_cases"] if c["bounds"]["t"] == 4096 and c["d"]["t"] == 1][0]
    _, cost = tra.tra_choose("Attn softmax hst->hst h=32,s=4096,t=4096 @S in=f32 out=bf16", 256)
    assert cost == full["cost"], full["_work"]


def _desc(nodes):
    lines = []
    for n in nodes:
        b = ",".join(f"{k}={v}" for k, v in n.bounds.items())
        lines.append(f"{n.name} {n.kind} {n.spec} {b} {','.join(n.inputs)}")
    return "\n".join(lines)


def _check_against_oracle(nodes, p):
    want_cost, want = chooser.dp(nodes, p)
    got, cost = tra.tra_choose(_desc(nodes), p)
    assert cost == want_cost
    for n, dv in zip(nodes, got):
        assert dv == [want[n.name][c] for c in n.labels()], n.name
    asg = {n.name: dict(zip(n.labels(), dv)) for n, dv in zip(nodes, got)}
    assert chooser.graph_cost(nodes, asg) == cost


def test_choose_equals_oracle_dp_small_graphs():
    b = {"i": 8, "j": 8, "k": 8, "l": 8}
    chain = [chooser.Node("A", "ij,jk->ik", b, ["@X", "@Y"]), chooser.Node("B", "ik,kl->il", b, ["A", "@W"])]
    for p in (4, 16):
        _check_against_oracle(chain, p)
    _check_against_oracle(chooser.mha_graph(s=32, a=32, h=4, dh=8), 16)


def test_choose_full_attention_graph():
    nodes = chooser.mha_graph(s=4096, a=4096, h=32, dh=128)
    got, cost = tra.tra_choose(_desc(nodes), 256)
    asg = {n.name: dict(zip(n.labels(), dv)) for n, dv in zip(nodes, got)}
    assert chooser.graph_cost(nodes, asg) == cost
    for n in nodes:
        t = chooser.n_tasks(n, asg[n.name])
        assert t >= 256 and t % 256 == 0
        for c, v in asg[n.name].items():
            assert v & (v - 1) == 0 and n.bounds[c] % v == 0


def test_choose_errors():
    with pytest.raises(tra.TraError) as e:
        tra.tra_choose("A einsum ij,jk->ik i=2,j=2,k=2 @X,@Y", 64)
    assert e.value.code == -11
    with pytest.raises(tra.TraError) as e:
        tra.tra_choose("A einsum ij,jk->ik i=2,j=2 @X,@Y", 1)
    assert e.value.code == -13
    with pytest.raises(tra.TraError) as e:
        tra.tra_choose("A einsum ij,jk->ik i=2,j=2,k=2 @X,B", 1)
    assert e.value.code == -13


def test_graph_plan_uses_the_chooser_and_lays_out_the_workspace():
    from tensor_relational_algebra_amd import workloads as wl
    for case, p in ((wl.MHA, 256), (wl.MHA_SMALL, 16)):
        desc = case.graph_desc()
        g = tra.tra_graph_plan(desc, p)
        ds, cost = tra.tra_choose(desc, p)
        assert g.info.cost == cost and g.info.n_nodes == 7
        assert [g.node_d(i) for i in range(7)] == ds
        assert [n for n, _, _ in g.leaves] == ["Q", "W_Q", "K", "W_K", "V", "W_V", "W_O"]
        assert g.info.out_elems == case.s * case.a
        assert g.info.workspace_bytes > 0
    # explicit d: all ones everywhere needs no repartition between nodes
    desc = wl.MHA_SMALL.graph_desc()
    ones = [1] * sum(len(tra.tra_canonical_labels(l.split()[2])) if l.split()[1] == "einsum" else 3
                     for l in desc.splitlines())
    g = tra.tra_graph_plan(desc, 1, ones)
    assert g.info.n_repartitions == 0


def test_graph_node_output_locations():
    """Where each node leaves its output in the workspace (host only): inside
    the workspace, the node's output size and dtype, a logsumexp only for the
    softmax node, and no output for nodes folded into a fused chain."""
    import ctypes
    import torch
    from tensor_relational_algebra_amd import workloads as wl
    case = wl.MHA_SMALL
    g = tra.tra_graph_plan(case.graph_desc(), 16)
    ws = torch.empty(g.info.workspace_bytes, dtype=torch.uint8)
    sizes = {"Q_proj": 128 * 4 * 32, "K_proj": 128 * 4 * 32, "V_proj": 128 * 4 * 32, "Scores": 4 * 128 * 128,
             "Attn": 4 * 128 * 128, "O": 128 * 4 * 32, "Output": 128 * 128}
    dtypes = {"Scores": torch.float32, "Output": torch.float32}
    for i, name in enumerate(sizes):
        rel, lse = g.node_output(i, ws)
        assert rel.numel() == sizes[name] and rel.dtype == dtypes.get(name, torch.bfloat16)
        assert (lse is not None) == (name == "Attn")
        if lse is not None:
            assert lse.numel() == 4 * 128 and lse.dtype == torch.float32
    gf = tra.tra_graph_plan_ex(case.graph_desc(), 16, None, tra.GRAPH_FUSE_ATTENTION)
    wf = torch.empty(gf.info.workspace_bytes, dtype=torch.uint8)
    for i in (3, 4):
        with pytest.raises(tra.TraError) as e:
            gf.node_output(i, wf)
        assert e.value.code == -7
    assert gf.node_output(5, wf)[0].numel() == sizes["O"]
    L = tra.lib()
    o, n, dt, lo, ln = ctypes.c_size_t(), ctypes.c_int64(), ctypes.c_int32(), ctypes.c_size_t(), ctypes.c_int64()
    assert L.tra_graph_node_output(g.handle, 7, ctypes.byref(o), ctypes.byref(n), ctypes.byref(dt),
                                   ctypes.byref(lo), ctypes.byref(ln)) == -13
    assert L.tra_graph_node_output(g.handle, 0, None, ctypes.byref(n), ctypes.byref(dt), ctypes.byref(lo),
                                   ctypes.byref(ln)) == -1


def test_graph_plan_errors():
    with pytest.raises(tra.TraError) as e:
        tra.tra_graph_plan("A softmax hst->hst h=2,s=2,t=2 @S in=bf16 out=bf16", 1)
    assert e.value.code == -13
    with pytest.raises(tra.TraError) as e:
        tra.tra_graph_plan("A einsum ij,jk->ik i=4,j=4,k=4 @X,@Y wat=1", 1)
    assert e.value.code == -13
    with pytest.raises(tra.TraError) as e:
        tra.tra_graph_plan("A einsum ij,jk->ik i=4,j=4,k=4 @X,@Y", 1, [1, 1])
    assert e.value.code == -5


def test_graph_plan_fuses_the_attention_chain():
    from tensor_relational_algebra_amd import workloads as wl
    for case, p in ((wl.MHA, 256), (wl.MHA_SMALL, 16), (wl.MhaCase(s=256, a=256, h=8, dh=64), 16)):
        desc = case.graph_desc()
        g0 = tra.tra_graph_plan(desc, p)
        g1 = tra.tra_graph_plan_ex(desc, p, None, tra.GRAPH_FUSE_ATTENTION)
        assert g0.info.n_fused == 0 and g1.info.n_fused == 1
        # same chooser result; the scores and softmax buffers are gone
        assert g1.info.cost == g0.info.cost
        assert [g1.node_d(i) for i in range(7)] == [g0.node_d(i) for i in range(7)]
        assert [n for n, _, _ in g1.leaves] == [n for n, _, _ in g0.leaves]
        s, h = case.s, case.h
        # unfused, S (fp32) and A (bf16) are both live at the softmax step; fused,
        # neither exists (at small sizes the peak may sit at another step)
        assert g0.info.workspace_bytes >= h * s * s * (4 + 2)
        assert g1.info.workspace_bytes <= g0.info.workspace_bytes
        if case is wl.MHA:
            assert g1.info.workspace_bytes <= g0.info.workspace_bytes - h * s * s * 4
    # a head dimension the kernel is not built for, and a softmax read twice, stay unfused
    g = tra.tra_graph_plan_ex(wl.MhaCase(s=128, a=128, h=4, dh=48).graph_desc(), 16, None,
                              tra.GRAPH_FUSE_ATTENTION)
    assert g.info.n_fused == 0
    lines = wl.MHA_SMALL.graph_desc().splitlines()
    lines[5] += " scale=0.5"   # a scaled weighted sum is not the chain the kernel computes
    assert lines[5].startswith("O einsum")
    g = tra.tra_graph_plan_ex("\n".join(lines), 16, None, tra.GRAPH_FUSE_ATTENTION)
    assert g.info.n_fused == 0
    with pytest.raises(tra.TraError) as e:
        tra.tra_graph_plan_ex(wl.MHA_SMALL.graph_desc(), 16, None, 8)
    assert e.value.code == -7


def test_graph_plan_overlapped_copies_layout():
    """TRA_GRAPH_OVERLAP_COPIES keeps the chooser's blockings; a graph input's
    copy is live from the first step, so on the full attention layer (every
    input copied into its node's blocking) all seven input copies are live at
    once and the workspace holds at least their bytes."""
    from tensor_relational_algebra_amd import workloads as wl
    desc = wl.MHA.graph_desc()
    g0 = tra.tra_graph_plan(desc, 256)
    g1 = tra.tra_graph_plan_ex(desc, 256, None, tra.GRAPH_OVERLAP_COPIES)
    assert [g1.node_d(i) for i in range(7)] == [g0.node_d(i) for i in range(7)]
    assert g1.info.n_repartitions == g0.info.n_repartitions and g1.info.cost == g0.info.cost
    leaf_bytes = sum(n * 2 for _, n, _ in g1.leaves)      # bf16 inputs
    assert g1.info.workspace_bytes >= g0.info.workspace_bytes
    assert g1.info.workspace_bytes >= leaf_bytes


def test_empty_tensors_plan():
    # an empty output: nothing to run
    p = tra.tra_plan("ij,jk->ik", {"i": 0, "j": 4, "k": 5}, {"i": 1, "j": 1, "k": 1})
    assert p.kernel == "empty" and p.info.z_elems == 0 and p.info.x_elems == 0
    # an empty contracted range: the output is the aggregate's identity (generic kernel, nothing read)
    p = tra.tra_plan("ij,jk->ik", {"i": 3, "j": 0, "k": 5}, {"i": 3, "j": 1, "k": 1}, "add", "max", "i32", "i32")
    assert p.kernel == "generic" and p.info.z_elems == 15 and p.info.x_elems == 0 and p.info.y_elems == 0
    # a zero extent takes d = 1; negative extents are rejected
    with pytest.raises(tra.TraError) as e:
        tra.tra_plan("ij,jk->ik", {"i": 3, "j": 0, "k": 5}, {"i": 1, "j": 2, "k": 1})
    assert e.value.code == -4
    with pytest.raises(tra.TraError) as e:
        tra.tra_plan("ij,jk->ik", {"i": -1, "j": 2, "k": 5}, {"i": 1, "j": 1, "k": 1})
    assert e.value.code == -4


def test_binding_fails_loudly_without_the_library():
    """No fallback: with the shared library absent, the first call raises (in a
    fresh interpreter, so this process's loaded library is not involved)."""
    import subprocess
    import sys
    code = ("import tensor_relational_algebra_amd._binding as B\n"
            "B.LIB_PATH = '/nonexistent/libtra.so'\n"
            "import tensor_relational_algebra_amd as tra\n"
            "try:\n"
            "    tra.tra_plan('ij,jk->ik', {'i': 4, 'j': 4, 'k': 4}, {'i': 1, 'j': 1, 'k': 1})\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.returncode == 0, r.stderr[-2000:]
    assert "raised: libtra is not built" in r.stdout


def test_execute_chain_host_errors():
    """tra_execute_chain validates on the host: plans that do not chain are
    refused before anything is launched."""
    L = tra.lib()
    a = tra.tra_plan("hst,hs->hst", {"h": 2, "s": 4, "t": 256}, {"h": 1, "s": 1, "t": 1}, "sub", "none", "f32",
                     "bf16")
    b = tra.tra_plan("hst,hst->hst", {"h": 2, "s": 4, "t": 256}, {"h": 1, "s": 1, "t": 1}, "mul", "none", "bf16",
                     "bf16")
    assert L.tra_execute_chain(None, b.handle, None, None, None, None, None) == -1
    # b's input dtype must be a's output dtype
    b32 = tra.tra_plan("hst,hst->hst", {"h": 2, "s": 4, "t": 256}, {"h": 1, "s": 1, "t": 1}, "mul", "none", "f32",
                       "bf16")
    assert L.tra_execute_chain(a.handle, b32.handle, 16, 16, 16, 16, None) == -7
    # the outputs must be the same relation (here: another blocking)
    b2 = tra.tra_plan("hst,hst->hst", {"h": 2, "s": 4, "t": 256}, {"h": 2, "s": 1, "t": 1}, "mul", "none", "bf16",
                      "bf16")
    assert L.tra_execute_chain(a.handle, b2.handle, 16, 16, 16, 16, None) == -7
    # not elementwise
    r = tra.tra_plan("hst->hs", {"h": 2, "s": 4, "t": 256}, {"h": 1, "s": 1, "t": 1}, "ident", "lse", "f32", "f32")
    assert L.tra_execute_chain(r.handle, b.handle, 16, 16, 16, 16, None) == -7
    # misaligned pointers
    assert L.tra_execute_chain(a.handle, b.handle, 16, 16, 16, 8, None) == -9


def test_execute_contract_chain_host_errors():
    """tra_execute_contract_chain validates on the host before any launch."""
    L = tra.lib()
    b3 = {"s": 512, "t": 512, "h": 2, "d": 32}
    pc = tra.tra_plan("shd,thd->hst", b3, {c: 1 for c in b3}, "mul", "sum", "bf16", "f32")
    out = {c: b3[c] for c in "hst"}
    pa = tra.tra_plan("hst,hs->hst", out, {c: 1 for c in out}, "sub", "none", "f32", "bf16")
    pb = tra.tra_plan("hst,hst->hst", out, {c: 1 for c in out}, "mul", "none", "bf16", "bf16")
    assert pc.kernel == "mfma_bf16" and pc.info.agg_split == 1
    assert L.tra_execute_contract_chain(None, pa.handle, pb.handle, 16, 16, 16, 16, 16, None) == -1
    # the product must be on the matrix cores (an fp32 product is not)
    p32 = tra.tra_plan("shd,thd->hst", b3, {c: 1 for c in b3}, "mul", "sum", "f32", "f32")
    assert L.tra_execute_contract_chain(p32.handle, pa.handle, pb.handle, 16, 16, 16, 16, 16, None) == -7
    # the steps must share the product's output relation (here: another blocking)
    pb2 = tra.tra_plan("hst,hst->hst", out, {"h": 2, "s": 1, "t": 1}, "mul", "none", "bf16", "bf16")
    assert L.tra_execute_contract_chain(pc.handle, pa.handle, pb2.handle, 16, 16, 16, 16, 16, None) == -7
    # one dtype for the intermediate and the result
    pb3 = tra.tra_plan("hst,hst->hst", out, {c: 1 for c in out}, "mul", "none", "bf16", "f32")
    assert L.tra_execute_contract_chain(pc.handle, pa.handle, pb3.handle, 16, 16, 16, 16, 16, None) == -7
    # a split contracted range is refused
    ps = tra.tra_plan("ik,kj->ij", {"i": 256, "j": 256, "k": 1024}, {"i": 1, "j": 1, "k": 1}, "mul", "sum", "bf16",
                      "f32")
    assert ps.info.agg_split > 1
    sa = tra.tra_plan("ij,i->ij", {"i": 256, "j": 256}, {"i": 1, "j": 1}, "sub", "none", "f32", "f32")
    sb = tra.tra_plan("ij,ij->ij", {"i": 256, "j": 256}, {"i": 1, "j": 1}, "mul", "none", "f32", "f32")
    assert L.tra_execute_contract_chain(ps.handle, sa.handle, sb.handle, 16, 16, 16, 16, 16, None) == -7
    # null and misaligned pointers
    assert L.tra_execute_contract_chain(pc.handle, pa.handle, pb.handle, 16, 16, None, 16, 16, None) == -1
    assert L.tra_execute_contract_chain(pc.handle, pa.handle, pb.handle, 16, 16, 16, 16, 8, None) == -9
