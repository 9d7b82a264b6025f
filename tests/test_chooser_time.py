"""The chooser's measured time model (tra_choose_ex / TRA_GRAPH_CHOOSE_TIME), CPU only.

The model's pieces are read through the ABI (tra_predict_ns of a node's plan
under a candidate d, tra_predict_repartition_ns of a tensor); the tests check
that the dynamic programme finds the exact minimum of their sum over every
assignment of partition vectors (brute force on a small attention chain), and
what the model implies on the full attention layer: one blocking throughout,
so no repartition at all.
"""
import itertools

import numpy as np
import pytest

import tensor_relational_algebra_amd as tra
from tensor_relational_algebra_amd import workloads as wl

CHAIN = "\n".join([
    "S einsum shd,thd->hst s=8,t=8,h=2,d=4 @Q,@K in=bf16 out=f32 scale=0.5",
    "A softmax hst->hst h=2,s=8,t=8 S in=f32 out=bf16",
    "O einsum hst,thd->shd h=2,s=8,t=8,d=4 A,@V in=bf16 out=bf16",
])
B = {"s": 8, "t": 8, "h": 2, "d": 4}


def _cands(labels):
    opts = [[k for k in (1, 2, 4, 8, 16) if k <= B[c] and B[c] % k == 0] for c in labels]
    return [dict(zip(labels, v)) for v in itertools.product(*opts)]


def _rep(labels, dtype):
    return tra.tra_predict_repartition_ns([B[c] for c in labels], dtype)


def _node_ns(spec, d, idt, odt, scale, leaves, root_out=None):
    p = tra.tra_plan(spec, B, d, "mul", "sum", idt, odt, scale)
    ns = tra.tra_predict_ns(p)
    for lab, dt in leaves:                       # graph inputs arrive dense
        if any(d[c] != 1 for c in lab):
            ns += _rep(lab, dt)
    if root_out and any(d[c] != 1 for c in root_out[0]):
        ns += _rep(*root_out)                      # the output is returned dense
    return ns


def _softmax_ns(d):
    p1 = tra.tra_plan("hst->hs", B, d, "ident", "lse", "f32", "f32")
    p2 = tra.tra_plan("hst,hs->hst", B, d, "exp_sub", "none", "f32", "bf16")
    return tra.tra_predict_ns(p1) + tra.tra_predict_ns(p2)


def test_dp_finds_the_exact_minimum_of_the_time_model():
    cs = _cands(tra.tra_canonical_labels("shd,thd->hst"))
    ca = _cands("hst")
    co = _cands(tra.tra_canonical_labels("hst,thd->shd"))
    ns_s = np.array([_node_ns("shd,thd->hst", d, "bf16", "f32", 0.5, [("shd", "bf16"), ("thd", "bf16")]) for d in cs])
    ns_a = np.array([_softmax_ns(d) for d in ca])
    ns_o = np.array([_node_ns("hst,thd->shd", d, "bf16", "bf16", 1.0, [("thd", "bf16")], ("shd", "bf16"))
                     for d in co])
    blk = lambda d: tuple(d[c] for c in "hst")
    rep_s = _rep("hst", "f32")
    rep_a = _rep("hst", "bf16")
    e_sa = np.array([[0 if blk(x) == blk(y) else rep_s for y in ca] for x in cs])
    e_ao = np.array([[0 if blk(x) == blk(y) else rep_a for y in co] for x in ca])
    total = ns_s[:, None, None] + e_sa[:, :, None] + ns_a[None, :, None] + e_ao[None, :, :] + ns_o[None, None, :]
    best = int(total.min())
    ds, cost = tra.tra_choose(CHAIN, 1, tra.CHOOSE_TIME)
    assert cost == best
    i = cs.index(dict(zip(tra.tra_canonical_labels("shd,thd->hst"), ds[0])))
    j = ca.index(dict(zip("hst", ds[1])))
    k = co.index(dict(zip(tra.tra_canonical_labels("hst,thd->shd"), ds[2])))
    assert int(total[i, j, k]) == best


def test_full_attention_layer_keeps_one_blocking():
    desc = wl.MHA.graph_desc()
    g = tra.tra_graph_plan_ex(desc, 256, None, tra.GRAPH_CHOOSE_TIME)
    assert g.info.n_repartitions == 0
    ds, cost = tra.tra_choose(desc, 256, tra.CHOOSE_TIME)
    assert cost == g.info.cost
    assert all(x == 1 for d in ds for x in d)
    # the pages' numbers-moved choice, priced by the time model, costs more: the
    # same kernels plus its repartitions
    g0 = tra.tra_graph_plan_ex(desc, 256, None, 0)
    assert g0.info.n_repartitions > 0


def test_time_model_pieces_and_errors():
    p = tra.tra_plan("sa,ahd->shd", {"s": 4096, "a": 4096, "h": 32, "d": 128},
                     {"s": 1, "a": 1, "h": 1, "d": 1}, "mul", "sum", "bf16", "bf16")
    assert p.kernel == "mfma_bf16" and p.info.tile == 4
    ns = tra.tra_predict_ns(p)
    assert 100_000 < ns < 200_000          # ~2 * 4096^3 * 32 * 128 / 4096 flop at ~0.97 PFLOP/s
    r = tra.tra_predict_repartition_ns([16384, 8192], "f32")
    assert 150_000 < r < 250_000
    assert tra.tra_predict_repartition_ns([0, 5], "f32") == 0
    with pytest.raises(tra.TraError) as e:
        tra.tra_predict_repartition_ns([4, -1], "f32")
    assert e.value.code == -4
    with pytest.raises(tra.TraError) as e:
        tra.tra_choose(CHAIN, 1, 2)
    assert e.value.code == -7


def test_row_reduce_needs_both_operands_contiguous_along_the_run():
    b = {"i": 2000, "j": 1000, "k": 2000}
    d = {"i": 1, "j": 1, "k": 1}
    assert tra.tra_plan("ij,kj->ik", b, d, "mul", "sum", "f32", "f32").kernel == "rowreduce"
    assert tra.tra_plan("ij,jk->ik", b, d, "mul", "sum", "f32", "f32").kernel == "generic"
    assert tra.tra_plan("hst->hs", {"h": 2, "s": 8, "t": 256}, {"h": 1, "s": 1, "t": 1},
                        "ident", "lse", "f32", "f32").kernel == "rowreduce"
