"""Pins of the oracle's cost model and partition-vector search (CPU only).

Costs are checked against hand-worked values of the section 3.1 formula; the
dynamic programme of section 3.2 against exhaustive search over every joint
assignment on small EinGraphs; the candidate sets against the pruning rules
(at least P tasks, a multiple of P, power-of-two parts dividing the extents).
"""
import json
import os

import pytest

from oracle import chooser

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_costs():
    g = json.load(open(os.path.join(GOLDEN, "chooser_costs.json")))
    for c in g["cases"]:
        assert chooser.einsum_cost(c["spec"], c["bounds"], c["d"]) == c["cost"], c["_work"]


def _softmax_node(bounds):
    return chooser.Node("Attn", "hst->hst", dict(bounds), ["S"], kind="softmax")


def test_hand_worked_softmax_node_costs():
    """The softmax node (LSE = lse_t S, then Attn = exp(S - LSE), one d over
    h, s, t) costs the sum of its two EinSums' terms; worked by hand."""
    g = json.load(open(os.path.join(GOLDEN, "chooser_costs.json")))
    assert len(g["softmax_cases"]) >= 4
    for c in g["softmax_cases"]:
        assert chooser.node_cost(_softmax_node(c["bounds"]), c["d"]) == c["cost"], c["_work"]


def test_softmax_node_best_blocking_closed_form():
    """2*H*S*T + (2*d_t - 1)*H*S is least at d_t = 1: for P = 8 on h=2, s=4, t=4
    the search must pick d_t = 1, h and s cut 8 ways, at cost 2*32 + 8 = 72."""
    node = _softmax_node({"h": 2, "s": 4, "t": 4})
    total, asg = chooser.dp([node], 8)
    assert total == 72
    assert asg["Attn"]["t"] == 1 and asg["Attn"]["h"] * asg["Attn"]["s"] == 8
    assert chooser.exhaustive([node], 8)[0] == 72


def test_candidates_respect_pruning_rules():
    node = chooser.Node("n", "ij,jk->ik", {"i": 24, "j": 16, "k": 8}, ["@x", "@y"])
    cands = chooser.candidates(node, 16)
    assert cands
    for d in cands:
        n = d["i"] * d["j"] * d["k"]
        assert n >= 16 and n % 16 == 0
        for c, v in d.items():
            assert v & (v - 1) == 0 and node.bounds[c] % v == 0
    # 24 has power-of-two divisors 1, 2, 4, 8 only
    assert {d["i"] for d in cands} <= {1, 2, 4, 8}
    assert chooser.candidates(chooser.Node("m", "ij,jk->ik", {"i": 2, "j": 2, "k": 2}, []), 16) == []


def _chain():
    b = {"i": 8, "j": 8, "k": 8, "l": 8}
    return [chooser.Node("A", "ij,jk->ik", b, ["@X", "@Y"]),
            chooser.Node("B", "ik,kl->il", b, ["A", "@W"])]


def _fork():
    g = chooser.mha_graph(s=4, a=4, h=2, dh=2)
    keep = {"Q_proj", "K_proj", "Scores"}
    return [n for n in g if n.name in keep]


def _softmax_chain():
    g = chooser.mha_graph(s=4, a=4, h=2, dh=4)
    keep = {"Scores", "Attn", "O"}
    nodes = [n for n in g if n.name in keep]
    for n in nodes:
        n.inputs = [s if s in keep else "@" + s for s in n.inputs]
    return nodes


@pytest.mark.parametrize("make,p", [(_chain, 4), (_chain, 16), (_fork, 4), (_softmax_chain, 8)])
def test_dp_equals_exhaustive_search(make, p):
    nodes = make()
    best, _ = chooser.exhaustive(nodes, p)
    total, asg = chooser.dp(nodes, p)
    assert total == best
    assert chooser.graph_cost(nodes, asg) == best


def test_repartition_term():
    nodes = _chain()
    a, b = nodes
    same = {"i": 2, "j": 1, "k": 4, "l": 1}
    # producer output [i,k] blocked (2,4); consumer reads it as [i,k] too
    assert chooser.repartition_cost(a, same, b, 0, same) == 0
    other = dict(same, k=2)
    assert chooser.repartition_cost(a, same, b, 0, other) == 64


def test_mha_graph_dp_mid_size():
    nodes = chooser.mha_graph(s=32, a=32, h=4, dh=8)
    total, asg = chooser.dp(nodes, 16)
    assert set(asg) == {n.name for n in nodes}
    assert chooser.graph_cost(nodes, asg) == total
    for n in nodes:
        d = asg[n.name]
        assert chooser.n_tasks(n, d) >= 16 and chooser.n_tasks(n, d) % 16 == 0
