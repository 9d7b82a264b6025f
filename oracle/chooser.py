"""Partition-vector choice by the communication cost model (TEST INFRASTRUCTURE).

Page "EinDecomp：基于爱因斯坦求和与张量关系代数的自动张量并行分解算法":

Section 3.1 (problem statement and cost model).  Every node's TRA plan must
produce at least P independent kernel calls, ideally exactly P.  The cost of
a node under d counts numbers moved, in three parts:
  * join inputs:  P * (|X sub-tensor| + |Y sub-tensor|)
  * aggregation:  (P / n_agg) * (n_agg - 1) * |Z sub-tensor|, n_agg being the
                  number of partitions along the aggregated labels
  * repartition between nodes when the producer's blocking d_u differs from
                  what the consumer's d_v needs.
Section 3.2 (dynamic programming): candidates are pruned to those giving at
least P tasks and whose parts divide the extents;
DP[v][d_v] = min over d_u of (DP[u][d_u] + RepartitionCost(d_u, d_v)) +
Cost(v, d_v); the answer is read back from the output node.
Section 4.3: only powers of two are tried as part counts, and the task count
may be forced to be a multiple of P.

Readings where the page is loose (each is listed in the design notes):
  * "P" inside the two cost terms is the node's own join-task count N.
  * Repartition cost is 0 when, dimension by dimension, the producer's part
    count on its output label equals the consumer's on the matching input
    label; otherwise it is the tensor's element count.  Graph inputs are free.
  * With several predecessors the DP adds each predecessor's best term.
  * Admissible d: every part a power of two dividing the extent, N >= P and
    N a multiple of P.
  * Ties: lower cost, then fewer tasks, then the lexicographically smaller d
    (labels in canonical order: output labels, then contracted labels).
  * The softmax node is the pair LSE = lse_t S ("hst->hs") and
    Attn = exp(S - LSE) ("hst,hs->hst") under one d over (h, s, t); its cost
    is the sum of the two EinSums' costs.

This module is independent of the product's C++ chooser.
"""
from __future__ import annotations

import dataclasses
import itertools
import math
from typing import Dict, List, Optional, Sequence, Tuple

from . import ref


@dataclasses.dataclass
class Node:
    name: str
    spec: str                      # e.g. "sa,ahd->shd"; for softmax "hst->hst"
    bounds: Dict[str, int]
    inputs: List[str]              # producer node names or "@leaf" names
    kind: str = "einsum"           # "einsum" or "softmax"

    def labels(self) -> List[str]:
        """Canonical label order: output labels, then contracted labels."""
        if self.kind == "softmax":
            return list(self.spec.split("->")[1])
        ops, out, con = ref.parse(self.spec)
        return list(out) + list(con)

    def input_labels(self) -> List[str]:
        return self.spec.split("->")[0].split(",")

    def output_labels(self) -> str:
        return self.spec.split("->")[1]


def _prod(xs) -> int:
    r = 1
    for v in xs:
        r *= int(v)
    return r


def einsum_cost(spec: str, bounds: Dict[str, int], d: Dict[str, int]) -> int:
    """Join-input term plus aggregation term for one EinSum under d."""
    ops, out, con = ref.parse(spec)
    n = _prod(d[c] for c in set("".join(ops)))
    n_agg = _prod(d[c] for c in con)
    blk = lambda labels: _prod(bounds[c] // d[c] for c in labels)
    join_in = n * sum(blk(o) for o in ops)
    agg = (n // n_agg) * (n_agg - 1) * blk(out)
    return join_in + agg


def node_cost(node: Node, d: Dict[str, int]) -> int:
    if node.kind == "softmax":
        h, s, t = node.output_labels()
        lse = einsum_cost(f"{h}{s}{t}->{h}{s}", node.bounds, d)
        nrm = einsum_cost(f"{h}{s}{t},{h}{s}->{h}{s}{t}", node.bounds, d)
        return lse + nrm
    return einsum_cost(node.spec, node.bounds, d)


def n_tasks(node: Node, d: Dict[str, int]) -> int:
    return _prod(d[c] for c in node.labels())


def candidates(node: Node, p: int) -> List[Dict[str, int]]:
    """All admissible partition vectors of a node (power-of-two parts)."""
    labels = node.labels()
    opts = []
    for c in labels:
        b = node.bounds[c]
        opts.append([k for k in (1 << e for e in range(0, 31)) if k <= b and b % k == 0])
    out = []
    for combo in itertools.product(*opts):
        d = dict(zip(labels, combo))
        n = _prod(combo)
        if n >= p and n % p == 0:
            out.append(d)
    return out


def repartition_cost(producer: Node, d_u: Dict[str, int], consumer: Node,
                     slot: int, d_v: Dict[str, int]) -> int:
    """0 when the tensor is already blocked as the consumer needs, else its size."""
    zl = producer.output_labels()
    il = consumer.input_labels()[slot] if consumer.kind != "softmax" else consumer.output_labels()
    if len(zl) != len(il):
        raise ValueError("edge rank mismatch")
    if all(d_u[a] == d_v[b] for a, b in zip(zl, il)):
        return 0
    return _prod(producer.bounds[c] for c in zl)


def _key(node: Node, cost: int, d: Dict[str, int]):
    return (cost, n_tasks(node, d), tuple(d[c] for c in node.labels()))


def exhaustive(nodes: List[Node], p: int) -> Tuple[int, Dict[str, Dict[str, int]]]:
    """Minimum total graph cost over every joint assignment (small graphs)."""
    by = {n.name: n for n in nodes}
    cands = [candidates(n, p) for n in nodes]
    for n, c in zip(nodes, cands):
        if not c:
            raise ValueError(f"no admissible partition vector for {n.name}")
    best = None
    for combo in itertools.product(*cands):
        asg = {n.name: d for n, d in zip(nodes, combo)}
        tot = sum(node_cost(n, asg[n.name]) for n in nodes)
        for v in nodes:
            for slot, src in enumerate(v.inputs):
                if src in by:
                    tot += repartition_cost(by[src], asg[src], v, slot, asg[v.name])
        if best is None or tot < best[0]:
            best = (tot, asg)
    return best


def dp(nodes: List[Node], p: int, output: Optional[str] = None
       ) -> Tuple[int, Dict[str, Dict[str, int]]]:
    """The page's dynamic programme over a tree-shaped EinGraph, with backtracking."""
    by = {n.name: n for n in nodes}
    order: List[str] = []
    seen = set()

    def visit(name):
        if name in seen or name not in by:
            return
        for s in by[name].inputs:
            visit(s)
        seen.add(name)
        order.append(name)

    for n in nodes:
        visit(n.name)
    table: Dict[str, List[Tuple[int, Dict[str, int], List[int]]]] = {}
    for name in order:
        v = by[name]
        cands = candidates(v, p)
        if not cands:
            raise ValueError(f"no admissible partition vector for {name}")
        rows = []
        for dv in cands:
            tot = node_cost(v, dv)
            picks = []
            for slot, src in enumerate(v.inputs):
                if src not in by:
                    picks.append(-1)
                    continue
                u = by[src]
                best_i, best_k = -1, None
                for i, (cu, du, _) in enumerate(table[src]):
                    k = _key(u, cu + repartition_cost(u, du, v, slot, dv), du)
                    if best_k is None or k < best_k:
                        best_i, best_k = i, k
                tot += best_k[0]
                picks.append(best_i)
            rows.append((tot, dv, picks))
        table[name] = rows
    root = output or order[-1]
    ri = min(range(len(table[root])), key=lambda i: _key(by[root], table[root][i][0], table[root][i][1]))
    total = table[root][ri][0]
    asg: Dict[str, Dict[str, int]] = {}

    def back(name, i):
        _, d, picks = table[name][i]
        asg[name] = d
        for src, j in zip(by[name].inputs, picks):
            if j >= 0:
                back(src, j)

    back(root, ri)
    return total, asg


def graph_cost(nodes: List[Node], asg: Dict[str, Dict[str, int]]) -> int:
    by = {n.name: n for n in nodes}
    tot = sum(node_cost(n, asg[n.name]) for n in nodes)
    for v in nodes:
        for slot, src in enumerate(v.inputs):
            if src in by:
                tot += repartition_cost(by[src], asg[src], v, slot, asg[v.name])
    return tot


def mha_graph(s: int, a: int, h: int, dh: int) -> List[Node]:
    """The attention layer as an EinGraph (section 2.1's example)."""
    proj = {"s": s, "a": a, "h": h, "d": dh}
    return [
        Node("Q_proj", "sa,ahd->shd", dict(proj), ["@Q", "@W_Q"]),
        Node("K_proj", "sa,ahd->shd", dict(proj), ["@K", "@W_K"]),
        Node("V_proj", "sa,ahd->shd", dict(proj), ["@V", "@W_V"]),
        Node("Scores", "shd,thd->hst", {"s": s, "t": s, "h": h, "d": dh}, ["Q_proj", "K_proj"]),
        Node("Attn", "hst->hst", {"h": h, "s": s, "t": s}, ["Scores"], kind="softmax"),
        Node("O", "hst,thd->shd", {"h": h, "s": s, "t": s, "d": dh}, ["Attn", "V_proj"]),
        Node("Output", "shd,ahd->sa", {"s": s, "h": h, "d": dh, "a": a}, ["O", "@W_O"]),
    ]
