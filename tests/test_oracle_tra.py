"""Pins of the literal TRA evaluator and the relation layout (CPU only).

* the partition rule and the flat layout against a hand-worked example;
* d-invariance: for every admissible d on tiny shapes, the TRA plan's result
  equals the plain EinSum (exact for integers);
* the page's three matmul partition vectors: task structure worked by hand,
  and the result at 256^3;
* the 2.5D SUMMA block equations of the ColossalAI 2.5D page.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import ref, tra_cpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _divisors(n):
    return [k for k in range(1, n + 1) if n % k == 0]


def test_partition_rule_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "partition_rule_4x6.json")))
    t = np.array(g["tensor"])
    rel = tra_cpu.partition(t, g["d"])
    assert len(rel) == 6
    for key, block in g["relation"].items():
        k = tuple(int(v) for v in key.split(","))
        np.testing.assert_array_equal(rel[k], np.array(block))
    np.testing.assert_array_equal(tra_cpu.to_buffer(t, g["d"]), np.array(g["flat_buffer"]))
    np.testing.assert_array_equal(tra_cpu.from_buffer(np.array(g["flat_buffer"]), g["shape"], g["d"]), t)


def test_layout_closed_form_and_round_trips():
    # the element at global index g sits at offset rowmajor(k; d) * vol + rowmajor(r; b)
    shape, d = (6, 4, 8), (3, 2, 4)
    t = np.arange(np.prod(shape)).reshape(shape)
    buf = tra_cpu.to_buffer(t, d)
    b = [s // k for s, k in zip(shape, d)]
    vol = int(np.prod(b))
    for g in itertools.product(*[range(s) for s in shape]):
        k = [gi // bi for gi, bi in zip(g, b)]
        r = [gi % bi for gi, bi in zip(g, b)]
        off = np.ravel_multi_index(k, d) * vol + np.ravel_multi_index(r, b)
        assert buf[off] == t[g]
    # all-ones partition is the dense row-major array
    np.testing.assert_array_equal(tra_cpu.to_buffer(t, (1, 1, 1)), t.reshape(-1))
    # d_u -> d_v -> d_u is the identity, and a permutation of the elements
    for du, dv in [((3, 2, 4), (1, 4, 2)), ((6, 1, 8), (2, 4, 1))]:
        bu = tra_cpu.to_buffer(t, du)
        bv = tra_cpu.repartition_buffer(bu, shape, du, dv)
        assert sorted(bv.tolist()) == sorted(bu.tolist())
        np.testing.assert_array_equal(tra_cpu.repartition_buffer(bv, shape, dv, du), bu)
    with pytest.raises(ValueError):
        tra_cpu.to_buffer(t, (4, 2, 4))


def test_buffer_offset_agrees_with_the_partitioned_buffer():
    for shape, d in [((6, 4, 8), (3, 2, 4)), ((4, 6), (2, 3)), ((16,), (4,)), ((2, 3, 4, 5), (1, 3, 2, 5))]:
        t = np.arange(int(np.prod(shape))).reshape(shape)
        buf = tra_cpu.to_buffer(t, d)
        for g in itertools.product(*[range(s) for s in shape]):
            assert buf[tra_cpu.buffer_offset(g, shape, d)] == t[g]


CASES = [
    ("ij,jk->ik", {"i": 4, "j": 6, "k": 2}),
    ("abef,cfed->abcd", {"a": 2, "b": 2, "c": 2, "d": 2, "e": 4, "f": 2}),
    ("bij,bjk->bik", {"b": 2, "i": 2, "j": 4, "k": 2}),
    ("shd,thd->hst", {"s": 2, "t": 4, "h": 2, "d": 2}),
    ("hst->hs", {"h": 2, "s": 2, "t": 4}),
    ("ij,k->ijk", {"i": 2, "j": 2, "k": 4}),
]


@pytest.mark.parametrize("spec,bounds", CASES)
def test_d_invariance_every_admissible_d(spec, bounds):
    ops, out, con = ref.parse(spec)
    rng = np.random.default_rng(11)
    combos = [(j, a) for j in (["ident"] if len(ops) == 1 else ["mul", "sqdiff", "add"])
              for a in ["sum", "max", "min"]]
    labels = sorted(bounds)
    for is_int in (True, False):
        arrs = []
        for o in ops:
            shape = tuple(bounds[c] for c in o)
            arrs.append(rng.integers(-7, 8, shape).astype(np.int64) if is_int else rng.normal(0, 1, shape))
        y = arrs[1] if len(ops) == 2 else None
        for join, agg in combos + ([] if is_int else [("ident" if len(ops) == 1 else "sqdiff", "lse")]):
            want = ref.einsum(spec, arrs[0], y, join, agg)
            for dv in itertools.product(*[_divisors(bounds[c]) for c in labels]):
                dmap = dict(zip(labels, dv))
                got = tra_cpu.tra_einsum(spec, arrs[0], y, dmap, join, agg)
                if is_int:
                    np.testing.assert_array_equal(got, want, err_msg=f"{spec} {join} {agg} {dmap}")
                else:
                    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12,
                                               err_msg=f"{spec} {join} {agg} {dmap}")


def test_matmul_partition_examples():
    g = json.load(open(os.path.join(GOLDEN, "matmul_partition_examples.json")))
    for c in g["cases"]:
        di, djx, djy, dk = c["d4"]
        dmap = {"i": di, "j": djx, "k": dk}
        n, grp, n_agg = tra_cpu.task_counts("ij,jk->ik", dmap)
        assert (n, grp, n_agg) == (c["N"], c["G"], c["n_agg"])
        assert (n_agg > 1) == c["needs_aggregation"]


def test_matmul_256_under_the_three_partition_vectors():
    rng = np.random.default_rng(12)
    xi = rng.integers(-8, 9, (256, 256)).astype(np.int64)
    yi = rng.integers(-8, 9, (256, 256)).astype(np.int64)
    xf = rng.uniform(-1, 1, (256, 256))
    yf = rng.uniform(-1, 1, (256, 256))
    wi = xi @ yi
    wf = ref.einsum("ij,jk->ik", xf, yf)
    for d4 in ([4, 1, 1, 4], [1, 4, 4, 1], [2, 2, 2, 2]):
        dmap = {"i": d4[0], "j": d4[1], "k": d4[3]}
        np.testing.assert_array_equal(tra_cpu.tra_einsum("ij,jk->ik", xi, yi, dmap), wi)
        np.testing.assert_allclose(tra_cpu.tra_einsum("ij,jk->ik", xf, yf, dmap), wf, rtol=0, atol=1e-12)


def test_summa_25d_block_equations():
    g = json.load(open(os.path.join(GOLDEN, "summa25d_q2_d2.json")))
    rng = np.random.default_rng(13)
    br, bc, bn = 3, 5, 4                        # X block rows, shared cols, A block cols
    rx, cx = g["x_blocks"]
    ra, ca = g["a_blocks"]
    x = rng.normal(0, 1, (rx * br, cx * bc))
    a = rng.normal(0, 1, (ra * bc, ca * bn))
    X = {f"{r}{c}": x[r * br:(r + 1) * br, c * bc:(c + 1) * bc] for r in range(rx) for c in range(cx)}
    A = {f"{r}{c}": a[r * bc:(r + 1) * bc, c * bn:(c + 1) * bn] for r in range(ra) for c in range(ca)}
    want = ref.einsum("ij,jk->ik", x, a)
    for yk, terms in g["y"].items():
        r, c = int(yk[0]), int(yk[1])
        blk = sum(X[xs] @ A[as_] for xs, as_ in terms)
        np.testing.assert_allclose(blk, want[r * br:(r + 1) * br, c * bn:(c + 1) * bn], rtol=0, atol=1e-12)
    # the same blocking as a TRA plan: i cut d*q = 4, j cut q = 2, k cut q = 2
    got = tra_cpu.tra_einsum("ij,jk->ik", x, a, {"i": 4, "j": 2, "k": 2})
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
