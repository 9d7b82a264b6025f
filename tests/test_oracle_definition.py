"""Pins of the oracle's extended EinSum against things other than itself.

Each test checks the nested-loop C oracle (oracle.ref.einsum) against values
fixed by the mathematics: hand-worked cases, an independent pure-Python brute
force, library routines for the special cases that are ordinary linear
algebra, and closed forms (squared distance, max-plus reductions, logsumexp).
"""
import itertools
import json
import zlib
import math
import os

import numpy as np
import pytest

from oracle import ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

TWO_OPERAND_SPECS = [
    "ij,jk->ik", "ij,kj->ik", "ij,jk->ki", "bij,bjk->bik", "ij,j->i",
    "abef,cfed->abcd", "ij,k->ijk", "ijk,jl->il", "i,j->", "ij,ij->ij", "ij,ji->",
    "hst,thd->shd",
]
UNARY_SPECS = ["ij->i", "ijk->ik", "ij->ij", "ij->", "hst->hs"]
FLOAT_JOINS = ["mul", "sqdiff", "add", "exp_sub", "sub"]
INT_JOINS = ["mul", "sqdiff", "add", "sub"]
AGGS = ["none", "sum", "max", "min", "lse"]


def _operands(spec, rng, is_int, lo=1, hi=4):
    ops, out, con = ref.parse(spec)
    ext = {c: int(rng.integers(lo, hi + 1)) for c in sorted(set("".join(ops)))}
    arrs = []
    for o in ops:
        shape = tuple(ext[c] for c in o)
        if is_int:
            arrs.append(rng.integers(-9, 10, size=shape).astype(np.int64))
        else:
            arrs.append(rng.uniform(-1, 1, size=shape))
    return ops, out, con, arrs


def _valid(con, join, agg, is_int):
    if agg == "none" and con:
        return False
    if is_int and (join == "exp_sub" or agg == "lse"):
        return False
    return True


def test_hand_cases():
    cases = json.load(open(os.path.join(GOLDEN, "hand_cases.json")))["cases"]
    for c in cases:
        dt = np.int64 if c["dtype"] == "int" else np.float64
        x = np.array(c["x"], dtype=dt)
        y = np.array(c["y"], dtype=dt) if "y" in c else None
        z = ref.einsum(c["spec"], x, y, c["join"], c["agg"], c.get("post_scale", 1.0))
        want = np.array(c["z"], dtype=dt)
        if dt == np.int64:
            np.testing.assert_array_equal(z, want, err_msg=c["spec"])
        else:
            np.testing.assert_allclose(z, want, rtol=1e-14, atol=1e-14, err_msg=c["spec"])


@pytest.mark.parametrize("spec", TWO_OPERAND_SPECS + UNARY_SPECS)
@pytest.mark.parametrize("is_int", [False, True])
def test_c_oracle_equals_brute_force(spec, is_int):
    rng = np.random.default_rng(zlib.crc32(f"{spec}{is_int}".encode()))
    unary = "," not in spec
    joins = ["ident"] if unary else (INT_JOINS if is_int else FLOAT_JOINS)
    for join, agg in itertools.product(joins, AGGS):
        ops, out, con, arrs = _operands(spec, rng, is_int)
        if not _valid(con, join, agg, is_int):
            continue
        y = None if unary else arrs[1]
        ps = 1.0 if is_int else 0.75
        got = ref.einsum(spec, arrs[0], y, join, agg, ps)
        want = ref.brute_einsum(spec, arrs[0], y, join, agg, ps)
        if is_int:
            np.testing.assert_array_equal(got, want, err_msg=f"{spec} {join} {agg}")
        else:
            np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12, err_msg=f"{spec} {join} {agg}")


@pytest.mark.parametrize("spec", TWO_OPERAND_SPECS + UNARY_SPECS)
def test_dense_evaluator_equals_brute_force(spec):
    rng = np.random.default_rng(7)
    unary = "," not in spec
    joins = ["ident"] if unary else FLOAT_JOINS
    for join, agg in itertools.product(joins, AGGS):
        ops, out, con, arrs = _operands(spec, rng, False)
        if not _valid(con, join, agg, False):
            continue
        y = None if unary else arrs[1]
        got = ref.dense_einsum(spec, arrs[0], y, join, agg, 1.25)
        want = ref.brute_einsum(spec, arrs[0], y, join, agg, 1.25)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12, err_msg=f"{spec} {join} {agg}")


def test_matmul_equals_library_product():
    rng = np.random.default_rng(1)
    x = rng.uniform(-1, 1, (256, 256))
    y = rng.uniform(-1, 1, (256, 256))
    np.testing.assert_allclose(ref.einsum("ij,jk->ik", x, y), x @ y, rtol=0, atol=1e-12)
    xi = rng.integers(-8, 9, (64, 96)).astype(np.int64)
    yi = rng.integers(-8, 9, (96, 80)).astype(np.int64)
    np.testing.assert_array_equal(ref.einsum("ij,jk->ik", xi, yi), xi @ yi)
    # transposed operand layouts
    np.testing.assert_allclose(ref.einsum("ij,kj->ik", x, y), x @ y.T, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ref.einsum("ij,jk->ki", x, y), (x @ y).T, rtol=0, atol=1e-12)


def test_four_index_contraction_equals_library():
    rng = np.random.default_rng(3)
    a = rng.normal(0, 0.1, (8, 6, 4, 5))     # a b e f
    b = rng.normal(0, 0.1, (7, 5, 4, 3))     # c f e d
    want = np.tensordot(a, b, axes=([2, 3], [2, 1]))  # a b c d
    np.testing.assert_allclose(ref.einsum("abef,cfed->abcd", a, b), want, rtol=0, atol=1e-13)


def test_batched_and_attention_specs_equal_library():
    rng = np.random.default_rng(4)
    attn = rng.uniform(0, 1, (3, 5, 6))      # h s t
    v = rng.normal(0, 1, (6, 3, 4))          # t h d
    want = np.einsum("hst,thd->shd", attn, v)
    np.testing.assert_allclose(ref.einsum("hst,thd->shd", attn, v), want, rtol=0, atol=1e-13)
    q = rng.normal(0, 1, (5, 3, 4))          # s h d
    k = rng.normal(0, 1, (6, 3, 4))          # t h d
    want = np.einsum("shd,thd->hst", q, k) / math.sqrt(4)
    np.testing.assert_allclose(ref.einsum("shd,thd->hst", q, k, post_scale=0.5), want, rtol=0, atol=1e-13)


def test_squared_distance_closed_form():
    rng = np.random.default_rng(5)
    x = rng.normal(0, 1, (40, 32))
    y = rng.normal(0, 1, (32, 50))
    got = ref.einsum("ij,jk->ik", x, y, "sqdiff", "sum")
    closed = (x * x).sum(1)[:, None] + (y * y).sum(0)[None, :] - 2 * x @ y
    np.testing.assert_allclose(got, closed, rtol=1e-10, atol=0)
    assert (got >= 0).all()


def test_max_plus_special_cases():
    rng = np.random.default_rng(6)
    x = rng.integers(-1000, 1001, (20, 30)).astype(np.int64)
    y = rng.integers(-1000, 1001, (30, 25)).astype(np.int64)
    # Y == 0 reduces to the row maximum of X
    z0 = ref.einsum("ij,jk->ik", x, np.zeros_like(y), "add", "max")
    np.testing.assert_array_equal(z0, np.repeat(x.max(1)[:, None], 25, axis=1))
    # one contracted index reduces to the outer sum
    z1 = ref.einsum("ij,jk->ik", x[:, :1], y[:1, :], "add", "max")
    np.testing.assert_array_equal(z1, x[:, :1] + y[:1, :])
    # min-plus of negated operands is minus max-plus
    zmin = ref.einsum("ij,jk->ik", -x, -y, "add", "min")
    np.testing.assert_array_equal(zmin, -ref.einsum("ij,jk->ik", x, y, "add", "max"))
    # against an explicit broadcast maximum
    want = (x[:, :, None] + y[None, :, :]).max(axis=1)
    np.testing.assert_array_equal(ref.einsum("ij,jk->ik", x, y, "add", "max"), want)


def test_sub_join_closed_forms():
    # The difference join (used by the softmax backward, dS = P * (dP - rowsum)):
    # summed over j it separates into row sums of X minus column sums of Y.
    rng = np.random.default_rng(11)
    x = rng.uniform(-1, 1, (12, 9))
    y = rng.uniform(-1, 1, (9, 7))
    got = ref.einsum("ij,jk->ik", x, y, "sub", "sum")
    np.testing.assert_allclose(got, x.sum(1)[:, None] - y.sum(0)[None, :], rtol=1e-12, atol=1e-12)
    # broadcast over a missing label, no aggregate: S[h,s,t] - L[h,s]
    s3 = rng.uniform(-2, 2, (3, 5, 6))
    l2 = rng.uniform(-2, 2, (3, 5))
    np.testing.assert_array_equal(ref.einsum("hst,hs->hst", s3, l2, "sub", "none"), s3 - l2[:, :, None])
    # integers: max_j (x - y) with y == 0 is the row maximum; exact
    xi = rng.integers(-1000, 1001, (8, 11)).astype(np.int64)
    yi = np.zeros((11, 4), dtype=np.int64)
    np.testing.assert_array_equal(ref.einsum("ij,jk->ik", xi, yi, "sub", "max"),
                                  np.repeat(xi.max(1)[:, None], 4, axis=1))
    # the operand order matters: x - y, not y - x
    assert ref.einsum("i,i->i", np.array([5.0]), np.array([2.0]), "sub", "none")[0] == 3.0


def test_logsumexp_closed_forms():
    # lse of a constant c over n terms is c + ln n
    for c, n in [(0.0, 1), (2.5, 7), (-3.0, 4096)]:
        z = ref.einsum("ij->i", np.full((3, n), c), None, "ident", "lse")
        np.testing.assert_allclose(z, c + math.log(n), rtol=1e-14, atol=1e-14)
    # exp(S - lse(S)) sums to one along the reduced label
    rng = np.random.default_rng(8)
    s = rng.normal(0, 4, (3, 5, 9))
    lse = ref.einsum("hst->hs", s, None, "ident", "lse")
    attn = ref.einsum("hst,hs->hst", s, lse, "exp_sub", "none")
    np.testing.assert_allclose(attn.sum(axis=2), 1.0, rtol=0, atol=1e-13)
    assert (attn > 0).all()
    # huge values do not overflow
    big = ref.einsum("ij->i", np.array([[1000.0, 1000.0]]), None, "ident", "lse")
    np.testing.assert_allclose(big, 1000.0 + math.log(2), rtol=1e-15)


def test_sampled_outputs_equal_full():
    rng = np.random.default_rng(9)
    x = rng.normal(0, 1, (17, 9))
    y = rng.normal(0, 1, (9, 13))
    full = ref.einsum("ij,jk->ik", x, y, "sqdiff", "sum")
    idx = rng.choice(full.size, 40, replace=False)
    np.testing.assert_array_equal(ref.einsum("ij,jk->ik", x, y, "sqdiff", "sum", out_index=idx),
                                  full.reshape(-1)[idx])


def test_rejects_undefined_combinations():
    x = np.ones((2, 3), dtype=np.int64)
    with pytest.raises(ValueError):
        ref.einsum("ij,jk->ik", x, x.T.copy(), "mul", "none")          # contracted label, no aggregate
    with pytest.raises(ValueError):
        ref.einsum("ij->i", x, None, "ident", "lse")                     # lse on integers
    with pytest.raises(ValueError):
        ref.einsum("ij,jk->iq", x, x.T.copy())                           # output label in no operand
    with pytest.raises(ValueError):
        ref.einsum("ii,jk->ik", x, x.T.copy())                           # repeated label


def test_empty_ranges_give_the_aggregates_identity():
    """An empty contracted range folds nothing: sum 0, max -inf, min +inf,
    lse -inf (float; times post_scale), and INT64_MIN / INT64_MAX / 0 for the
    integer oracle; an empty output label gives an empty result."""
    x = np.ones((3, 0))
    y = np.ones((0, 2))
    z = ref.einsum("ij,jk->ik", x, y, "mul", "sum")
    assert z.shape == (3, 2) and np.all(z == 0.0)
    assert np.all(ref.einsum("ij,jk->ik", x, y, "add", "max") == -np.inf)
    assert np.all(ref.einsum("ij,jk->ik", x, y, "add", "min") == np.inf)
    assert np.all(ref.einsum("ij,jk->ik", x, y, "mul", "lse") == -np.inf)
    assert np.all(ref.einsum("ij,jk->ik", x, y, "add", "max", post_scale=2.0) == -np.inf)
    xi, yi = np.ones((3, 0), dtype=np.int64), np.ones((0, 2), dtype=np.int64)
    assert np.all(ref.einsum("ij,jk->ik", xi, yi, "add", "max") == np.iinfo(np.int64).min)
    assert np.all(ref.einsum("ij,jk->ik", xi, yi, "add", "min") == np.iinfo(np.int64).max)
    assert np.all(ref.einsum("ij,jk->ik", xi, yi, "mul", "sum") == 0)
    # an empty output label: nothing to compute
    z = ref.einsum("ij,jk->ik", np.ones((0, 4)), np.ones((4, 5)), "mul", "sum")
    assert z.shape == (0, 5)
    # brute force agrees on the empty range
    bz = ref.brute_einsum("ij,jk->ik", x, y, "add", "max")
    assert np.all(np.asarray(bz) == -np.inf)
