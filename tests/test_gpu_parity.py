"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case draws its inputs from the seeded generators, runs dense ->
relation -> join + aggregation -> dense on the GPU, and compares with the
oracle: integers and max-plus bit-exact, fp32 to 1e-4 and bf16-in / fp32-acc
to 2e-2 (max-norm relative error).  Reduced sizes are compared element by
element (they span several tiles and partitions); the full workload sizes,
in the launch configuration the bench uses, are compared on sampled outputs.
"""
import itertools

import numpy as np
import pytest
import torch

import tensor_relational_algebra_amd as tra
from oracle import ref, tra_cpu
from tensor_relational_algebra_amd import workloads as wl
from tests.gpu_util import DEV, check, gate, maxnorm_rel_err, run_gpu

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------ repartition

REPART_CASES = [
    ((16,), (1,), (4,)),
    ((8, 12), (2, 3), (4, 1)),
    ((64, 32), (1, 1), (4, 8)),
    ((64, 32), (4, 8), (16, 2)),
    ((6, 8, 10), (3, 2, 5), (1, 4, 1)),
    ((32, 16, 8, 4), (2, 4, 2, 1), (8, 1, 4, 2)),
    ((256, 96), (16, 3), (2, 12)),
]


@pytest.mark.parametrize("shape,du,dv", REPART_CASES)
@pytest.mark.parametrize("dtype", [torch.int32, torch.float32, torch.bfloat16])
def test_repartition_matches_the_partition_rule(shape, du, dv, dtype):
    n = int(np.prod(shape))
    dense = torch.arange(n, dtype=torch.int64).reshape(shape)
    t = dense.to(dtype) if dtype != torch.bfloat16 else (dense % 256).to(dtype)
    src = torch.from_numpy(tra_cpu.to_buffer(t.view(torch.int16).numpy() if dtype == torch.bfloat16 else t.numpy(), du))
    if dtype == torch.bfloat16:
        src = src.view(torch.bfloat16)
    want = tra_cpu.to_buffer(t.view(torch.int16).numpy() if dtype == torch.bfloat16 else t.numpy(), dv)
    got = tra.tra_repartition(src.to(DEV), list(shape), list(du), list(dv)).cpu()
    got = got.view(torch.int16).numpy() if dtype == torch.bfloat16 else got.numpy()
    np.testing.assert_array_equal(got, want)
    # round trip and dense <-> relation
    back = tra.tra_repartition(tra.tra_repartition(src.to(DEV), list(shape), list(du), list(dv)),
                               list(shape), list(dv), list(du))
    assert torch.equal(back.cpu(), src)
    dn = tra.from_relation(src.to(DEV), list(shape), list(du)).cpu()
    assert torch.equal(dn, t)


def test_repartition_gemm_output_full_size():
    """The blocked GEMM's output Y [16384, 8192] re-cut from [16, 4] to [4, 16]."""
    shape = (16384, 8192)
    n = shape[0] * shape[1]
    iota = torch.arange(n, dtype=torch.int32, device=DEV)
    rel = tra.tra_repartition(iota, list(shape), [1, 1], list(wl.GEMM25D_Y_FROM))
    out = tra.tra_repartition(rel, list(shape), list(wl.GEMM25D_Y_FROM), list(wl.GEMM25D_Y_TO))
    rng = np.random.default_rng(5)
    gi = rng.integers(0, shape[0], 20000)
    gj = rng.integers(0, shape[1], 20000)
    pos_from = [tra_cpu.buffer_offset((a, b), shape, wl.GEMM25D_Y_FROM) for a, b in zip(gi, gj)]
    pos_to = [tra_cpu.buffer_offset((a, b), shape, wl.GEMM25D_Y_TO) for a, b in zip(gi, gj)]
    want = torch.from_numpy((gi * shape[1] + gj).astype(np.int32))
    assert torch.equal(rel[torch.tensor(pos_from, device=DEV)].cpu(), want)
    assert torch.equal(out[torch.tensor(pos_to, device=DEV)].cpu(), want)
    back = tra.tra_repartition(out, list(shape), list(wl.GEMM25D_Y_TO), [1, 1])
    assert torch.equal(back, iota)


# ------------------------------------------------------------ partitioned matmul

@pytest.mark.parametrize("d4", [[4, 1, 1, 4], [1, 4, 4, 1], [2, 2, 2, 2], [1, 1, 1, 1]])
@pytest.mark.parametrize("base", [wl.MATMUL_F32, wl.MATMUL_I32], ids=["f32", "i32"])
def test_partitioned_matmul_256(base, d4):
    check(base.with_d(wl.matmul_d(d4)))


# ------------------------------------------------------------ squared distance / max-plus

SMALL_NL = {"i": 512, "j": 96, "k": 384}


@pytest.mark.parametrize("d", [{"i": 1, "j": 1, "k": 1}, {"i": 2, "j": 1, "k": 3}, {"i": 4, "j": 3, "k": 2},
                               {"i": 4, "j": 1, "k": 2}, {"i": 2, "j": 2, "k": 2}])
@pytest.mark.parametrize("base", [wl.SQDIST, wl.MAXPLUS], ids=["sqdist", "maxplus"])
def test_nonlinear_joins_small(base, d):
    check(base.scaled(SMALL_NL, d))


@pytest.mark.parametrize("d", [wl.matmul_d([16, 1, 1, 16]), wl.matmul_d([8, 1, 1, 32]), wl.matmul_d([16, 2, 2, 16])])
@pytest.mark.parametrize("base", [wl.SQDIST, wl.MAXPLUS], ids=["sqdist", "maxplus"])
def test_nonlinear_joins_full_size_sampled(base, d):
    err, plan = check(base.with_d(d), sample=1 << 17)
    assert plan.kernel == "valu_tile"


def test_min_plus_variant():
    b = {"i": 256, "j": 64, "k": 256}
    check(wl.EinsumCase("minplus", 77, "ij,jk->ik", b, {"i": 2, "j": 2, "k": 1}, "add", "min", "i32", "i32",
                        (("int", {"lo": -50, "hi": 50}), ("int", {"lo": -50, "hi": 50}))))



# ------------------------------------------------------------ int32 max-plus / min-plus: packed 16-bit path

def _run_small_int(spec, bounds, d, agg, xs):
    """Run an int32 add-join through the C ABI with an explicit workspace;
    returns (dense output, plan, the range-check flag words)."""
    case = wl.EinsumCase("si", 0, spec, bounds, d, "add", agg, "i32", "i32", ())
    plan = tra.tra_plan(spec, bounds, d, "add", agg, "i32", "i32")
    ws = torch.empty(plan.info.workspace_bytes, dtype=torch.uint8, device=DEV)
    rels = [tra.to_relation(t.to(DEV), [d[c] for c in o]) for t, o in zip(xs, case.operand_labels())]
    zr = tra.tra_execute(plan, rels[0], rels[1], None, ws)
    out = case.out_labels()
    z = tra.from_relation(zr, [bounds[c] for c in out], [d[c] for c in out])
    torch.cuda.synchronize()
    flags = ws[-1024:].view(torch.int32).cpu().numpy()
    return z.cpu(), plan, flags


def _si_inputs(spec, bounds, seed, lo, hi):
    ops = spec.split("->")[0].split(",")
    rng = np.random.default_rng(seed)
    return [torch.from_numpy(rng.integers(lo, hi, size=[bounds[c] for c in o], endpoint=True, dtype=np.int32))
            for o in ops]


SI_CASES = [
    ("ij,jk->ik", {"i": 2048, "j": 64, "k": 1024}, {"i": 2, "j": 2, "k": 4}),   # 128 tiles, no split
    ("ij,jk->ik", {"i": 512, "j": 128, "k": 256}, {"i": 2, "j": 4, "k": 1}),    # X K-major, Y MN-major
    ("ji,kj->ik", {"i": 256, "j": 64, "k": 128}, {"i": 1, "j": 2, "k": 2}),     # X MN-major, Y K-major
    ("ij,kj->ik", {"i": 128, "j": 64, "k": 256}, {"i": 2, "j": 1, "k": 2}),     # both K-major
    ("ji,jk->ik", {"i": 128, "j": 128, "k": 256}, {"i": 1, "j": 2, "k": 2}),    # both MN-major
    ("ij,jk->ik", {"i": 256, "j": 2048, "k": 256}, {"i": 1, "j": 4, "k": 1}),   # 64-way split of the contraction
]


@pytest.mark.parametrize("agg", ["max", "min"])
@pytest.mark.parametrize("spec,bounds,d", SI_CASES, ids=["nosplit", "ij,jk", "ji,kj", "ij,kj", "ji,jk", "split64"])
def test_small_int_packed_path_is_exact(spec, bounds, d, agg):
    """Inputs within [-1024, 1024], the extremes included: the range check
    clears every flag (so the packed 16-bit kernel produced the output) and
    the result equals the oracle's exactly."""
    xs = _si_inputs(spec, bounds, 5, -1024, 1024)
    for t, v in zip(xs, (-1024, 1024)):     # both extremes present in both operands
        t.view(-1)[0] = v
        t.view(-1)[-1] = -v
    z, plan, flags = _run_small_int(spec, bounds, d, agg, xs)
    assert plan.kernel == "valu_tile" and plan.info.tile == 1
    assert not flags.any()
    want = ref.einsum(spec, xs[0], xs[1], "add", agg)
    assert np.array_equal(z.numpy().astype(np.int64), want)


@pytest.mark.parametrize("agg", ["max", "min"])
@pytest.mark.parametrize("where", ["x", "y", "both_wide"])
@pytest.mark.parametrize("spec,bounds,d", SI_CASES[:3] + SI_CASES[5:], ids=["nosplit", "ij,jk", "ji,kj", "split64"])
def test_small_int_out_of_range_takes_the_32_bit_path(spec, bounds, d, agg, where):
    """One input just outside [-1024, 1024] (or every input spread over +-2^29):
    the range check sets a flag, the 32-bit kernel produces the output, and it
    equals the oracle's exactly."""
    if where == "both_wide":
        xs = _si_inputs(spec, bounds, 6, -(1 << 29), 1 << 29)
    else:
        xs = _si_inputs(spec, bounds, 6, -1024, 1024)
        t = xs[0] if where == "x" else xs[1]
        t.view(-1)[t.numel() // 3] = 1025 if agg == "max" else -1025
    z, plan, flags = _run_small_int(spec, bounds, d, agg, xs)
    assert flags.any()
    want = ref.einsum(spec, xs[0], xs[1], "add", agg)
    assert np.array_equal(z.numpy().astype(np.int64), want)


def test_small_int_path_on_the_full_workload_sampled():
    """The max-plus workload (values in [-1000, 1000]) at its full size and
    blocking, as the bench runs it: flags clear, sampled outputs exact."""
    c = wl.MAXPLUS
    xs = c.make_inputs()
    z, plan, flags = _run_small_int(c.spec, c.bounds, c.d, c.agg, xs)
    assert not flags.any() and plan.info.tile == 1
    idx = np.sort(np.random.default_rng(3).choice(z.numel(), size=4096, replace=False))
    want = ref.einsum(c.spec, xs[0], xs[1], "add", "max", out_index=idx)
    assert np.array_equal(z.reshape(-1)[torch.from_numpy(idx)].numpy().astype(np.int64), want)

# ------------------------------------------------------------ four-index contraction

C3_SMALL = {"a": 16, "b": 8, "c": 16, "d": 32, "e": 16, "f": 8}


@pytest.mark.parametrize("d", [dict(a=1, b=1, c=1, d=1, e=1, f=1), dict(a=2, b=2, c=2, d=2, e=4, f=4),
                               dict(a=4, b=1, c=2, d=1, e=2, f=1), dict(a=1, b=2, c=4, d=4, e=1, f=2)])
def test_contract4_small(d):
    check(wl.CONTRACT4.scaled(C3_SMALL, d))


@pytest.mark.parametrize("d", [wl.CONTRACT4.d, dict(a=1, b=1, c=1, d=1, e=1, f=1),
                               dict(a=4, b=4, c=4, d=4, e=1, f=1)])
def test_contract4_full_size_sampled(d):
    err, plan = check(wl.CONTRACT4.with_d(d), sample=1 << 18, seed=3)
    if d == wl.CONTRACT4.d:
        assert plan.kernel == "mfma_bf16"


# ------------------------------------------------------------ blocked GEMM

@pytest.mark.parametrize("d", [{"i": 16, "j": 4, "k": 4}, {"i": 4, "j": 2, "k": 2}, {"i": 1, "j": 1, "k": 1}])
def test_gemm25d_small(d):
    check(wl.GEMM25D.scaled({"i": 2048, "j": 1024, "k": 512}, d))


def test_gemm25d_full_size_sampled():
    err, plan = check(wl.GEMM25D, sample=1 << 16, seed=4)
    assert plan.kernel == "mfma_bf16"


def test_gemm25d_full_size_whole_rows():
    """32 whole rows of Y (two in each of the 16 row blocks, every column, so
    every output tile column and all four contracted partitions) against the
    oracle, in the bench's launch configuration."""
    c = wl.GEMM25D
    xs = c.make_inputs()
    z, plan = run_gpu(c, xs)
    assert plan.kernel == "mfma_bf16" and plan.info.agg_split == 1
    rng = np.random.default_rng(44)
    rows = np.sort(np.concatenate([b * 1024 + rng.choice(1024, 2, replace=False) for b in range(16)]))
    idx = (rows[:, None] * 8192 + np.arange(8192)[None, :]).reshape(-1)
    want = ref.einsum(c.spec, xs[0], xs[1], c.join, c.agg, out_index=idx)
    gate("gemm25d 32 whole rows", plan.kernel, z[torch.from_numpy(rows)].double().numpy(), want, 2e-2, 2e-2)


def test_gemm_bf16_output_and_post_scale():
    c = wl.EinsumCase("gemm_bf16out", 78, "ij,jk->ik", {"i": 512, "j": 256, "k": 256}, {"i": 2, "j": 2, "k": 2},
                      "mul", "sum", "bf16", "bf16", (("normal", {"std": 1.0}), ("normal", {"std": 1.0})),
                      post_scale=0.125)
    check(c)


# ------------------------------------------------------------ softmax as two EinSums

@pytest.mark.parametrize("d", [dict(h=1, s=1, t=1), dict(h=2, s=4, t=1), dict(h=2, s=2, t=4)])
def test_logsumexp_and_normalise(d):
    b = {"h": 4, "s": 64, "t": 512}
    s_case = wl.EinsumCase("lse", 79, "hst->hs", b, d, "ident", "lse", "f32", "f32",
                           (("normal", {"std": 3.0}),))
    (scores,) = s_case.make_inputs()
    lse_gpu, plan = run_gpu(s_case, [scores])
    want_lse = ref.einsum("hst->hs", scores, None, "ident", "lse")
    assert maxnorm_rel_err(lse_gpu.double().numpy(), want_lse) <= 1e-4
    n_case = wl.EinsumCase("norm", 80, "hst,hs->hst", b, d, "exp_sub", "none", "f32", "f32", ((), ()))
    attn, plan2 = run_gpu(n_case, [scores, torch.from_numpy(want_lse.astype(np.float32))])
    want = ref.einsum("hst,hs->hst", scores, want_lse.astype(np.float32), "exp_sub", "none")
    assert maxnorm_rel_err(attn.double().numpy(), want) <= 1e-4
    assert plan2.kernel == "elemwise"
    np.testing.assert_allclose(attn.double().sum(-1).numpy(), 1.0, atol=1e-4)


# ------------------------------------------------------------ generic path, property style

GENERIC_SPECS = [
    ("ij,jk->ik", {"i": 5, "j": 7, "k": 3}),
    ("bij,bjk->bik", {"b": 3, "i": 4, "j": 6, "k": 5}),
    ("ijk,jl->il", {"i": 6, "j": 4, "k": 3, "l": 5}),
    ("ij,k->ijk", {"i": 4, "j": 3, "k": 6}),
    ("ij,ji->", {"i": 6, "j": 8}),
    ("hst->hs", {"h": 3, "s": 4, "t": 10}),
    ("ij,jk->ki", {"i": 6, "j": 9, "k": 4}),
    ("abef,cfed->abcd", {"a": 2, "b": 3, "c": 2, "d": 3, "e": 4, "f": 2}),
]


def _divisors(n):
    return [k for k in range(1, n + 1) if n % k == 0]


@pytest.mark.parametrize("spec,bounds", GENERIC_SPECS)
def test_every_join_aggregate_dtype_on_small_shapes(spec, bounds):
    ops, out, con = ref.parse(spec)
    rng = np.random.default_rng(21)
    labels = tra.tra_canonical_labels(spec)
    for idt in ("i32", "f32", "bf16"):
        joins = ["ident"] if len(ops) == 1 else (["mul", "sqdiff", "add", "sub"] if idt == "i32"
                                                  else ["mul", "sqdiff", "add", "exp_sub", "sub"])
        aggs = (["none"] if not con else []) + ["sum", "max", "min"] + ([] if idt == "i32" else ["lse"])
        for join, agg in itertools.product(joins, aggs):
            dmap = {c: int(rng.choice(_divisors(bounds[c]))) for c in labels}
            dist = ("int", {"lo": -9, "hi": 9}) if idt == "i32" else ("uniform", {"lo": -1.0, "hi": 1.0})
            odt = "i32" if idt == "i32" else "f32"
            case = wl.EinsumCase(f"prop_{spec}_{join}_{agg}", 300, spec, bounds, dmap, join, agg, idt, odt,
                                 tuple([dist] * len(ops)))
            check(case)


# ------------------------------------------------------------ determinism

@pytest.mark.parametrize("case", [wl.CONTRACT4, wl.SQDIST.scaled({"i": 1024, "j": 256, "k": 1024}),
                                  wl.MATMUL_F32.with_d(wl.matmul_d([1, 4, 4, 1]))], ids=["mfma", "valu", "split"])
def test_bitwise_reproducible(case):
    a, _ = run_gpu(case)
    b, _ = run_gpu(case)
    assert torch.equal(a, b)


# ------------------------------------------------------------ empty and ragged inputs

@pytest.mark.parametrize("idt,agg", [("f32", "sum"), ("f32", "max"), ("f32", "min"), ("f32", "lse"),
                                     ("i32", "sum"), ("i32", "max"), ("i32", "min")])
def test_empty_contracted_range_gives_the_identity(idt, agg):
    """The fold over no terms is the aggregate's identity; for int32 outputs
    the identity of max / min is the int32 extreme (the oracle's int64
    identity does not fit int32)."""
    join = "add" if agg in ("max", "min") else "mul"
    case = wl.EinsumCase("empty_j", 301, "ij,jk->ik", {"i": 3, "j": 0, "k": 5}, {"i": 3, "j": 1, "k": 1}, join,
                         agg, idt, idt, (("int", {"lo": -3, "hi": 3}),) * 2 if idt == "i32" else (wl.U11,) * 2,
                         2.0 if idt == "f32" else 1.0)
    xs = case.make_inputs()
    z, plan = run_gpu(case, xs)
    assert plan.kernel == "generic"
    want = ref.einsum(case.spec, xs[0], xs[1], join, agg, case.post_scale)
    if idt == "i32":
        want = np.clip(want, np.iinfo(np.int32).min, np.iinfo(np.int32).max)
        assert np.array_equal(z.numpy().astype(np.int64), want)
    else:
        assert np.array_equal(z.double().numpy(), want)


def test_empty_output_and_empty_repartition():
    case = wl.EinsumCase("empty_i", 302, "ij,jk->ik", {"i": 0, "j": 4, "k": 5}, {"i": 1, "j": 2, "k": 5}, "mul",
                         "sum", "f32", "f32", (wl.U11, wl.U11))
    z, plan = run_gpu(case)
    assert plan.kernel == "empty" and z.numel() == 0
    src = torch.empty(0, dtype=torch.float32, device=DEV)
    out = tra.tra_repartition(src, [0, 8], [1, 1], [1, 4])
    assert out.numel() == 0


RAGGED = {"i": 300, "j": 70, "k": 260}   # no tile divides these extents


@pytest.mark.parametrize("d", [{"i": 1, "j": 1, "k": 1}, {"i": 3, "j": 7, "k": 2}, {"i": 5, "j": 1, "k": 4}])
@pytest.mark.parametrize("base", [wl.SQDIST, wl.MAXPLUS, wl.MATMUL_F32, wl.GEMM25D],
                         ids=["sqdist", "maxplus", "matmul", "bf16gemm"])
def test_ragged_extents(base, d):
    """Extents no tile divides run on the untiled kernels (generic, or one
    wavefront per output when the contracted run is contiguous)."""
    err, plan = check(base.scaled(RAGGED, d))
    assert plan.kernel in ("generic", "rowreduce")


# ------------------------------------------------------------ transposed operands on the matrix cores

N002 = ("normal", {"std": 0.02})
SMALL_T = {"i": 1024, "j": 512, "k": 256}


@pytest.mark.parametrize("spec", ["ik,jk->ij", "ij,ik->jk", "ji,jk->ik", "ji,kj->ik"],
                         ids=["XYt", "XtY", "XtY2", "XtYt"])
@pytest.mark.parametrize("d", [{"i": 1, "j": 1, "k": 1}, {"i": 4, "j": 2, "k": 1}, {"i": 2, "j": 1, "k": 4}])
def test_transposed_operands_on_the_matrix_cores(spec, d):
    """Products whose operands are stored contiguous along an output label
    (X^T Y, X Y^T, X^T Y^T) run on the matrix-core kernel with transposing
    LDS reads for either operand."""
    case = wl.EinsumCase(f"t_{spec}", 61, spec, SMALL_T, d, "mul", "sum", "bf16", "f32", (N002, N002))
    err, plan = check(case)
    assert plan.kernel == "mfma_bf16"


K64_CASES = [
    # (spec, bounds, d, out dtype, post_scale): both operands contiguous along
    # the contracted label over at least 64 elements
    ("ik,jk->ij", {"i": 4096, "j": 2048, "k": 64}, {"i": 1, "j": 1, "k": 1}, "f32", 1.0),      # one k-tile
    ("ik,jk->ij", {"i": 4096, "j": 2048, "k": 128}, {"i": 2, "j": 2, "k": 2}, "f32", 1.0),    # blocked k
    ("ik,jk->ij", {"i": 2048, "j": 2048, "k": 1024}, {"i": 4, "j": 1, "k": 2}, "f32", 1.0),   # split 4 ways
    ("hsd,htd->hst", {"h": 4, "s": 512, "t": 512, "d": 128}, {"h": 2, "s": 1, "t": 2, "d": 1}, "bf16", 0.125),
    ("ik,jk->ij", {"i": 1024, "j": 1024, "k": 2048}, {"i": 1, "j": 1, "k": 1}, "bf16", 1.0),  # 32 k-tiles, split
]


@pytest.mark.parametrize("case", K64_CASES, ids=["one-ktile", "blocked-k", "split4", "batched-bf16", "long-k"])
def test_k_major_products_on_the_64_deep_tile(case):
    """Products whose operands are both K-major over 64 or more contiguous
    elements run on the four-wave tile with 64-deep stages (variant 4):
    parity with the oracle for one k-tile, blocked and split contracted
    ranges, a batch with bf16 output and a post-scale."""
    spec, bounds, d, odt, scale = case
    case = wl.EinsumCase(f"k64_{spec}", 64, spec, bounds, d, "mul", "sum", "bf16", odt, (N002, N002),
                         post_scale=scale)
    err, plan = check(case)
    assert plan.kernel == "mfma_bf16" and plan.info.tile == 4, (plan.kernel, plan.info.tile)


NARROW_CASES = [
    # (spec, bounds, d, out dtype): 128-wide outputs on the 64-deep tile's
    # 256 x 128 form (variant 5), all operand layouts, a blocked relation,
    # a batch and a split contracted range
    ("ik,jk->ij", {"i": 1024, "j": 128, "k": 512}, {"i": 1, "j": 1, "k": 1}, "f32"),
    ("ik,kj->ij", {"i": 2048, "j": 128, "k": 1024}, {"i": 2, "j": 1, "k": 2}, "bf16"),
    ("ki,kj->ij", {"i": 1024, "j": 128, "k": 256}, {"i": 1, "j": 1, "k": 1}, "f32"),
    ("ki,jk->ij", {"i": 512, "j": 128, "k": 256}, {"i": 1, "j": 1, "k": 1}, "f32"),
    ("hst,thd->shd", {"h": 4, "s": 512, "t": 512, "d": 128}, {"h": 2, "s": 1, "t": 2, "d": 1}, "bf16"),
    ("ik,jk->ij", {"i": 256, "j": 128, "k": 8192}, {"i": 1, "j": 1, "k": 1}, "f32"),
]


@pytest.mark.parametrize("case", NARROW_CASES, ids=["kk", "k-mn-blocked", "mn-mn", "mn-k",
                                                     "attention-weighted-sum", "split"])
def test_narrow_products_on_the_64_deep_tile(case):
    """Products whose output is 128 wide (or whose blocking leaves 128-wide
    column blocks) run on the 256 x 128 form of the 64-deep tile: parity with
    the oracle on every element for each operand layout, bf16 and fp32
    outputs, and a long contracted range split over workgroups."""
    spec, bounds, d, odt = case
    c = wl.EinsumCase(f"narrow_{spec}", 67, spec, bounds, d, "mul", "sum", "bf16", odt, (N002, N002))
    err, plan = check(c)
    assert plan.kernel == "mfma_bf16" and plan.info.tile == 5, (plan.kernel, plan.info.tile)


def test_narrow_tile_weighted_sum_without_split_sampled():
    """The attention weighted sum at 32 heads x 2048 queries x 1024 keys,
    head dimension 128: 256 narrow tiles, one per workgroup and no split,
    on 8192 sampled outputs spread over every tile."""
    c = wl.EinsumCase("narrow_weighted_sum", 68, "hst,thd->shd", {"h": 32, "s": 2048, "t": 1024, "d": 128},
                      {"h": 1, "s": 1, "t": 1, "d": 1}, "mul", "sum", "bf16", "bf16", (N002, N002))
    err, plan = check(c, sample=8192, seed=13)
    assert plan.kernel == "mfma_bf16" and plan.info.tile == 5 and plan.info.agg_split == 1


SHORT_CASES = [
    # (spec, bounds, d, post_scale): one or two 64-deep k-tiles, fp32 output,
    # more output tiles than compute units (the persistent tile loop)
    ("ik,jk->ij", {"i": 8192, "j": 4096, "k": 128}, {"i": 1, "j": 1, "k": 1}, 1.0),
    ("ik,jk->ij", {"i": 8192, "j": 4096, "k": 64}, {"i": 2, "j": 2, "k": 1}, 1.0),
    ("hsd,htd->hst", {"h": 8, "s": 2048, "t": 2048, "d": 128}, {"h": 2, "s": 2, "t": 1, "d": 1}, 0.088),
    ("ki,kj->ij", {"i": 4096, "j": 8192, "k": 128}, {"i": 1, "j": 1, "k": 1}, 1.0),
    ("ik,kj->ij", {"i": 8192, "j": 4096, "k": 128}, {"i": 2, "j": 1, "k": 2}, 1.0),
]


@pytest.mark.parametrize("case", SHORT_CASES, ids=["kk-two-ktiles", "kk-one-ktile-blocked", "scores-batched",
                                                    "mn-mn", "k-mn-blocked"])
def test_short_products_over_many_tiles(case):
    """Short contractions (64 or 128 deep) with fp32 output and 512 output
    tiles: each workgroup walks several tiles, overlapping one tile's stores
    with the next tile's copies and products.  16384 sampled outputs spread
    over every tile against the oracle, for all operand layouts."""
    spec, bounds, d, scale = case
    c = wl.EinsumCase(f"short_{spec}", 66, spec, bounds, d, "mul", "sum", "bf16", "f32", (N002, N002),
                      post_scale=scale)
    err, plan = check(c, sample=16384, seed=11)
    assert plan.kernel == "mfma_bf16" and plan.info.tile == 4, (plan.kernel, plan.info.tile)


@pytest.mark.parametrize("which", ["dX", "dA"])
def test_blocked_gemm_backward_full_size_sampled(which):
    """The blocked GEMM's backward products at full size: dX = dY A^T
    (16384 x 8192, sum over 8192) and dA = X^T dY (8192 x 8192, sum over
    16384), under the forward's blocking (i, j, k) = (16, 4, 4)."""
    b = {"i": 16384, "j": 8192, "k": 8192}
    d = {"i": 16, "j": 4, "k": 4}
    spec = "ik,jk->ij" if which == "dX" else "ij,ik->jk"
    case = wl.EinsumCase(f"gemm25d_{which}", 62 if which == "dX" else 63, spec, b, d, "mul", "sum", "bf16", "f32",
                         (N002, N002))
    err, plan = check(case, sample=2048, seed=5)
    assert plan.kernel == "mfma_bf16"


# ------------------------------------------------------------ two elementwise EinSums in one pass

CHAIN_CASES = [
    # (spec a, join a, in a, out a, spec b, join b, out b, bounds, d)
    ("hst,hs->hst", "sub", "f32", "bf16", "hst,hst->hst", "mul", "bf16", {"h": 4, "s": 64, "t": 512},
     {"h": 2, "s": 4, "t": 2}),
    ("hst,hs->hst", "exp_sub", "f32", "f32", "hst,hst->hst", "mul", "f32", {"h": 2, "s": 32, "t": 1024},
     {"h": 1, "s": 1, "t": 1}),
    ("ij,j->ij", "add", "bf16", "f32", "ij,ij->ij", "sub", "bf16", {"i": 128, "j": 256}, {"i": 4, "j": 2}),
    # extents without the power-of-two form: the one-thread-per-element chain
    ("hst,hs->hst", "sub", "f32", "bf16", "hst,hst->hst", "mul", "bf16", {"h": 3, "s": 20, "t": 384},
     {"h": 3, "s": 2, "t": 3}),
]


@pytest.mark.parametrize("case", CHAIN_CASES, ids=["sub-mul-bf16", "expsub-mul-f32", "add-sub-mixed", "ragged"])
def test_execute_chain_matches_two_launches(case):
    """z = b(xb, a(xa, ya)) in one pass is bit-identical to the two launches
    through an intermediate buffer."""
    spec_a, join_a, ia, oa, spec_b, join_b, ob, bounds, d = case
    pa = tra.tra_plan(spec_a, bounds, d, join_a, "none", ia, oa)
    pb = tra.tra_plan(spec_b, bounds, d, join_b, "none", oa, ob)
    assert pa.kernel == pb.kernel == "elemwise"
    g = torch.Generator().manual_seed(11)
    t_a = {"f32": torch.float32, "bf16": torch.bfloat16}
    xa = torch.randn(pa.info.x_elems, generator=g).to(t_a[ia]).to(DEV)
    ya = torch.randn(pa.info.y_elems, generator=g).to(t_a[ia]).to(DEV)
    xb = torch.randn(pb.info.x_elems, generator=g).to(t_a[oa]).to(DEV)
    t = tra.tra_execute(pa, xa, ya)
    want = tra.tra_execute(pb, xb, t)
    got = tra.tra_execute_chain(pa, pb, xa, ya, xb)
    torch.cuda.synchronize()
    assert torch.equal(got, want)


CONTRACT_CHAIN_CASES = [
    # (product spec, bounds, d, step a (spec, join), chain dtype, step b join);
    # enough output tiles that no plan splits its contracted range
    # the attention backward's softmax Jacobian: Attn * (dO.V^T - Rows), dense
    ("shd,thd->hst", {"s": 512, "t": 512, "h": 2, "d": 32}, {"s": 1, "t": 1, "h": 1, "d": 1},
     ("hst,hs->hst", "sub"), "bf16", "mul"),
    # the same, blocked: every label of the output cut in two
    ("shd,thd->hst", {"s": 512, "t": 512, "h": 2, "d": 32}, {"s": 2, "t": 2, "h": 2, "d": 1},
     ("hst,hs->hst", "sub"), "bf16", "mul"),
    # a column vector, fp32 chain, a one-tile (128 x 128) product
    ("ik,kj->ij", {"i": 128, "j": 128, "k": 32}, {"i": 1, "j": 2, "k": 1},
     ("ij,j->ij", "add"), "f32", "sqdiff"),
    # a full operand for the first step, a batched product with a K-major Y
    ("bik,bjk->bij", {"b": 4, "i": 256, "j": 256, "k": 32}, {"b": 2, "i": 1, "j": 1, "k": 1},
     ("bij,bij->bij", "mul"), "bf16", "sub"),
    # the Jacobian over four k-tiles and 128 output tiles of 256 x 256
    ("shd,thd->hst", {"s": 1024, "t": 1024, "h": 8, "d": 128}, {"s": 1, "t": 1, "h": 1, "d": 1},
     ("hst,hs->hst", "sub"), "bf16", "mul"),
    # the Jacobian with an fp32 chain, blocked rows
    ("shd,thd->hst", {"s": 1024, "t": 1024, "h": 8, "d": 64}, {"s": 2, "t": 1, "h": 1, "d": 1},
     ("hst,hs->hst", "sub"), "f32", "mul"),
]


@pytest.mark.parametrize("case", CONTRACT_CHAIN_CASES, ids=["jacobian", "jacobian-blocked", "colvec-f32", "full-op",
                                                          "jacobian-4k-tiles", "jacobian-f32"])
def test_execute_contract_chain_matches_three_launches(case):
    """A matrix-core product with two elementwise steps in its epilogue is
    bit-identical to the product, then the two steps, each launched alone."""
    spec_c, bounds, d, (spec_a, join_a), dt, join_b = case
    dd = {k: v for k, v in d.items()}
    pc = tra.tra_plan(spec_c, bounds, dd, "mul", "sum", "bf16", "f32")
    out = spec_c.split("->")[1]
    ba = {c: bounds[c] for c in set(spec_a.replace(",", "").replace("->", ""))}
    da = {c: d[c] for c in ba}
    pa = tra.tra_plan(spec_a, ba, da, join_a, "none", "f32", dt)
    pb = tra.tra_plan(f"{out},{out}->{out}", {c: bounds[c] for c in out}, {c: d[c] for c in out}, join_b, "none",
                      dt, dt)
    assert pc.kernel == "mfma_bf16" and pc.info.agg_split == 1, (pc.kernel, pc.info.agg_split)
    g = torch.Generator().manual_seed(12)
    t_a = {"f32": torch.float32, "bf16": torch.bfloat16}
    xc = torch.randn(pc.info.x_elems, generator=g).to(torch.bfloat16).to(DEV)
    yc = torch.randn(pc.info.y_elems, generator=g).to(torch.bfloat16).to(DEV)
    ya = torch.randn(pa.info.y_elems, generator=g).to(DEV)
    xb = torch.randn(pb.info.x_elems, generator=g).to(t_a[dt]).to(DEV)
    prod = tra.tra_execute(pc, xc, yc)
    t = tra.tra_execute(pa, prod, ya)
    want = tra.tra_execute(pb, xb, t)
    got = tra.tra_execute_contract_chain(pc, pa, pb, xc, yc, ya, xb)
    torch.cuda.synchronize()
    assert torch.equal(got, want)


# ------------------------------------------------------------ few outputs over long contracted ranges

U01 = ("uniform", {"lo": 0.0, "hi": 1.0})
REDUCE_CASES = [
    # (name, spec, bounds, d, join, agg, dtype, inputs)
    ("full_sum", "ij->", {"i": 4096, "j": 4096}, {"i": 1, "j": 1}, "ident", "sum", "f32", (U01,)),
    ("full_sum_blocked", "ij->", {"i": 4096, "j": 4096}, {"i": 4, "j": 8}, "ident", "sum", "f32", (U01,)),
    ("trace_of_product", "ij,ji->", {"i": 4096, "j": 4096}, {"i": 1, "j": 1}, "mul", "sum", "f32", (U01, U01)),
    ("row_max_int", "ij->i", {"i": 16, "j": 1 << 20}, {"i": 1, "j": 1}, "ident", "max", "i32",
     (("int", {"lo": -1000000, "hi": 1000000}),)),
    ("sum_int", "ij->", {"i": 2048, "j": 4096}, {"i": 2, "j": 1}, "ident", "sum", "i32",
     (("int", {"lo": -8, "hi": 8}),)),
    ("column_min", "ij->j", {"i": 65536, "j": 64}, {"i": 1, "j": 1}, "ident", "min", "f32",
     (("normal", {"std": 1.0}),)),
    ("lse_long_rows", "hst->hs", {"h": 4, "s": 16, "t": 65536}, {"h": 2, "s": 4, "t": 2}, "ident", "lse", "f32",
     (("normal", {"std": 3.0}),)),
    ("sqdist_bf16", "ij,ij->", {"i": 4096, "j": 4096}, {"i": 4, "j": 8}, "sqdiff", "sum", "bf16",
     (("normal", {"std": 1.0}),) * 2),
]


@pytest.mark.parametrize("case", REDUCE_CASES, ids=[c[0] for c in REDUCE_CASES])
def test_few_outputs_long_contracted_range(case):
    """A reduction to a handful of outputs is cut into chunks folded by whole
    workgroups (their waves combined in order through LDS), and the chunks'
    partials are folded in order by a second pass; against the oracle over
    every output, and bitwise reproducible."""
    name, spec, bounds, d, join, agg, dt, inputs = case
    c = wl.EinsumCase(name, 320 + REDUCE_CASES.index(case), spec, bounds, d, join, agg, dt,
                      "i32" if dt == "i32" else "f32", inputs)
    err, plan = check(c)
    assert plan.info.agg_split > 1 and plan.kernel in ("generic", "rowreduce"), plan.info.agg_split
    xs = c.make_inputs()
    a, _ = run_gpu(c, xs)
    b, _ = run_gpu(c, xs)
    assert torch.equal(a, b)


# ------------------------------------------------------------ masked edge tiles (ragged extents)

RAGGED_TILE_CASES = [
    # (name, spec, bounds, d, join, agg, dtype)
    ("sqdist_300x64x260", "ij,jk->ik", {"i": 300, "j": 64, "k": 260}, {"i": 1, "j": 1, "k": 1}, "sqdiff", "sum", "f32"),
    ("maxplus_300x64x260", "ij,jk->ik", {"i": 300, "j": 64, "k": 260}, {"i": 1, "j": 1, "k": 1}, "add", "max", "i32"),
    ("matmul_int_blocked", "ij,jk->ik", {"i": 300, "j": 64, "k": 260}, {"i": 3, "j": 2, "k": 1}, "mul", "sum", "i32"),
    ("sqdist_mn_major_blocked", "ji,jk->ik", {"i": 644, "j": 128, "k": 1000}, {"i": 7, "j": 4, "k": 5},
     "sqdiff", "sum", "f32"),
    ("matmul_k_major_split", "ij,kj->ik", {"i": 1000, "j": 512, "k": 100}, {"i": 5, "j": 2, "k": 1}, "mul", "sum",
     "f32"),
    ("minplus_narrow", "ij,kj->ik", {"i": 130, "j": 32, "k": 4}, {"i": 1, "j": 1, "k": 1}, "add", "min", "f32"),
]


@pytest.mark.parametrize("case", RAGGED_TILE_CASES, ids=[c[0] for c in RAGGED_TILE_CASES])
def test_ragged_extents_on_the_tile_kernel(case):
    """Output extents no tile divides, and relation blocks that are not powers
    of two, stay on the vector-ALU tile kernel: the last tile row and column
    read clamped rows and drop them at the store.  Every output against the
    oracle (integers exact)."""
    name, spec, bounds, d, join, agg, dt = case
    dist = ("int", {"lo": -1000, "hi": 1000}) if dt == "i32" and join == "add" else \
        (("int", {"lo": -8, "hi": 8}) if dt == "i32" else ("normal", {"std": 1.0}))
    c = wl.EinsumCase(name, 340 + RAGGED_TILE_CASES.index(case), spec, bounds, d, join, agg, dt, dt, (dist, dist))
    err, plan = check(c)
    assert plan.kernel == "valu_tile", plan.kernel


@pytest.mark.parametrize("base", [wl.SQDIST, wl.MAXPLUS], ids=["sqdist", "maxplus"])
def test_ragged_full_size_8000(base):
    """8000 x 256 x 8000 under d = [16,1,1,16] (relation blocks of 500 rows and
    columns) on the tile kernel, sampled outputs against the oracle."""
    c = base.scaled({"i": 8000, "j": 256, "k": 8000}, base.d)
    err, plan = check(c, sample=1 << 16, seed=8)
    assert plan.kernel == "valu_tile"
