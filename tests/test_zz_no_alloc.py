"""tra_execute_static (the entry point that allocates nothing: the plan's
scratch lives in the library's fixed per-device array) against tra_execute
with a caller-provided workspace, through the C ABI, on the same inputs:
results identical bit for bit, over two calls in a row whose second is
smaller (the array keeps the first call's contents), for each kind of
scratch the kernels use; a plan needing more scratch than the array holds is
refused before anything is launched."""
import pytest
import torch

import tensor_relational_algebra_amd as tra
from tensor_relational_algebra_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _pair(spec, bounds, d, join, agg, idt, odt, seed, dist=("normal", {"std": 1.0})):
    p = tra.tra_plan(spec, bounds, d, join, agg, idt, odt)
    ops = spec.split("->")[0].split(",")
    xs = [wl.draw(seed + i, [bounds[c] for c in o], dist[0], idt, **dist[1]).to(DEV) for i, o in enumerate(ops)]
    rel = [tra.to_relation(x, [d[c] for c in o]) for x, o in zip(xs, ops)]
    z_ref = tra.tra_execute(p, rel[0], rel[1] if len(rel) > 1 else None)
    z = torch.full_like(z_ref, 7)
    tra.tra_execute_static(p, rel[0], rel[1] if len(rel) > 1 else None, z)
    torch.cuda.synchronize()
    return p, z, z_ref


def test_scratch_array_size():
    assert tra.tra_static_scratch_bytes() == 16 << 20


@pytest.mark.parametrize("sizes", [(1024, 256), (512, 128)], ids=["1024-then-256", "512-then-128"])
def test_split_aggregation_partials_two_calls_second_smaller(sizes):
    for n in sizes:
        p, z, z_ref = _pair("ij,jk->ik", {"i": n, "j": n, "k": n}, {"i": 1, "j": 1, "k": 1}, "mul", "sum",
                            "f32", "f32", 8100 + n, ("uniform", {"lo": -1.0, "hi": 1.0}))
        assert p.info.agg_split > 1 and 0 < p.info.workspace_bytes <= tra.tra_static_scratch_bytes()
        assert torch.equal(z, z_ref), n


def test_matrix_core_split_and_int_max_plus_flags():
    for n in (1024, 512):
        p, z, z_ref = _pair("ij,jk->ik", {"i": 256, "j": n, "k": 256}, {"i": 1, "j": 1, "k": 1}, "mul", "sum",
                            "bf16", "f32", 8200 + n, ("normal", {"std": 0.1}))
        assert p.kernel == "mfma_bf16" and p.info.agg_split > 1
        assert torch.equal(z, z_ref), n
    for n in (512, 256):
        p, z, z_ref = _pair("ij,jk->ik", {"i": n, "j": 128, "k": n}, {"i": 2, "j": 1, "k": 2}, "add", "max",
                            "i32", "i32", 8300 + n, ("int", {"lo": -1000, "hi": 1000}))
        assert p.info.tile == 1 and p.info.workspace_bytes > 0
        assert torch.equal(z, z_ref), n


def test_plan_without_scratch_and_too_large_a_plan():
    p, z, z_ref = _pair("ij,jk->ik", {"i": 2048, "j": 256, "k": 2048}, {"i": 2, "j": 1, "k": 2}, "sqdiff", "sum",
                        "f32", "f32", 8400)
    assert p.info.workspace_bytes == 0 and torch.equal(z, z_ref)
    # one output tile over a long contracted range: split 128 ways, 32 MiB of partials
    big = tra.tra_plan("ij,jk->ik", {"i": 256, "j": 8192, "k": 256}, {"i": 1, "j": 1, "k": 1}, "mul", "sum",
                       "bf16", "f32")
    assert big.info.workspace_bytes > tra.tra_static_scratch_bytes()
    x = torch.zeros(256 * 8192, dtype=torch.bfloat16, device=DEV)
    y = torch.zeros(8192 * 256, dtype=torch.bfloat16, device=DEV)
    out = torch.full((256 * 256,), 5.0, dtype=torch.float32, device=DEV)
    with pytest.raises(tra.TraError) as e:
        tra.tra_execute_static(big, x, y, out)
    assert e.value.code == -8
    torch.cuda.synchronize()
    assert torch.all(out == 5.0)      # refused before anything ran
