"""Helpers for the GPU parity tests: run one EinSum case through the C ABI
(dense -> relation, join + aggregation, relation -> dense) and compare with
the CPU oracle on the same seeded inputs."""
import numpy as np
import torch

import tensor_relational_algebra_amd as tra
from oracle import ref
from tensor_relational_algebra_amd import workloads as wl

DEV = torch.device("cuda:0")
TOL = {"f32": 1e-4, "bf16": 2e-2}


def maxnorm_rel_err(got: np.ndarray, want: np.ndarray) -> float:
    """max |g - r| / max |r| over the compared elements."""
    den = float(np.abs(want).max()) if want.size else 1.0
    return float(np.abs(got.astype(np.float64) - want).max()) / max(den, 1e-300)


def run_gpu(case: wl.EinsumCase, inputs=None, d=None):
    """Returns (dense output on the host, plan)."""
    d = dict(case.d if d is None else d)
    ops = case.operand_labels()
    xs = case.make_inputs() if inputs is None else inputs
    plan = tra.tra_plan(case.spec, case.bounds, d, case.join, case.agg, case.in_dtype, case.out_dtype,
                        case.post_scale)
    rels = [tra.to_relation(t.to(DEV), [d[c] for c in o]) for t, o in zip(xs, ops)]
    zr = tra.tra_execute(plan, rels[0], rels[1] if len(rels) > 1 else None)
    out = case.out_labels()
    if out:
        z = tra.from_relation(zr, [case.bounds[c] for c in out], [d[c] for c in out])
    else:
        z = zr.reshape(())
    torch.cuda.synchronize()
    return z.cpu(), plan


def check(case: wl.EinsumCase, d=None, sample: int = 0, seed: int = 0, inputs=None):
    """Compare the GPU result with the oracle: every element, or `sample`
    random output elements.  Integers bit-exact; floats to the max-norm
    relative tolerance of their input dtype."""
    xs = case.make_inputs() if inputs is None else inputs
    z, plan = run_gpu(case, xs, d)
    y = xs[1] if len(xs) > 1 else None
    zf = z.reshape(-1)
    if sample:
        rng = np.random.default_rng(seed)
        idx = np.sort(rng.choice(zf.numel(), size=min(sample, zf.numel()), replace=False))
        want = ref.einsum(case.spec, xs[0], y, case.join, case.agg, case.post_scale, out_index=idx)
        got = zf[torch.from_numpy(idx)]
    else:
        want = ref.einsum(case.spec, xs[0], y, case.join, case.agg, case.post_scale).reshape(-1)
        got = zf
    if case.out_dtype == "i32":
        g = got.numpy().astype(np.int64)
        bad = np.nonzero(g != want)[0]
        assert bad.size == 0, f"{case.name} d={d or case.d} via {plan.kernel}: {bad.size} mismatches, first at {bad[:5]}"
        return 0.0, plan
    err = maxnorm_rel_err(got.to(torch.float64).numpy(), want)
    tol = TOL[case.in_dtype]
    assert err <= tol, f"{case.name} d={d or case.d} via {plan.kernel}: max-norm relative error {err:.3g} > {tol}"
    return err, plan
