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


# (case, kernel, compared elements, max-norm error, floored element-wise error),
# printed at the end of the session by conftest.py
REPORT = []
FLOOR = 1e-2


def maxnorm_rel_err(got: np.ndarray, want: np.ndarray) -> float:
    """max |g - r| / max |r| over the compared elements."""
    den = float(np.abs(want).max()) if want.size else 1.0
    return float(np.abs(got.astype(np.float64) - want).max()) / max(den, 1e-300)


def floored_rel_err(got: np.ndarray, want: np.ndarray, floor: float = FLOOR) -> float:
    """max |g - r| / |r| over the elements with |r| >= floor * max |r|: the
    element-wise relative error, ill-posed where r is near 0, so taken only
    where r is not small against the tensor's scale."""
    want = np.asarray(want, dtype=np.float64)
    if not want.size:
        return 0.0
    big = float(np.abs(want).max())
    mask = np.abs(want) >= floor * big
    if not mask.any():
        return 0.0
    g = np.asarray(got, dtype=np.float64)[mask]
    return float((np.abs(g - want[mask]) / np.abs(want[mask])).max())


def gate(name: str, kernel: str, got: np.ndarray, want: np.ndarray, tol: float,
         elementwise_tol: "float | None" = None) -> float:
    """The max-norm relative error against `tol` (the gate the tolerances are
    stated for); the floored element-wise error is recorded for the session
    report beside it, and held to `elementwise_tol` when one is given."""
    got = np.asarray(got, dtype=np.float64).reshape(-1)
    want = np.asarray(want, dtype=np.float64).reshape(-1)
    err = maxnorm_rel_err(got, want)
    fl = floored_rel_err(got, want)
    REPORT.append((name, kernel, int(want.size), err, fl))
    assert err <= tol, f"{name} via {kernel}: max-norm relative error {err:.3g} > {tol}"
    if elementwise_tol is not None:
        assert fl <= elementwise_tol, f"{name} via {kernel}: floored element-wise relative error {fl:.3g}"
    return err


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
    # bf16 inputs are exact and their products exact in fp32, so the error is
    # fp32 accumulation only and the element-wise bound holds too; fp32 sums
    # of cancelling terms are gated on the max-norm alone
    tol = TOL[case.in_dtype]
    err = gate(f"{case.name} d={d or case.d}", plan.kernel, got.to(torch.float64).numpy(), want, tol,
               elementwise_tol=tol if case.in_dtype == "bf16" else None)
    return err, plan
