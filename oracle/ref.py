"""The extended EinSum, written out as its definition (TEST INFRASTRUCTURE).

Page "EinDecomp：基于爱因斯坦求和与张量关系代数的自动张量并行分解算法", section 2.1:
labels on the right of an EinSum that are missing on the left are contracted;
the extension allows any associative and commutative aggregate (sum, max,
min, logsumexp) in place of the sum and any binary scalar function (such as
(x-y)^2) in place of the product.  For every output index z:

    Z[z] = post_scale * AGG_{c} JOIN(X[(z,c)|X], Y[(z,c)|Y])

Three independent evaluators of that one formula live here:

* ``einsum``        -- calls the nested-loop C code in einsum_ref.c (fp64 /
                       int64, OpenMP over output elements). This is the oracle
                       the GPU results are compared with and the one timed as
                       the CPU baseline.
* ``brute_einsum``  -- pure-Python loops over itertools.product, tiny shapes.
* ``dense_einsum``  -- numpy: every operand broadcast onto the full index
                       space of all labels, JOIN applied elementwise, AGG
                       applied over the contracted axes. Small shapes.

Joins: mul x*y, sqdiff (x-y)^2, add x+y, ident x (one operand),
exp_sub exp(x-y), sub x-y.  Aggregates: none, sum, max, min, lse.
Floating inputs are widened exactly to float64, integers to int64.
"""
from __future__ import annotations

import ctypes
import itertools
import math
import os
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import build as _build

JOINS = {"mul": 0, "sqdiff": 1, "add": 2, "ident": 3, "exp_sub": 4, "sub": 5}
AGGS = {"none": 0, "sum": 1, "max": 2, "min": 3, "lse": 4}

_lib = None


def _load():
    global _lib
    if _lib is None:
        # TRA_ORACLE_LIBRARY names another build of einsum_ref.c (the
        # sanitizer run of the CPU suite loads an ASan/UBSan build this way)
        path = os.environ.get("TRA_ORACLE_LIBRARY") or _build.LIB
        if not os.path.exists(path):
            path = _build.build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L = ctypes.c_int64
        lib.oracle_einsum_f64.argtypes = [I, P, I, P, P, I, P, P, I, P, I, P, I, I,
                                          ctypes.c_double, L, P, P, I]
        lib.oracle_einsum_i64.argtypes = [I, P, I, P, P, I, P, P, I, P, I, P, I, I,
                                          L, P, P, I]
        lib.oracle_einsum_f64.restype = I
        lib.oracle_einsum_i64.restype = I
        lib.oracle_max_threads.restype = I
        _lib = lib
    return _lib


def parse(spec: str) -> Tuple[List[str], str, List[str]]:
    """Split "ab,bc->ac" into operand label strings, output labels and the
    contracted labels in order of first appearance (X first, then Y)."""
    spec = spec.replace(" ", "")
    if "->" not in spec:
        raise ValueError(f"spec {spec!r} has no '->'")
    lhs, out = spec.split("->")
    ops = lhs.split(",")
    if not 1 <= len(ops) <= 2:
        raise ValueError("one or two operands")
    for o in ops + [out]:
        if len(set(o)) != len(o):
            raise ValueError(f"repeated label in {o!r}")
    seen = "".join(ops)
    for c in out:
        if c not in seen:
            raise ValueError(f"output label {c!r} is in no operand")
    contracted = []
    for c in seen:
        if c not in out and c not in contracted:
            contracted.append(c)
    return ops, out, contracted


def _as_np(t) -> np.ndarray:
    if hasattr(t, "numpy"):  # torch tensor
        import torch
        if t.dtype in (torch.int32, torch.int64):
            return t.to(torch.int64).numpy()
        return t.to(torch.float64).numpy()
    a = np.asarray(t)
    if a.dtype.kind in "iu":
        return a.astype(np.int64)
    return a.astype(np.float64)


def einsum(spec: str, x, y=None, join: str = "mul", agg: str = "sum",
           post_scale: float = 1.0, out_index: Optional[np.ndarray] = None,
           threads: int = 0) -> np.ndarray:
    """Evaluate the extended EinSum with the nested-loop C oracle.

    Returns float64 (float inputs) or int64 (integer inputs) with the output
    shape, or, when ``out_index`` (row-major flat output indices) is given,
    the 1-D array of just those elements.
    """
    ops, out, contracted = parse(spec)
    xa = np.ascontiguousarray(_as_np(x))
    ya = None if y is None else np.ascontiguousarray(_as_np(y))
    if (len(ops) == 2) != (ya is not None):
        raise ValueError("operand count does not match the spec")
    labels = sorted(set("".join(ops)))
    lid = {c: i for i, c in enumerate(labels)}
    bounds = np.zeros(len(labels), dtype=np.int64)
    for o, a in zip(ops, [xa] + ([ya] if ya is not None else [])):
        if a.ndim != len(o):
            raise ValueError(f"operand {o!r} has rank {a.ndim}")
        for c, n in zip(o, a.shape):
            if bounds[lid[c]] and bounds[lid[c]] != n:
                raise ValueError(f"label {c!r} has two extents")
            bounds[lid[c]] = n
    arr = lambda s: np.array([lid[c] for c in s], dtype=np.int32)
    xl, zl, cl = arr(ops[0]), arr(out), arr(contracted)
    yl = arr(ops[1]) if ya is not None else np.zeros(0, dtype=np.int32)
    out_shape = tuple(int(bounds[lid[c]]) for c in out)
    n_all = int(np.prod(out_shape, dtype=np.int64)) if out_shape else 1
    if out_index is None:
        n_out, oi = n_all, None
    else:
        oi = np.ascontiguousarray(np.asarray(out_index, dtype=np.int64))
        if oi.size and (oi.min() < 0 or oi.max() >= n_all):
            raise ValueError("out_index out of range")
        n_out = oi.size
    is_int = xa.dtype == np.int64
    if ya is not None and (ya.dtype == np.int64) != is_int:
        raise ValueError("mixed integer / float operands")
    lib = _load()
    ptr = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    ny = len(yl)
    if is_int:
        if post_scale != 1.0:
            raise ValueError("post_scale applies to floating point only")
        z = np.zeros(n_out, dtype=np.int64)
        rc = lib.oracle_einsum_i64(len(labels), ptr(bounds), len(xl), ptr(xl), ptr(xa),
                                   ny, ptr(yl) if ny else None, ptr(ya), len(zl), ptr(zl),
                                   len(cl), ptr(cl) if len(cl) else None,
                                   JOINS[join], AGGS[agg], n_out, ptr(oi), ptr(z), threads)
    else:
        z = np.zeros(n_out, dtype=np.float64)
        rc = lib.oracle_einsum_f64(len(labels), ptr(bounds), len(xl), ptr(xl), ptr(xa),
                                   ny, ptr(yl) if ny else None, ptr(ya), len(zl), ptr(zl),
                                   len(cl), ptr(cl) if len(cl) else None,
                                   JOINS[join], AGGS[agg], float(post_scale), n_out,
                                   ptr(oi), ptr(z), threads)
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return z if out_index is not None else z.reshape(out_shape)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


# ---------------------------------------------------------------- scalar ops

def _join(op: str, x, y):
    if op == "mul":
        return x * y
    if op == "sqdiff":
        return (x - y) * (x - y)
    if op == "add":
        return x + y
    if op == "ident":
        return x
    if op == "exp_sub":
        return math.exp(x - y)
    if op == "sub":
        return x - y
    raise ValueError(op)


INT64_MIN, INT64_MAX = -(1 << 63), (1 << 63) - 1


def brute_einsum(spec: str, x, y=None, join: str = "mul", agg: str = "sum",
                 post_scale: float = 1.0) -> np.ndarray:
    """Pure-Python loops over every label: for tiny shapes only."""
    ops, out, contracted = parse(spec)
    arrs = [_as_np(x)] + ([] if y is None else [_as_np(y)])
    is_int = arrs[0].dtype == np.int64
    ext: Dict[str, int] = {}
    for o, a in zip(ops, arrs):
        for c, n in zip(o, a.shape):
            ext[c] = n
    res = np.zeros(tuple(ext[c] for c in out), dtype=np.int64 if is_int else np.float64)
    for zi in itertools.product(*[range(ext[c]) for c in out]):
        terms = []
        for ci in itertools.product(*[range(ext[c]) for c in contracted]):
            env = dict(zip(out, zi))
            env.update(zip(contracted, ci))
            xv = arrs[0][tuple(env[c] for c in ops[0])].item()
            yv = arrs[1][tuple(env[c] for c in ops[1])].item() if len(arrs) == 2 else 0
            terms.append(_join(join, xv, yv))
        if agg == "none":
            if contracted:
                raise ValueError("aggregate none with contracted labels")
            v = terms[0]
        # a fold over no terms (an empty contracted range) is the identity
        elif agg == "sum":
            v = sum(terms)
        elif agg == "max":
            v = max(terms, default=INT64_MIN if is_int else -math.inf)
        elif agg == "min":
            v = min(terms, default=INT64_MAX if is_int else math.inf)
        elif agg == "lse":
            m = max(terms, default=-math.inf)
            v = m if m == -math.inf else m + math.log(sum(math.exp(t - m) for t in terms))
        else:
            raise ValueError(agg)
        res[zi] = v if is_int else post_scale * v
    return res


def dense_einsum(spec: str, x, y=None, join: str = "mul", agg: str = "sum",
                 post_scale: float = 1.0) -> np.ndarray:
    """numpy: broadcast onto the full index space of all labels, then reduce.

    Memory is the product of all extents, so this is for small shapes.
    """
    ops, out, contracted = parse(spec)
    arrs = [_as_np(x)] + ([] if y is None else [_as_np(y)])
    is_int = arrs[0].dtype == np.int64
    full = list(out) + list(contracted)
    ext: Dict[str, int] = {}
    for o, a in zip(ops, arrs):
        for c, n in zip(o, a.shape):
            ext[c] = n

    def lift(a, labels):
        # transpose the operand's axes into `full` order, insert size-1 axes
        perm = [labels.index(c) for c in full if c in labels]
        b = np.transpose(a, perm)
        shape = [ext[c] if c in labels else 1 for c in full]
        return b.reshape(shape)

    xv = lift(arrs[0], ops[0])
    yv = lift(arrs[1], ops[1]) if len(arrs) == 2 else np.zeros(1, dtype=xv.dtype)
    if join == "mul":
        v = xv * yv
    elif join == "sqdiff":
        v = (xv - yv) ** 2
    elif join == "add":
        v = xv + yv
    elif join == "ident":
        v = xv + 0 * yv
    elif join == "exp_sub":
        v = np.exp(xv - yv)
    elif join == "sub":
        v = xv - yv
    else:
        raise ValueError(join)
    v = np.broadcast_to(v, tuple(ext[c] for c in full))
    axes = tuple(range(len(out), len(full)))
    if agg == "none":
        if contracted:
            raise ValueError("aggregate none with contracted labels")
        r = np.array(v)
    elif agg == "sum":
        r = v.sum(axis=axes)
    elif agg == "max":
        r = v.max(axis=axes)
    elif agg == "min":
        r = v.min(axis=axes)
    elif agg == "lse":
        m = v.max(axis=axes, keepdims=True)
        with np.errstate(invalid="ignore"):
            s = np.exp(v - m).sum(axis=axes)
        m = m.reshape(s.shape)
        r = np.where(np.isneginf(m), m, m + np.log(s))
    else:
        raise ValueError(agg)
    r = np.asarray(r, dtype=np.int64 if is_int else np.float64)
    return r if is_int else post_scale * r
