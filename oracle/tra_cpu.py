"""Tensor-relational algebra taken literally (TEST INFRASTRUCTURE).

Page "EinDecomp：基于爱因斯坦求和与张量关系代数的自动张量并行分解算法", section 2.2:

* Partition rule: a tensor of shape [B1, B2, ...] under a partition vector
  d = [D1, D2, ...] (each Di dividing Bi) is a relation with D1*D2*... entries;
  the entry with key k = [k1, k2, ...] is the sub-tensor of shape
  [B1/D1, B2/D2, ...] covering [k1*B1/D1, (k1+1)*B1/D1) x [k2*B2/D2, ...) ...
* Join: every pair of sub-tensors whose keys agree on the shared EinSum
  labels is fed to a kernel function that yields a new sub-tensor.
* Aggregation: the join results are grouped by the output (non-contracted)
  part of the key and reduced inside each group by the aggregate.
* Repartition: the same tensor re-cut under another partition vector.
* EinSum -> TRA: cut X and Y by d, join all key-matched pairs, aggregate over
  the output labels.

Relations here are Python dicts {key tuple: numpy block}.  The kernel
function applied to a block pair is the same extended EinSum on the blocks
(``ref.dense_einsum``); partials of one group are folded in ascending order of
the contracted part of the key with the aggregate's binary form (sum: +,
max / min, lse: logaddexp).

The flat buffer layout (``to_buffer`` / ``from_buffer``) is how one relation
sits in one linear allocation: the sub-tensors one after another in row-major
order of their key, each stored dense row-major.  The pages leave storage
open; this is the layout the GPU path is specified to use, so a tensor under
d = all-ones is its ordinary dense row-major array.
"""
from __future__ import annotations

import itertools
from typing import Dict, List, Sequence, Tuple

import numpy as np

from . import ref

Rel = Dict[Tuple[int, ...], np.ndarray]


def _check(shape: Sequence[int], d: Sequence[int]) -> None:
    if len(shape) != len(d):
        raise ValueError("partition vector length differs from the rank")
    for b, k in zip(shape, d):
        if k < 1 or b % k:
            raise ValueError(f"{k} does not divide {b}")


def partition(t: np.ndarray, d: Sequence[int]) -> Rel:
    """Cut a dense tensor into {key: sub-tensor} by the partition rule."""
    _check(t.shape, d)
    blk = [b // k for b, k in zip(t.shape, d)]
    rel: Rel = {}
    for key in itertools.product(*[range(k) for k in d]):
        sl = tuple(slice(ki * bi, (ki + 1) * bi) for ki, bi in zip(key, blk))
        rel[key] = np.array(t[sl])
    return rel


def merge(rel: Rel, shape: Sequence[int], d: Sequence[int]) -> np.ndarray:
    """Put the sub-tensors of a relation back into one dense tensor."""
    _check(shape, d)
    blk = [b // k for b, k in zip(shape, d)]
    first = next(iter(rel.values()))
    out = np.zeros(tuple(shape), dtype=first.dtype)
    for key, sub in rel.items():
        sl = tuple(slice(ki * bi, (ki + 1) * bi) for ki, bi in zip(key, blk))
        out[sl] = sub
    return out


def to_buffer(t: np.ndarray, d: Sequence[int]) -> np.ndarray:
    """The flat relation layout: blocks in row-major key order, each row-major."""
    rel = partition(t, d)
    keys = sorted(rel)  # lexicographic == row-major order of the key vector
    return np.concatenate([rel[k].reshape(-1) for k in keys]) if keys else np.zeros(0, t.dtype)


def from_buffer(buf: np.ndarray, shape: Sequence[int], d: Sequence[int]) -> np.ndarray:
    """Inverse of ``to_buffer``: read the blocks back in key order."""
    _check(shape, d)
    blk = tuple(b // k for b, k in zip(shape, d))
    vol = int(np.prod(blk, dtype=np.int64))
    keys = sorted(itertools.product(*[range(k) for k in d]))
    if buf.size != vol * len(keys):
        raise ValueError("buffer size does not match the shape")
    rel = {k: buf[i * vol:(i + 1) * vol].reshape(blk) for i, k in enumerate(keys)}
    return merge(rel, shape, d)


def repartition_buffer(buf: np.ndarray, shape: Sequence[int], d_from: Sequence[int],
                       d_to: Sequence[int]) -> np.ndarray:
    """Re-cut a flat relation from d_from to d_to (through the dense tensor)."""
    return to_buffer(from_buffer(buf, shape, d_from), d_to)


def _combine(agg: str, a: np.ndarray, b: np.ndarray) -> np.ndarray:
    if agg == "sum":
        return a + b
    if agg == "max":
        return np.maximum(a, b)
    if agg == "min":
        return np.minimum(a, b)
    if agg == "lse":
        return np.logaddexp(a, b)
    raise ValueError(f"aggregate {agg!r} has no binary form")


def tra_einsum(spec: str, x, y, dmap: Dict[str, int], join: str = "mul", agg: str = "sum",
               post_scale: float = 1.0) -> np.ndarray:
    """EinSum -> TRA plan -> result, following the page's three steps.

    ``dmap`` gives the number of partitions of every label.  Returns the dense
    float64 / int64 result (the output relation merged back).
    """
    ops, out, contracted = ref.parse(spec)
    arrs = [ref._as_np(x)] + ([] if y is None else [ref._as_np(y)])
    rels = [partition(a, [dmap[c] for c in o]) for o, a in zip(ops, arrs)]
    labels = list(out) + list(contracted)

    # Join: all key tuples over the labels of X and Y; each names one matched pair.
    partials: Dict[Tuple[int, ...], np.ndarray] = {}
    for kappa in itertools.product(*[range(dmap[c]) for c in labels]):
        env = dict(zip(labels, kappa))
        blocks = [rel[tuple(env[c] for c in o)] for o, rel in zip(ops, rels)]
        partials[kappa] = ref.dense_einsum(spec, blocks[0], blocks[1] if len(blocks) == 2 else None,
                                           join, agg, 1.0)

    # Aggregation: group by the output part of the key, ascending contracted key.
    groups: Rel = {}
    for kappa in sorted(partials):
        zk = kappa[:len(out)]
        if zk in groups:
            if agg == "none":
                raise ValueError("aggregate none with more than one partial")
            groups[zk] = _combine(agg, groups[zk], partials[kappa])
        else:
            groups[zk] = partials[kappa]
    ext = {c: n for o, a in zip(ops, arrs) for c, n in zip(o, a.shape)}
    shape = [ext[c] for c in out]
    z = merge(groups, shape, [dmap[c] for c in out])
    if z.dtype == np.int64:
        return z
    return post_scale * z


def task_counts(spec: str, dmap: Dict[str, int]) -> Tuple[int, int, int]:
    """(join tasks N, aggregation groups G, partials per group n_agg)."""
    ops, out, contracted = ref.parse(spec)
    n_agg = int(np.prod([dmap[c] for c in contracted], dtype=np.int64)) if contracted else 1
    g = int(np.prod([dmap[c] for c in out], dtype=np.int64)) if out else 1
    return g * n_agg, g, n_agg


def buffer_offset(g: Sequence[int], shape: Sequence[int], d: Sequence[int]) -> int:
    """Position of the element with global index g in the flat relation buffer:
    its sub-tensor's key k = g // b comes first (row-major over d, times the
    sub-tensor volume), then its place r = g % b inside the sub-tensor."""
    _check(shape, d)
    b = [s // k for s, k in zip(shape, d)]
    key = [gi // bi for gi, bi in zip(g, b)]
    r = [gi % bi for gi, bi in zip(g, b)]
    vol = 1
    for bi in b:
        vol *= bi
    kpos = 0
    for ki, di in zip(key, d):
        kpos = kpos * di + ki
    rpos = 0
    for ri, bi in zip(r, b):
        rpos = rpos * bi + ri
    return kpos * vol + rpos
