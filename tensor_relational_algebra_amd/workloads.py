"""Seeded synthetic workloads: shapes, partition vectors and input generators.

This module holds no arithmetic of the method. It only draws the input
tensors (from numpy's PCG64 with a fixed seed per tensor), rounds them to the
storage dtype the workload names, and lists the workload shapes. Both the GPU
path's tests/bench and the oracle's callers take their inputs from here, so
that the two sides see bit-identical operands.

Seed rule: seed = 1000 * workload_id + tensor_index.
Distributions: ``uniform(lo, hi)`` is continuous on [lo, hi); ``normal(std)``
is ``standard_normal() * std`` drawn in float32; ``int(lo, hi)`` is uniform on
the inclusive integer range. bf16 tensors are drawn in float32 and rounded to
bfloat16 with round-to-nearest-even (torch's conversion).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

# Workload ids used in the seed rule.
WL_MATMUL_F32 = 1
WL_MATMUL_I32 = 11
WL_SQDIST = 2
WL_MAXPLUS = 12
WL_CONTRACT4 = 3
WL_MHA = 4
WL_GEMM25D = 5


def draw(seed: int, shape: Sequence[int], dist: str, dtype: str,
         lo: float = -1.0, hi: float = 1.0, std: float = 1.0) -> torch.Tensor:
    """Draw one tensor on the host.

    dist: 'uniform' (continuous [lo, hi)), 'normal' (N(0, std)), 'int'
    (integers in [lo, hi] inclusive).  dtype: 'f32', 'bf16' or 'i32'.
    Returns a contiguous CPU torch tensor of that dtype.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = tuple(int(s) for s in shape)
    if dist == "int":
        a = rng.integers(int(lo), int(hi), size=shape, endpoint=True, dtype=np.int32)
        if dtype != "i32":
            raise ValueError("integer draws are stored as i32")
        return torch.from_numpy(np.ascontiguousarray(a))
    if dist == "uniform":
        a = rng.uniform(lo, hi, size=shape).astype(np.float32)
    elif dist == "normal":
        a = (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "f32":
        return t
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    raise ValueError(f"float draw cannot be stored as {dtype!r}")


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a host tensor (f32 / bf16 / i32) to float64 or int64."""
    if t.dtype in (torch.int32, torch.int64):
        return t.to(torch.int64).numpy()
    return t.to(torch.float64).numpy()


@dataclasses.dataclass(frozen=True)
class EinsumCase:
    """One extended-EinSum node with its sizes and a partition vector.

    ``bounds`` and ``d`` map each label to its extent and its number of
    partitions.  ``inputs`` lists, per operand, (dist, kwargs) for ``draw``.
    """
    name: str
    wid: int
    spec: str
    bounds: Dict[str, int]
    d: Dict[str, int]
    join: str
    agg: str
    in_dtype: str
    out_dtype: str
    inputs: Tuple[Tuple[str, dict], ...]
    post_scale: float = 1.0

    def operand_labels(self) -> List[str]:
        return self.spec.split("->")[0].split(",")

    def out_labels(self) -> str:
        return self.spec.split("->")[1]

    def shape(self, labels: str) -> Tuple[int, ...]:
        return tuple(self.bounds[c] for c in labels)

    def make_inputs(self) -> List[torch.Tensor]:
        out = []
        for t, (labels, (dist, kw)) in enumerate(zip(self.operand_labels(), self.inputs)):
            out.append(draw(1000 * self.wid + t, self.shape(labels), dist, self.in_dtype, **kw))
        return out

    def with_d(self, d: Dict[str, int], name: Optional[str] = None) -> "EinsumCase":
        return dataclasses.replace(self, d=dict(d), name=name or self.name)

    def scaled(self, bounds: Dict[str, int], d: Optional[Dict[str, int]] = None,
               name: Optional[str] = None) -> "EinsumCase":
        nd = dict(self.d if d is None else d)
        return dataclasses.replace(self, bounds=dict(bounds), d=nd, name=name or self.name + "_small")


def matmul_d(d4: Sequence[int]) -> Dict[str, int]:
    """The per-operand matmul vector [d_i, d_j(X), d_j(Y), d_k] as a per-label map."""
    di, djx, djy, dk = d4
    if djx != djy:
        raise ValueError("the two occurrences of j must be split alike")
    return {"i": di, "j": djx, "k": dk}


U11 = ("uniform", {"lo": -1.0, "hi": 1.0})

# Partitioned matmul, 256^3, three partition vectors.
MATMUL_F32 = EinsumCase("matmul_f32", WL_MATMUL_F32, "ij,jk->ik",
                        {"i": 256, "j": 256, "k": 256}, matmul_d([4, 1, 1, 4]),
                        "mul", "sum", "f32", "f32", (U11, U11))
MATMUL_I32 = EinsumCase("matmul_i32", WL_MATMUL_I32, "ij,jk->ik",
                        {"i": 256, "j": 256, "k": 256}, matmul_d([4, 1, 1, 4]),
                        "mul", "sum", "i32", "i32",
                        (("int", {"lo": -8, "hi": 8}), ("int", {"lo": -8, "hi": 8})))
MATMUL_D4 = ([4, 1, 1, 4], [1, 4, 4, 1], [2, 2, 2, 2])

# Pairwise squared distance and max-plus product, 8192 x 256 x 8192.
SQDIST = EinsumCase("sqdist", WL_SQDIST, "ij,jk->ik",
                    {"i": 8192, "j": 256, "k": 8192}, matmul_d([16, 1, 1, 16]),
                    "sqdiff", "sum", "f32", "f32",
                    (("normal", {"std": 1.0}), ("normal", {"std": 1.0})))
MAXPLUS = EinsumCase("maxplus", WL_MAXPLUS, "ij,jk->ik",
                     {"i": 8192, "j": 256, "k": 8192}, matmul_d([16, 1, 1, 16]),
                     "add", "max", "i32", "i32",
                     (("int", {"lo": -1000, "hi": 1000}), ("int", {"lo": -1000, "hi": 1000})))

# Four-index contraction C[a,b,c,d] = sum_e sum_f A[a,b,e,f] B[c,f,e,d].
CONTRACT4 = EinsumCase("contract4", WL_CONTRACT4, "abef,cfed->abcd",
                       {"a": 64, "b": 64, "c": 64, "d": 64, "e": 32, "f": 32},
                       {"a": 2, "b": 2, "c": 2, "d": 2, "e": 4, "f": 4},
                       "mul", "sum", "bf16", "f32",
                       (("normal", {"std": 0.1}), ("normal", {"std": 0.1})))

# Blocked GEMM Y = X A, X 16384 x 8192 in 16 x 4 blocks, A 8192 x 8192 in 4 x 4.
GEMM25D = EinsumCase("gemm25d", WL_GEMM25D, "ij,jk->ik",
                     {"i": 16384, "j": 8192, "k": 8192}, {"i": 16, "j": 4, "k": 4},
                     "mul", "sum", "bf16", "f32",
                     (("normal", {"std": 0.02}), ("normal", {"std": 0.02})))
GEMM25D_Y_FROM = (16, 4)
GEMM25D_Y_TO = (4, 16)


@dataclasses.dataclass(frozen=True)
class MhaCase:
    """One multi-head attention layer written as EinSum nodes."""
    s: int = 4096
    a: int = 4096
    h: int = 32
    dh: int = 128
    wid: int = WL_MHA

    def graph_desc(self) -> str:
        """The layer as an EinGraph in the node-per-line format of the C ABI.

        Storage dtypes: the inputs, weights and the projected / weighted
        tensors are bf16; scores and their logsumexp are fp32; the output is
        fp32.  The score node carries the 1/sqrt(dh) scale."""
        s, a, h, d = self.s, self.a, self.h, self.dh
        pb = f"s={s},a={a},h={h},d={d}"
        return "\n".join([
            f"Q_proj einsum sa,ahd->shd {pb} @Q,@W_Q in=bf16 out=bf16",
            f"K_proj einsum sa,ahd->shd {pb} @K,@W_K in=bf16 out=bf16",
            f"V_proj einsum sa,ahd->shd {pb} @V,@W_V in=bf16 out=bf16",
            f"Scores einsum shd,thd->hst s={s},t={s},h={h},d={d} Q_proj,K_proj in=bf16 out=f32 "
            f"scale={1.0 / math.sqrt(d)!r}",
            f"Attn softmax hst->hst h={h},s={s},t={s} Scores in=f32 out=bf16",
            f"O einsum hst,thd->shd h={h},s={s},t={s},d={d} Attn,V_proj in=bf16 out=bf16",
            f"Output einsum shd,ahd->sa s={s},h={h},d={d},a={a} O,@W_O in=bf16 out=f32",
        ])

    def make_inputs(self) -> Dict[str, torch.Tensor]:
        t = {}
        for i, name in enumerate(("Q", "K", "V")):
            t[name] = draw(1000 * self.wid + i, (self.s, self.a), "normal", "bf16", std=1.0)
        for i, name in enumerate(("W_Q", "W_K", "W_V", "W_O")):
            t[name] = draw(1000 * self.wid + 3 + i, (self.a, self.h, self.dh), "normal", "bf16", std=0.02)
        return t

    def make_output_gradient(self) -> torch.Tensor:
        """dL/dOutput [s, a] for the backward pass: bf16 N(0, 1), tensor index 7."""
        return draw(1000 * self.wid + 7, (self.s, self.a), "normal", "bf16", std=1.0)


MHA = MhaCase()
MHA_SMALL = MhaCase(s=128, a=128, h=4, dh=32)
