"""One multi-head attention layer, forward and backward, as a fixed sequence of
extended EinSums run through tra_plan / tra_execute (every step is one launch
of the library's kernels; this module only plans the steps and hands device
buffers from one step to the next).

Page "EinDecomp：基于爱因斯坦求和与张量关系代数的自动张量并行分解算法",
section 2.1 writes the layer's forward as EinSums (projections, scores,
softmax, weighted sum, output projection).  The backward is the chain rule of
those EinSums, one EinSum per step, with two joins beyond the product:

* the softmax Jacobian, dScores = Attn * (dAttn - r), where the row term
  r[h,s] = sum_t Attn[h,s,t] dAttn[h,s,t] equals sum_d dO[s,h,d] O[s,h,d]
  (both are the derivative of the layer output along one query row and head),
  so r is formed from [s,h,d] tensors instead of a second pass over [h,s,t];
* dAttn - r is the join sub with r broadcast over t, formed in fp32 from the
  fp32 product dAttn and stored in bf16; the Jacobian then multiplies it by
  the forward's stored bf16 Attn (as the autograd of a bf16 softmax does, from
  its saved output), so the backward never re-reads the fp32 scores.

Storage dtypes follow the forward EinGraph: operands of the matrix-core
products are bf16, the product dAttn that feeds the subtraction is fp32,
weight and input gradients are fp32.  Of the [h,s,t] tensors, only dAttn is
written in fp32: the three elementwise steps of the first version (re-forming
Attn in fp32, the subtraction and the product, all in fp32) moved 15 bytes per
[h,s,t] element, these two move 6.  All tensors are dense (the all-ones
partition vector): every kernel reads its operands in place through per-label
strides, so the layout costs nothing here.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Tuple

import torch

from ._binding import Plan, tra_execute, tra_execute_chain, tra_execute_contract_chain, tra_plan

# (output name, spec, operand names, join, aggregate, input dtype, output dtype, scaled by 1/sqrt(dh))
FORWARD: List[Tuple[str, str, Tuple[str, ...], str, str, str, str, bool]] = [
    ("Q_proj", "sa,ahd->shd", ("Q", "W_Q"), "mul", "sum", "bf16", "bf16", False),
    ("K_proj", "ta,ahd->thd", ("K", "W_K"), "mul", "sum", "bf16", "bf16", False),
    ("V_proj", "ta,ahd->thd", ("V", "W_V"), "mul", "sum", "bf16", "bf16", False),
    ("Scores", "shd,thd->hst", ("Q_proj", "K_proj"), "mul", "sum", "bf16", "f32", True),
    ("LSE", "hst->hs", ("Scores",), "ident", "lse", "f32", "f32", False),
    ("Attn", "hst,hs->hst", ("Scores", "LSE"), "exp_sub", "none", "f32", "bf16", False),
    ("O", "hst,thd->shd", ("Attn", "V_proj"), "mul", "sum", "bf16", "bf16", False),
    ("Output", "shd,ahd->sa", ("O", "W_O"), "mul", "sum", "bf16", "f32", False),
]

BACKWARD: List[Tuple[str, str, Tuple[str, ...], str, str, str, str, bool]] = [
    ("dO", "sa,ahd->shd", ("dOutput", "W_O"), "mul", "sum", "bf16", "bf16", False),
    ("dW_O", "sa,shd->ahd", ("dOutput", "O"), "mul", "sum", "bf16", "f32", False),
    ("Rows", "shd,shd->hs", ("dO", "O"), "mul", "sum", "bf16", "f32", False),
    ("dAttn", "shd,thd->hst", ("dO", "V_proj"), "mul", "sum", "bf16", "f32", False),
    ("dV_proj", "hst,shd->thd", ("Attn", "dO"), "mul", "sum", "bf16", "bf16", False),
    ("dAttn_c", "hst,hs->hst", ("dAttn", "Rows"), "sub", "none", "f32", "bf16", False),
    ("dScores", "hst,hst->hst", ("Attn", "dAttn_c"), "mul", "none", "bf16", "bf16", False),
    ("dQ_proj", "hst,thd->shd", ("dScores", "K_proj"), "mul", "sum", "bf16", "bf16", True),
    ("dK_proj", "hst,shd->thd", ("dScores", "Q_proj"), "mul", "sum", "bf16", "bf16", True),
    ("dW_Q", "sa,shd->ahd", ("Q", "dQ_proj"), "mul", "sum", "bf16", "f32", False),
    ("dQ", "shd,ahd->sa", ("dQ_proj", "W_Q"), "mul", "sum", "bf16", "f32", False),
    ("dW_K", "ta,thd->ahd", ("K", "dK_proj"), "mul", "sum", "bf16", "f32", False),
    ("dK", "thd,ahd->ta", ("dK_proj", "W_K"), "mul", "sum", "bf16", "f32", False),
    ("dW_V", "ta,thd->ahd", ("V", "dV_proj"), "mul", "sum", "bf16", "f32", False),
    ("dV", "thd,ahd->ta", ("dV_proj", "W_V"), "mul", "sum", "bf16", "f32", False),
]

_TORCH = {"bf16": torch.bfloat16, "f32": torch.float32}

# Consecutive elementwise steps run as one tra_execute_chain (the first step's
# output is only the second's second operand, and is never written): the
# subtraction dAttn - r and the Jacobian product read dAttn, Attn and r once
# and write dScores, 8 bytes per [h,s,t] element instead of 12.
CHAINED = {"dAttn_c": "dScores"}
# A product whose epilogue runs such a chain (tra_execute_contract_chain):
# dScores = Attn * (dO.V^T - Rows) in one launch, dAttn never written.  Used
# (the default) when the product's plan runs on the matrix-core kernel with no
# split; otherwise, or with fuse_product_chain=False, the product writes dAttn
# and the chain above follows.
CONTRACT_CHAINED = {"dAttn": ("dAttn_c", "dScores")}


def _launches(fused: bool) -> List[str]:
    """The names on_step reports, in launch order: a chained pair reports its
    second step's name at its first step's position; with the product chain
    fused, the product dAttn runs the pair in its epilogue and reports dScores
    at dAttn's position."""
    order: List[str] = []
    chained_into = {b: a for a, b in CHAINED.items()}
    in_contract = {m for v in CONTRACT_CHAINED.values() for m in v}
    for n, *_ in BACKWARD:
        if fused and n in CONTRACT_CHAINED:
            order.append(CONTRACT_CHAINED[n][-1])
        elif (fused and n in in_contract) or n in chained_into:
            continue
        elif n in CHAINED:
            order.append(CHAINED[n])
        else:
            order.append(n)
    return order


# The steps as they are launched (and reported to on_step), with the product
# chain fused (the full-size layer) and without it.
BACKWARD_LAUNCHES = _launches(True)
BACKWARD_LAUNCHES_UNFUSED = _launches(False)


class AttentionLayer:
    """Plans (host only, once) and runs the forward and backward EinSums of one layer.

    s query positions, t key positions, a model width, h heads of width dh.
    """

    def __init__(self, s: int, a: int, h: int, dh: int, t: Optional[int] = None, fuse_product_chain: bool = True):
        self.s, self.a, self.h, self.dh = s, a, h, dh
        self.t = s if t is None else t
        self.bounds = {"s": s, "t": self.t, "a": a, "h": h, "d": dh}
        self.scale = 1.0 / math.sqrt(dh)
        self.plans: Dict[str, Plan] = {}
        for step in FORWARD + BACKWARD:
            name, spec, _, join, agg, idt, odt, scaled = step
            labels = set(spec.replace(",", "").replace("->", ""))
            b = {c: self.bounds[c] for c in labels}
            self.plans[name] = tra_plan(spec, b, {c: 1 for c in labels}, join, agg, idt, odt,
                                        self.scale if scaled else 1.0)
        self.workspace_bytes = max(p.info.workspace_bytes for p in self.plans.values())
        pc = self.plans["dAttn"]
        # the default where the product runs unsplit on the matrix cores: its
        # result is bit-identical to the three launches it replaces, and it
        # never writes the fp32 dAttn
        self.fuse_product_chain = fuse_product_chain and pc.kernel == "mfma_bf16" and pc.info.agg_split == 1
        self.backward_launches = BACKWARD_LAUNCHES if self.fuse_product_chain else BACKWARD_LAUNCHES_UNFUSED

    def shape(self, name: str) -> Tuple[int, ...]:
        for out, spec, *_ in FORWARD + BACKWARD:
            if out == name:
                return tuple(self.bounds[c] for c in spec.split("->")[1])
        raise KeyError(name)

    def _run(self, steps, env: Dict[str, torch.Tensor], ws: Optional[torch.Tensor], stream, on_step) -> None:
        by_name = {st[0]: st for st in steps}
        done = set()
        for name, _, ins, *_rest in steps:
            if name in done or any(second == name and first in by_name for first, second in CHAINED.items()):
                continue   # ran with its first step
            if name in CONTRACT_CHAINED and self.fuse_product_chain:
                a_name, b_name = CONTRACT_CHAINED[name]
                _, _, ins_a, *_ = by_name[a_name]
                _, _, ins_b, *rest_b = by_name[b_name]
                assert ins_a[0] == name and ins_b[1] == a_name, "the chain reads the product, then its first step"
                pb = self.plans[b_name]
                z = env.get(b_name)
                if z is None or z.numel() != pb.info.z_elems or z.dtype != _TORCH[rest_b[3]]:
                    z = torch.empty(pb.info.z_elems, dtype=_TORCH[rest_b[3]], device=env[ins[0]].device)
                tra_execute_contract_chain(self.plans[name], self.plans[a_name], pb, env[ins[0]].reshape(-1),
                                           env[ins[1]].reshape(-1), env[ins_a[1]].reshape(-1),
                                           env[ins_b[0]].reshape(-1), z.reshape(-1), stream)
                env[b_name] = z.view(self.shape(b_name))
                done.update((a_name, b_name))
                if on_step is not None:
                    on_step(b_name)
                continue
            out_name = CHAINED.get(name, name)
            p = self.plans[name]
            x = env[ins[0]].reshape(-1)
            y = env[ins[1]].reshape(-1) if len(ins) == 2 else None
            _, _, ins_b, *rest_b = by_name[out_name]
            z = env.get(out_name)
            pz = self.plans[out_name]
            if z is None or z.numel() != pz.info.z_elems or z.dtype != _TORCH[rest_b[3]]:
                z = torch.empty(pz.info.z_elems, dtype=_TORCH[rest_b[3]], device=x.device)
            if out_name != name:
                assert ins_b[1] == name, "a chained step reads its first step's output as its second operand"
                tra_execute_chain(p, pz, x, y, env[ins_b[0]].reshape(-1), z.reshape(-1), stream)
            else:
                tra_execute(p, x, y, z.reshape(-1), ws, stream)
            env[out_name] = z.view(self.shape(out_name))
            if on_step is not None:
                on_step(out_name)

    def workspace(self, device) -> Optional[torch.Tensor]:
        n = self.workspace_bytes
        return torch.empty(n, dtype=torch.uint8, device=device) if n else None

    def forward(self, inputs: Dict[str, torch.Tensor], ws: Optional[torch.Tensor] = None,
                stream=None, on_step=None) -> Dict[str, torch.Tensor]:
        """inputs: Q [s,a], K and V [t,a], W_Q/W_K/W_V/W_O [a,h,dh], all bf16 on the device.
        Returns every forward tensor (the backward reads Q_proj, K_proj, V_proj, Scores,
        LSE, Attn and O); Output is [s,a] fp32.  Tensors already present under a step's
        name (right size and dtype) are overwritten in place; on_step(name) is called
        after each step is enqueued."""
        env = dict(inputs)
        self._run(FORWARD, env, ws, stream, on_step)
        return env

    def backward(self, saved: Dict[str, torch.Tensor], d_output: torch.Tensor, ws: Optional[torch.Tensor] = None,
                 stream=None, on_step=None, out: Optional[Dict[str, torch.Tensor]] = None) -> Dict[str, torch.Tensor]:
        """saved: what forward() returned; d_output: dL/dOutput [s,a] bf16.
        Returns dQ [s,a], dK and dV [t,a], dW_Q/dW_K/dW_V/dW_O [a,h,dh] (fp32) and the
        intermediate gradients; buffers passed in `out` (a previous result) are reused."""
        env = dict(saved)
        if out:
            env.update(out)
        env["dOutput"] = d_output
        self._run(BACKWARD, env, ws, stream, on_step)
        return {k: env[k] for k, *_ in BACKWARD if k in env}
