"""Multi-head attention as EinSums, forward and backward, in float64 (TEST INFRASTRUCTURE).

Page "EinDecomp：基于爱因斯坦求和与张量关系代数的自动张量并行分解算法",
section 2.1, the multi-head attention example:

    Q_proj[s,h,d] = sum_a Q[s,a] W_Q[a,h,d]          (same for K and V)
    Scores[h,s,t] = (1/sqrt(d_k)) sum_d Q_proj[s,h,d] K_proj[t,h,d]
    Attn[h,s,t]   = softmax over t of Scores[h,s,t]
    O[s,h,d]      = sum_t Attn[h,s,t] V_proj[t,h,d]
    Output[s,a]   = sum_h sum_d O[s,h,d] W_O[a,h,d]

(t is the page's primed s; d_k is the per-head width.)  Softmax is written as
two EinSums: LSE[h,s] = logsumexp_t Scores[h,s,t] and
Attn[h,s,t] = exp(Scores[h,s,t] - LSE[h,s]).

Every contraction here is a library product (numpy tensordot / matmul in
float64) used as one step of the definition; every intermediate stays in
float64.  ``rows`` restricts the computation to a subset of query positions s
(all of K_proj and V_proj are still formed), so large layers can be checked
on a sample of rows.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from . import ref


def mha(t: Dict[str, object], rows: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    q, k, v = (ref._as_np(t[n]) for n in ("Q", "K", "V"))
    wq, wk, wv, wo = (ref._as_np(t[n]) for n in ("W_Q", "W_K", "W_V", "W_O"))
    a, h, dh = wq.shape
    if rows is not None:
        q = q[np.asarray(rows)]
    # projections: contract a
    qp = np.tensordot(q, wq, axes=([1], [0]))       # [s, h, d]
    kp = np.tensordot(k, wk, axes=([1], [0]))       # [t, h, d]
    vp = np.tensordot(v, wv, axes=([1], [0]))       # [t, h, d]
    # scores: contract d per head
    qh = np.transpose(qp, (1, 0, 2))                 # [h, s, d]
    kh = np.transpose(kp, (1, 2, 0))                 # [h, d, t]
    scores = np.matmul(qh, kh) / np.sqrt(dh)         # [h, s, t]
    m = scores.max(axis=2, keepdims=True)
    lse = m + np.log(np.exp(scores - m).sum(axis=2, keepdims=True))
    attn = np.exp(scores - lse)                      # [h, s, t]
    vh = np.transpose(vp, (1, 0, 2))                 # [h, t, d]
    o = np.transpose(np.matmul(attn, vh), (1, 0, 2))  # [s, h, d]
    out = np.tensordot(o, wo, axes=([1, 2], [1, 2]))  # [s, a]
    return {"Q_proj": qp, "K_proj": kp, "V_proj": vp, "Scores": scores,
            "LSE": lse[..., 0], "Attn": attn, "O": o, "Output": out}


def mha_backward(t: Dict[str, object], d_out, rows: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Gradients of sum(Output * d_out) with respect to the layer's inputs and weights.

    With ``rows``, only the gradients that belong to those query positions s
    are formed, each from those rows alone: dO, dAttn, dScores, dQ_proj and dQ
    (row s of each depends on row s of the forward and on all of K_proj and
    V_proj); the key-side and weight gradients, which sum over every row, are
    omitted.

    The pages give the forward EinSums only; the backward is their chain rule,
    one EinSum per step, all in float64:

        dW_O[a,h,d]  = sum_s dOut[s,a] O[s,h,d]
        dO[s,h,d]    = sum_a dOut[s,a] W_O[a,h,d]
        dAttn[h,s,t] = sum_d dO[s,h,d] V_proj[t,h,d]
        dV_proj      = sum_s Attn[h,s,t] dO[s,h,d]                 -> [t,h,d]
        dScores      = Attn * (dAttn - sum_t' Attn[h,s,t'] dAttn[h,s,t'])
                       (the Jacobian of softmax over t, applied row by row)
        dQ_proj      = (1/sqrt(d_k)) sum_t dScores[h,s,t] K_proj[t,h,d]
        dK_proj      = (1/sqrt(d_k)) sum_s dScores[h,s,t] Q_proj[s,h,d]
        dW_X[a,h,d]  = sum_s X[s,a] dX_proj[s,h,d],   dX[s,a] = sum_hd dX_proj[s,h,d] W_X[a,h,d]
    """
    fwd = mha(t, rows=rows)
    q, k, v = (ref._as_np(t[n]) for n in ("Q", "K", "V"))
    wq, wk, wv, wo = (ref._as_np(t[n]) for n in ("W_Q", "W_K", "W_V", "W_O"))
    g = ref._as_np(d_out)                                        # [s, a]
    a, h, dh = wq.shape
    if rows is not None:
        q, g = q[np.asarray(rows)], g[np.asarray(rows)]
    attn, o = fwd["Attn"], fwd["O"]                               # [h,s,t], [s,h,d]
    qp, kp, vp = fwd["Q_proj"], fwd["K_proj"], fwd["V_proj"]
    d_o = np.tensordot(g, wo, axes=([1], [0]))                    # [s, h, d]
    d_attn = np.matmul(np.transpose(d_o, (1, 0, 2)), np.transpose(vp, (1, 2, 0)))   # [h, s, t]
    row = (attn * d_attn).sum(axis=2, keepdims=True)              # [h, s, 1]
    d_scores = attn * (d_attn - row)
    scale = 1.0 / np.sqrt(dh)
    d_qp = np.transpose(np.matmul(d_scores, np.transpose(kp, (1, 0, 2))), (1, 0, 2)) * scale
    if rows is not None:
        return {"dO": d_o, "dAttn": d_attn, "dScores": d_scores, "dQ_proj": d_qp,
                "dQ": np.tensordot(d_qp, wq, axes=([1, 2], [1, 2]))}
    d_wo = np.tensordot(g, o, axes=([0], [0]))                    # [a, h, d]
    d_vp = np.transpose(np.matmul(np.transpose(attn, (0, 2, 1)), np.transpose(d_o, (1, 0, 2))), (1, 0, 2))
    d_kp = np.transpose(np.matmul(np.transpose(d_scores, (0, 2, 1)), np.transpose(qp, (1, 0, 2))),
                        (1, 0, 2)) * scale
    out = {"dW_O": d_wo, "dO": d_o, "dAttn": d_attn, "dV_proj": d_vp, "dScores": d_scores,
           "dQ_proj": d_qp, "dK_proj": d_kp}
    for name, x, w, dxp in (("Q", q, wq, d_qp), ("K", k, wk, d_kp), ("V", v, wv, d_vp)):
        out["dW_" + name] = np.tensordot(x, dxp, axes=([0], [0]))          # [a, h, d]
        out["d" + name] = np.tensordot(dxp, w, axes=([1, 2], [1, 2]))      # [s, a]
    return out
