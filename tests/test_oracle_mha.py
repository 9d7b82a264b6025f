"""Pins of the fp64 attention-graph oracle (CPU only).

The library-product evaluation in oracle.mha is checked against the node-by-
node nested-loop evaluation of the same EinSums, and against closed forms:
softmax rows sum to one, and with K_proj == 0 every attention weight is 1/t
so O is the mean of V_proj over t.
"""
import math

import numpy as np
import torch

from oracle import mha, ref
from tensor_relational_algebra_amd import workloads


def _inputs(s, a, h, dh, seed=0):
    case = workloads.MhaCase(s=s, a=a, h=h, dh=dh, wid=90 + seed)
    return case.make_inputs()


def test_graph_equals_node_by_node_loops():
    t = _inputs(12, 16, 2, 4)
    r = mha.mha(t)
    qp = ref.einsum("sa,ahd->shd", t["Q"], t["W_Q"])
    kp = ref.einsum("sa,ahd->shd", t["K"], t["W_K"])
    vp = ref.einsum("sa,ahd->shd", t["V"], t["W_V"])
    sc = ref.einsum("shd,thd->hst", qp, kp, post_scale=1 / math.sqrt(4))
    lse = ref.einsum("hst->hs", sc, None, "ident", "lse")
    at = ref.einsum("hst,hs->hst", sc, lse, "exp_sub", "none")
    o = ref.einsum("hst,thd->shd", at, vp)
    out = ref.einsum("shd,ahd->sa", o, t["W_O"])
    for name, want in [("Q_proj", qp), ("K_proj", kp), ("V_proj", vp), ("Scores", sc),
                       ("LSE", lse), ("Attn", at), ("O", o), ("Output", out)]:
        np.testing.assert_allclose(r[name], want, rtol=1e-12, atol=1e-12, err_msg=name)


def test_softmax_rows_sum_to_one():
    r = mha.mha(_inputs(16, 32, 4, 8, seed=1))
    np.testing.assert_allclose(r["Attn"].sum(axis=2), 1.0, rtol=0, atol=1e-12)


def test_zero_keys_give_uniform_attention():
    t = _inputs(8, 16, 2, 4, seed=2)
    t["W_K"] = torch.zeros_like(t["W_K"])
    r = mha.mha(t)
    # exp(0 - log 8) is 1/8 up to the rounding of exp and log
    np.testing.assert_allclose(r["Attn"], np.full(r["Attn"].shape, 1.0 / 8), rtol=1e-15, atol=0)
    want_o = np.broadcast_to(r["V_proj"].mean(axis=0, keepdims=True), r["O"].shape)
    np.testing.assert_allclose(r["O"], want_o, rtol=0, atol=1e-13)


def test_row_sample_equals_full():
    t = _inputs(16, 16, 2, 8, seed=3)
    full = mha.mha(t)
    rows = np.array([0, 5, 15])
    part = mha.mha(t, rows=rows)
    np.testing.assert_allclose(part["Output"], full["Output"][rows], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(part["Attn"], full["Attn"][:, rows], rtol=1e-13, atol=1e-13)


def _autograd_reference(t, d_out):
    """The same layer in float64 torch with autograd: an independent backward."""
    leaves = {n: torch.tensor(mha.ref._as_np(t[n]), dtype=torch.float64, requires_grad=True)
              for n in ("Q", "K", "V", "W_Q", "W_K", "W_V", "W_O")}
    dh = leaves["W_Q"].shape[2]
    qp = torch.einsum("sa,ahd->shd", leaves["Q"], leaves["W_Q"])
    kp = torch.einsum("sa,ahd->shd", leaves["K"], leaves["W_K"])
    vp = torch.einsum("sa,ahd->shd", leaves["V"], leaves["W_V"])
    sc = torch.einsum("shd,thd->hst", qp, kp) / math.sqrt(dh)
    attn = torch.softmax(sc, dim=2)
    o = torch.einsum("hst,thd->shd", attn, vp)
    out = torch.einsum("shd,ahd->sa", o, leaves["W_O"])
    # gradients of the intermediates too
    for x in (qp, o, attn):
        x.retain_grad()
    g = torch.tensor(mha.ref._as_np(d_out), dtype=torch.float64)
    out.backward(g)
    res = {"d" + n: leaves[n].grad.numpy() for n in leaves}
    res.update({"dQ_proj": qp.grad.numpy(), "dO": o.grad.numpy(), "dAttn": attn.grad.numpy()})
    # softmax Jacobian applied to dAttn, written out with torch's own softmax backward
    res["dScores"] = torch.ops.aten._softmax_backward_data(attn.grad, attn, 2, torch.float64).detach().numpy()
    return res


def test_backward_equals_autograd():
    t = _inputs(24, 16, 2, 8, seed=4)
    g = workloads.draw(4242, (24, 16), "normal", "bf16", std=1.0)
    got = mha.mha_backward(t, g)
    want = _autograd_reference(t, g)
    for name in ("dQ", "dK", "dV", "dW_Q", "dW_K", "dW_V", "dW_O"):
        np.testing.assert_allclose(got[name], want[name], rtol=1e-9, atol=1e-12, err_msg=name)


def test_backward_intermediates_equal_autograd():
    t = _inputs(24, 16, 2, 8, seed=6)
    g = workloads.draw(4244, (24, 16), "normal", "bf16", std=1.0)
    got = mha.mha_backward(t, g)
    want = _autograd_reference(t, g)
    for name in ("dQ_proj", "dO", "dAttn", "dScores"):
        np.testing.assert_allclose(got[name], want[name], rtol=1e-9, atol=1e-12, err_msg=name)


def test_backward_row_sample_equals_full():
    """The row-restricted backward (query rows only) equals those rows of the
    full backward, and of autograd's."""
    case = workloads.MhaCase(s=32, a=16, h=2, dh=8, wid=96)
    t = case.make_inputs()
    g = workloads.draw(9601, (32, 16), "normal", "bf16", std=1.0)
    full = mha.mha_backward(t, g)
    auto = _autograd_reference(t, g)
    rows = np.array([0, 7, 8, 31])
    part = mha.mha_backward(t, g, rows=rows)
    assert set(part) == {"dO", "dAttn", "dScores", "dQ_proj", "dQ"}
    for name in ("dO", "dQ_proj", "dQ"):
        np.testing.assert_allclose(part[name], full[name][rows], rtol=1e-12, atol=1e-13, err_msg=name)
        np.testing.assert_allclose(part[name], auto[name][rows], rtol=1e-9, atol=1e-12, err_msg=name)
    for name in ("dAttn", "dScores"):
        np.testing.assert_allclose(part[name], full[name][:, rows], rtol=1e-12, atol=1e-13, err_msg=name)
        np.testing.assert_allclose(part[name], auto[name][:, rows], rtol=1e-9, atol=1e-12, err_msg=name)


def test_backward_with_unequal_query_and_key_lengths():
    # s != t is allowed by the EinSums; the projections of K and V run over t
    case = workloads.MhaCase(s=8, a=16, h=2, dh=4, wid=95)
    t = case.make_inputs()
    t["K"] = workloads.draw(9501, (13, 16), "normal", "bf16", std=1.0)
    t["V"] = workloads.draw(9502, (13, 16), "normal", "bf16", std=1.0)
    g = workloads.draw(9503, (8, 16), "normal", "bf16", std=1.0)
    got = mha.mha_backward(t, g)
    want = _autograd_reference(t, g)
    for name in ("dQ", "dK", "dV", "dW_Q", "dW_K", "dW_V", "dW_O"):
        np.testing.assert_allclose(got[name], want[name], rtol=1e-9, atol=1e-12, err_msg=name)


def test_softmax_backward_row_sum_identity():
    # sum_t Attn * dAttn equals sum_d dO * O (both are dOut . Output restricted to one
    # row and head), which lets the row term be formed from [s,h,d] tensors instead of
    # [h,s,t] ones.
    t = _inputs(20, 16, 2, 8, seed=5)
    g = workloads.draw(4343, (20, 16), "normal", "bf16", std=1.0)
    fwd = mha.mha(t)
    b = mha.mha_backward(t, g)
    lhs = (fwd["Attn"] * b["dAttn"]).sum(axis=2)                       # [h, s]
    rhs = np.transpose((b["dO"] * fwd["O"]).sum(axis=2), (1, 0))        # [h, s]
    np.testing.assert_allclose(lhs, rhs, rtol=1e-10, atol=1e-12)
