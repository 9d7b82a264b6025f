"""GPU parity of the attention layer's forward and backward EinSums
(tensor_relational_algebra_amd.attention: every step one tra_plan /
tra_execute) against the fp64 oracle's chain rule of the same layer.

Operands of the matrix-core products are stored in bf16 on the GPU (the
forward graph's storage dtypes), so the gate is the bf16-input tolerance:
max-norm relative error 2e-2 per gradient tensor.
"""
import numpy as np
import pytest
import torch

import tensor_relational_algebra_amd as tra
from oracle import mha
from tensor_relational_algebra_amd import workloads as wl
from tests.gpu_util import DEV, gate, maxnorm_rel_err

pytestmark = pytest.mark.gpu

GRADS = ("dQ", "dK", "dV", "dW_Q", "dW_K", "dW_V", "dW_O")


def _run(case, t_len=None, fuse=True):
    host = case.make_inputs()
    if t_len is not None and t_len != case.s:
        host["K"] = wl.draw(1000 * case.wid + 8, (t_len, case.a), "normal", "bf16", std=1.0)
        host["V"] = wl.draw(1000 * case.wid + 9, (t_len, case.a), "normal", "bf16", std=1.0)
    g = case.make_output_gradient()
    layer = tra.AttentionLayer(case.s, case.a, case.h, case.dh, t=t_len, fuse_product_chain=fuse)
    dev = {k: v.to(DEV) for k, v in host.items()}
    ws = layer.workspace(DEV)
    saved = layer.forward(dev, ws)
    grads = layer.backward(saved, g.to(DEV), ws)
    torch.cuda.synchronize()
    got = {k: grads[k].double().cpu().numpy() for k in GRADS}
    got["Output"] = saved["Output"].double().cpu().numpy()
    return got, host, g, layer


def _check(got, host, g):
    want = mha.mha_backward(host, g)
    want["Output"] = mha.mha(host)["Output"]
    errs = {k: maxnorm_rel_err(got[k], want[k]) for k in GRADS + ("Output",)}
    bad = {k: e for k, e in errs.items() if not e <= 2e-2}
    assert not bad, errs


@pytest.mark.parametrize("case", [wl.MhaCase(s=256, a=256, h=4, dh=64, wid=41),
                                  wl.MhaCase(s=128, a=128, h=4, dh=32, wid=42)],
                         ids=["256x256x4x64", "128x128x4x32"])
def test_small_layer_backward(case):
    got, host, g, _ = _run(case)
    _check(got, host, g)


def test_unequal_query_and_key_lengths():
    got, host, g, _ = _run(wl.MhaCase(s=128, a=256, h=2, dh=64, wid=43), t_len=384)
    _check(got, host, g)


def _contractions():
    return [n for n, spec, *_ in tra.attention.BACKWARD if "->" in spec and n not in ("Rows", "dAttn_c", "dScores")]


def test_mid_size_layer_three_launch_path_on_the_matrix_cores():
    # the backward with the product chain off: the dAttn product writes fp32,
    # then the chained subtraction and Jacobian; head width 128 and tile
    # multiples of the full layer, so every contraction plans onto the
    # matrix-core kernel
    case = wl.MhaCase(s=1024, a=512, h=8, dh=128, wid=46)
    got, host, g, layer = _run(case, fuse=False)
    assert all(layer.plans[n].kernel == "mfma_bf16" for n in _contractions()), \
        {n: layer.plans[n].kernel for n in _contractions()}
    assert not layer.fuse_product_chain and "dAttn" in layer.backward_launches
    _check(got, host, g)


@pytest.mark.parametrize("fuse", [True, False], ids=["product_chain", "three_launches"])
def test_full_layer_backward_sampled_query_rows(fuse):
    """The full layer (s = t = a = 4096, 32 heads of 128), the default backward
    (the softmax Jacobian in the dAttn product's epilogue) and the one with
    the fp32 dAttn written: the gradients that belong to query rows (dO,
    dAttn when written, dScores, dQ_proj, dQ) on 64 rows spread over every
    256-row band, against the oracle's row-restricted chain rule; every
    gradient finite."""
    case = wl.MHA
    host = case.make_inputs()
    g = case.make_output_gradient()
    layer = tra.AttentionLayer(case.s, case.a, case.h, case.dh, fuse_product_chain=fuse)
    assert layer.fuse_product_chain == fuse
    assert all(layer.plans[n].kernel == "mfma_bf16" for n in _contractions())
    dev = {k: v.to(DEV) for k, v in host.items()}
    ws = layer.workspace(DEV)
    saved = layer.forward(dev, ws)
    grads = layer.backward(saved, g.to(DEV), ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(505)
    rows = np.sort(np.concatenate([b * 256 + rng.choice(256, 4, replace=False) for b in range(16)]))
    want = mha.mha_backward(host, g, rows=rows)
    r = torch.from_numpy(rows).to(DEV)
    for name, ax in (("dO", 0), ("dAttn", 1), ("dScores", 1), ("dQ_proj", 0), ("dQ", 0)):
        if name not in grads:
            assert fuse and name == "dAttn"
            continue
        got = grads[name].index_select(ax, r).double().cpu().numpy()
        assert np.isfinite(got).all(), name
        gate(f"attention backward {name} (64 rows)", layer.plans[name].kernel, got, want[name], 2e-2)
    for k in GRADS:
        assert torch.isfinite(grads[k]).all(), k


def test_mid_size_layer_on_the_matrix_cores():
    # the default backward; head width and tile multiples of the full layer:
    # every contraction of the backward plans onto the matrix-core kernel
    case = wl.MhaCase(s=1024, a=512, h=8, dh=128, wid=44)
    got, host, g, layer = _run(case, fuse=True)
    assert all(layer.plans[n].kernel == "mfma_bf16" for n in _contractions()), \
        {n: layer.plans[n].kernel for n in _contractions()}
    # the softmax Jacobian runs in the dAttn product's epilogue
    assert layer.fuse_product_chain and "dAttn" not in layer.backward_launches
    _check(got, host, g)


def test_backward_is_bitwise_reproducible():
    case = wl.MhaCase(s=256, a=256, h=4, dh=64, wid=45)
    a, *_ = _run(case)
    b, *_ = _run(case)
    for k in GRADS:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
