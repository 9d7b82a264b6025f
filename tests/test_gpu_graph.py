"""GPU parity of the attention EinGraph (projections, scores, softmax as
logsumexp + normalise, weighted sum, output projection) run by the C-ABI
graph executor, against the fp64 oracle of the same layer.

Intermediates the matrix cores consume are stored in bf16, so the gate is the
bf16-input tolerance (max-norm relative error 2e-2) on the layer output.
"""
import numpy as np
import pytest
import torch

import tensor_relational_algebra_amd as tra
from oracle import mha
from tensor_relational_algebra_amd import workloads as wl
from tests.gpu_util import DEV, gate, maxnorm_rel_err

pytestmark = pytest.mark.gpu


def _run(case, p=None, d_all=None, fuse=False, time_model=False, overlap=False):
    desc = case.graph_desc()
    flags = (tra.GRAPH_FUSE_ATTENTION if fuse else 0) | (tra.GRAPH_CHOOSE_TIME if time_model else 0) | \
        (tra.GRAPH_OVERLAP_COPIES if overlap else 0)
    g = tra.tra_graph_plan_ex(desc, p or 1, d_all, flags)
    host = case.make_inputs()
    dev = {k: v.to(DEV) for k, v in host.items()}
    out = tra.tra_graph_execute(g, dev).reshape(case.s, case.a)
    torch.cuda.synchronize()
    return out.cpu().double().numpy(), host, g


def _d_all(case, pick):
    ds = []
    for line in case.graph_desc().splitlines():
        f = line.split()
        labels = f[2].split("->")[1] if f[1] == "softmax" else tra.tra_canonical_labels(f[2])
        bounds = dict(kv.split("=") for kv in f[3].split(","))
        ds += [pick(c, int(bounds[c])) for c in labels]
    return ds


def test_small_layer_chooser_d():
    out, host, g = _run(wl.MHA_SMALL, p=16)
    want = mha.mha(host)["Output"]
    assert maxnorm_rel_err(out, want) <= 2e-2


def test_small_layer_all_ones_and_forced_repartitions():
    case = wl.MHA_SMALL
    want = mha.mha(case.make_inputs())["Output"]
    out, _, g = _run(case, d_all=_d_all(case, lambda c, b: 1))
    assert g.info.n_repartitions == 0
    assert maxnorm_rel_err(out, want) <= 2e-2
    # alternate the part counts label by label so consecutive nodes disagree
    flip = {"s": 4, "t": 2, "h": 1, "d": 2, "a": 4}
    out, _, g = _run(case, d_all=_d_all(case, lambda c, b: flip[c]))
    assert g.info.n_repartitions > 0
    assert maxnorm_rel_err(out, want) <= 2e-2


def test_full_layer_sampled_rows():
    case = wl.MHA
    out, host, g = _run(case, p=256)
    rows = np.array([0, 1, 777, 2048, 4095])
    want = mha.mha(host, rows=rows)["Output"]
    err = maxnorm_rel_err(out[rows], want)
    assert err <= 2e-2, err
    assert np.isfinite(out).all()


def _nodes(case):
    """(name, output labels, canonical labels, bounds) per node of the graph."""
    out = []
    for line in case.graph_desc().splitlines():
        f = line.split()
        spec = f[2]
        bounds = {k: int(v) for k, v in (kv.split("=") for kv in f[3].split(","))}
        canon = spec.split("->")[1] if f[1] == "softmax" else tra.tra_canonical_labels(spec)
        out.append((f[0], spec.split("->")[1], canon, bounds))
    return out


def _rows_spread(n, bands, per_band, seed):
    rng = np.random.default_rng(seed)
    b = n // bands
    return np.sort(np.concatenate([k * b + rng.choice(b, per_band, replace=False) for k in range(bands)]))


@pytest.mark.parametrize("fuse", [False, True], ids=["unfused", "fused"])
def test_full_layer_every_node_on_sampled_rows(fuse):
    """The full layer, chooser-picked d, run node by node: after each node its
    output relation is read from the workspace, made dense, and compared with
    the fp64 oracle's tensor on 64 query rows (4 in each 256-row band, every
    head): Q_proj, Scores, the logsumexp, Attn, O and Output on those rows,
    K_proj and V_proj whole.  Fused, the scores and softmax nodes write
    nothing of their own; the fused node's O and the rest are compared."""
    case = wl.MHA
    flags = tra.GRAPH_FUSE_ATTENTION if fuse else 0
    g = tra.tra_graph_plan_ex(case.graph_desc(), 256, None, flags)
    assert g.info.n_fused == (1 if fuse else 0)
    host = case.make_inputs()
    dev = {k: v.to(DEV) for k, v in host.items()}
    ws = g.workspace(DEV)
    out = torch.empty(g.info.out_elems, dtype=torch.float32, device=DEV)
    rows = _rows_spread(case.s, 16, 4, seed=404)
    want = mha.mha(host, rows=rows)
    # which axis of each node's output is the query position
    query_axis = {"Q_proj": 0, "Scores": 1, "Attn": 1, "O": 0, "Output": 0}
    compared = []
    for i, (name, olab, canon, bounds) in enumerate(_nodes(case)):
        root = i == g.info.n_nodes - 1
        tra.tra_graph_run_node(g, i, dev, out if root else None, ws)
        torch.cuda.synchronize()
        if fuse and name in ("Scores", "Attn"):
            with pytest.raises(tra.TraError):
                g.node_output(i, ws)
            continue
        rel, lse = g.node_output(i, ws)
        d = dict(zip(canon, g.node_d(i)))
        dense = tra.from_relation(rel, [bounds[c] for c in olab], [d[c] for c in olab])
        pairs = [(name, dense)]
        if lse is not None:
            pairs.append(("LSE", tra.from_relation(lse, [bounds[c] for c in olab[:-1]], [d[c] for c in olab[:-1]])))
        for nm, t in pairs:
            ax = query_axis.get(nm, None if nm != "LSE" else 1)
            if ax is not None:
                t = t.index_select(ax, torch.from_numpy(rows).to(DEV))
            got = t.double().cpu().numpy()
            assert np.isfinite(got).all(), nm
            gate(f"attention layer {'fused' if fuse else 'unfused'} {nm} (64 rows)", "graph", got, want[nm], 2e-2)
            compared.append(nm)
        if root:
            # the dense output written by the root node equals its relation
            assert torch.equal(out.reshape(case.s, case.a), dense)
    expect = {"Q_proj", "K_proj", "V_proj", "O", "Output"} | (set() if fuse else {"Scores", "Attn", "LSE"})
    assert set(compared) == expect


# --- the attention chain fused into one kernel (online logsumexp over t) ---

def test_small_layer_fused_chooser_d():
    out, host, g = _run(wl.MHA_SMALL, p=16, fuse=True)
    assert g.info.n_fused == 1
    want = mha.mha(host)["Output"]
    assert maxnorm_rel_err(out, want) <= 2e-2


def test_small_layer_fused_reads_every_blocking_in_place():
    case = wl.MHA_SMALL
    want = mha.mha(case.make_inputs())["Output"]
    for pick in (lambda c, b: 1, lambda c, b: {"s": 4, "t": 2, "h": 1, "d": 2, "a": 4}[c],
                 lambda c, b: {"s": 2, "t": 1, "h": 4, "d": 4, "a": 2}[c]):
        out, _, g = _run(case, d_all=_d_all(case, pick), fuse=True)
        assert g.info.n_fused == 1
        err = maxnorm_rel_err(out, want)
        assert err <= 2e-2, err


@pytest.mark.parametrize("s,a,h,dh", [(256, 256, 8, 64), (128, 512, 4, 128), (512, 256, 2, 128)])
def test_fused_head_dims(s, a, h, dh):
    case = wl.MhaCase(s=s, a=a, h=h, dh=dh, wid=40 + dh)
    out, host, g = _run(case, p=16, fuse=True)
    assert g.info.n_fused == 1
    want = mha.mha(host)["Output"]
    err = maxnorm_rel_err(out, want)
    assert err <= 2e-2, err


def test_full_layer_fused_sampled_rows_and_deterministic():
    case = wl.MHA
    out, host, g = _run(case, p=256, fuse=True)
    assert g.info.n_fused == 1
    rows = np.array([0, 1, 777, 2048, 4095])
    want = mha.mha(host, rows=rows)["Output"]
    err = maxnorm_rel_err(out[rows], want)
    assert err <= 2e-2, err
    out2, _, _ = _run(case, p=256, fuse=True)
    assert np.array_equal(out, out2)


# --- partition vectors chosen by the measured time model ---

@pytest.mark.parametrize("fuse", [False, True], ids=["unfused", "fused"])
def test_small_layer_time_model(fuse):
    out, host, g = _run(wl.MHA_SMALL, p=16, fuse=fuse, time_model=True)
    assert g.info.n_repartitions == 0
    assert g.info.n_fused == (1 if fuse else 0)
    want = mha.mha(host)["Output"]
    assert maxnorm_rel_err(out, want) <= 2e-2


def test_full_layer_time_model_sampled_rows():
    case = wl.MHA
    out, host, g = _run(case, p=256, time_model=True)
    assert g.info.n_repartitions == 0
    rows = np.array([0, 3, 1500, 4095])
    want = mha.mha(host, rows=rows)["Output"]
    err = maxnorm_rel_err(out[rows], want)
    assert err <= 2e-2, err


# --- workspace reuse and the memory cap ---

def test_memory_capped_chain_of_products():
    # three fp32 products; the cap forces a costlier, smaller plan, and the
    # executor reuses dead buffers; parity with the fp64 chain either way
    from oracle import ref
    desc = "\n".join([
        "A einsum ij,jk->ik i=256,j=256,k=256 @X,@Y in=f32 out=f32",
        "B einsum ik,kl->il i=256,k=256,l=256 A,@W in=f32 out=f32",
        "C einsum il,lm->im i=256,l=256,m=256 B,@V in=f32 out=f32",
    ])
    host = {n: wl.draw(7700 + i, (256, 256), "uniform", "f32") for i, n in enumerate(("X", "Y", "W", "V"))}
    want = ref.einsum("il,lm->im", ref.einsum("ik,kl->il", ref.einsum("ij,jk->ik", host["X"], host["Y"]), host["W"]),
                      host["V"])
    g0 = tra.tra_graph_plan(desc, 16)
    for g in (g0, tra.tra_graph_plan_cap(desc, 16, 0, g0.info.workspace_bytes - 1)):
        dev = {k: v.to(DEV) for k, v in host.items()}
        out = tra.tra_graph_execute(g, dev).reshape(256, 256)
        torch.cuda.synchronize()
        assert maxnorm_rel_err(out.cpu().double().numpy(), want) <= 1e-4


# --- repartition copies on a second stream, overlapped with the nodes ---

@pytest.mark.parametrize("fuse", [False, True], ids=["unfused", "fused"])
def test_overlapped_copies_match_the_in_order_run(fuse):
    """With TRA_GRAPH_OVERLAP_COPIES every copy runs on a side stream while the
    nodes run on the caller's: blockings that disagree between consecutive
    nodes force repartitions, and three calls in a row give the in-order run's
    output bit for bit (and the oracle's to the bf16 tolerance)."""
    case = wl.MHA_SMALL
    flip = {"s": 4, "t": 2, "h": 1, "d": 2, "a": 4}
    d_all = _d_all(case, lambda c, b: flip[c])
    host = case.make_inputs()
    dev = {k: v.to(DEV) for k, v in host.items()}
    flags = tra.GRAPH_FUSE_ATTENTION if fuse else 0
    g0 = tra.tra_graph_plan_ex(case.graph_desc(), 1, d_all, flags)
    g1 = tra.tra_graph_plan_ex(case.graph_desc(), 1, d_all, flags | tra.GRAPH_OVERLAP_COPIES)
    # fused, the chain reads its operands in place and only the graph inputs are copied
    assert g1.info.n_repartitions == g0.info.n_repartitions
    assert fuse or g0.info.n_repartitions > 0
    assert g1.info.workspace_bytes >= g0.info.workspace_bytes
    want = tra.tra_graph_execute(g0, dev)
    torch.cuda.synchronize()
    for _ in range(3):
        got = tra.tra_graph_execute(g1, dev)
        torch.cuda.synchronize()
        assert torch.equal(got, want)
    ref_out = mha.mha(host)["Output"]
    assert maxnorm_rel_err(want.reshape(case.s, case.a).cpu().double().numpy(), ref_out) <= 2e-2


def test_overlapped_copies_full_layer_sampled_rows():
    """The full layer under the pages' chooser (four repartitions between nodes
    and a copy of every graph input) with the copies overlapped."""
    case = wl.MHA
    out, host, g = _run(case, p=256, overlap=True)
    assert g.info.n_repartitions > 0
    rows = np.array([0, 3, 1500, 4095])
    want = mha.mha(host, rows=rows)["Output"]
    assert maxnorm_rel_err(out[rows], want) <= 2e-2


# --- the softmax node: one pass over each row when it fits in registers ---

@pytest.mark.parametrize("t,d_t,out_dtype", [(4096, 1, "bf16"), (4096, 2, "bf16"), (2048, 8, "f32"), (256, 1, "f32"),
                                             (8192, 1, "bf16"), (128, 1, "f32")],
                         ids=["4096", "4096-2blocks", "2048-8blocks-f32", "256-f32", "8192-twopass",
                              "128-twopass"])
def test_softmax_node(t, d_t, out_dtype):
    """Rows of up to 4096 elements run as one kernel (logsumexp and normalise
    with the row in registers); longer or shorter rows as the two EinSums.
    Both against the oracle's logsumexp: exp(S - lse) to the output dtype's
    tolerance, and every row summing to 1."""
    from oracle import ref
    h, s = 4, 64
    desc = f"A softmax hst->hst h={h},s={s},t={t} @S in=f32 out={out_dtype}"
    host = {"S": wl.draw(7900 + t, (h, s, t), "normal", "f32", std=3.0)}
    g = tra.tra_graph_plan(desc, 1, [2, 4, d_t])
    out = tra.tra_graph_execute(g, {"S": host["S"].to(DEV)}).reshape(h, s, t)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    lse = ref.einsum("hst->hs", host["S"], None, "ident", "lse")
    want = np.exp(host["S"].double().numpy() - lse[..., None])
    tol = 2e-2 if out_dtype == "bf16" else 1e-4
    assert maxnorm_rel_err(got, want) <= tol
    assert np.abs(got.sum(axis=2) - 1).max() <= (2e-2 if out_dtype == "bf16" else 1e-4)
