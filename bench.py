"""Benchmark of the extended-EinSum / TRA hot path on one MI355X.

Workload (one step): the pairwise squared distance D[i,k] = sum_j (X[i,j] -
Y[j,k])^2 with i = k = 8192, j = 256 (fp32, N(0,1) inputs) and its max-plus
variant Z[i,k] = max_j (X[i,j] + Y[j,k]) (int32, uniform [-1000, 1000]), both
under the partition vector d = [16, 1, 1, 16]:
  dense -> relation for X and Y (tra_repartition), join + aggregation
  (tra_execute), relation -> dense for the output (tra_repartition).
Plans are made once, before timing (host only).  Inputs are resident in HBM
before the timed region.

value = algorithmic operations of one step / step time, in GFLOP/s, counting
3 per (x-y)^2 + sum term and 2 per x+y / max term.

The JSON line also carries:
  roofline      the dominant kernel (squared-distance join) against the
                vector-ALU issue ceiling, timed with HIP events on its stream;
  cpu_baseline  the CPU oracle on a bounded sample of the same workload;
  extra         the other workloads measured in the same run (partitioned
                matmul, four-index contraction, blocked GEMM and its output
                repartition, attention EinGraph), each against its own roof.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published peaks and the vector-ALU issue ceiling derived from unit counts.
CU, CLK = 256, 2.4e9
HBM_PEAK = 8.0e12                 # bytes/s
BF16_MFMA_PEAK = 2.5166e15        # dense flop/s
# fp32 vector 157.3 TFLOP/s = 256 CUs x 128 fp32 lanes/clock x 2 (FMA) x 2.4 GHz, i.e.
# 78.6e12 single-instruction lane-ops per second (no packed math involved).
VALU_LANE_OPS = CU * 128 * CLK
# one (x-y)^2 + sum term = v_sub_f32 + v_fmac_f32: 2 lane-ops, counted as 3 flops
SQDIST_FLOP_PER_TERM = 3
SQDIST_OPS_PER_TERM = 2
VALU_SQDIST_PEAK = VALU_LANE_OPS / SQDIST_OPS_PER_TERM * SQDIST_FLOP_PER_TERM  # 117.96e12 flop/s

# HBM traffic of the squared-distance join kernel, from two rocprofv3 --pmc runs of
# `bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-extra` (FETCH_SIZE, then
# WRITE_SIZE, KiB per dispatch, mean over the dispatches), scaled by what the same
# counters read for a plain 1 GiB same-blocking copy (`bench.py --copy-probe 1024`):
# FETCH_SIZE read 524,300 KiB and WRITE_SIZE 1,048,576 KiB for 1,048,576 KiB moved,
# hence factors 2.0 and 1.0.  The record holds only while the kernel sources hash to
# `src_sha`; otherwise the kernel has changed since the counters were taken and
# `traffic` is reported as null.
TRAFFIC_SRCS = ("tensor_relational_algebra_amd/csrc/k_valu_tile.hip",
                "tensor_relational_algebra_amd/csrc/device_common.h",
                "tensor_relational_algebra_amd/csrc/tra_internal.h",
                "tensor_relational_algebra_amd/csrc/plan.h")
TRAFFIC_SQDIST = {"src_sha": "439559b799ea0b06", "fetch_kib": 40664.8, "write_kib": 262144.0,
                  "fetch_factor": 2.0, "write_factor": 1.0,
                  "profile": "profiles/valu_tile_sqdist_8192x256x8192_hbm_traffic.md"}


def _src_sha(paths) -> str:
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(rec) -> "float | None":
    """Calibrated HBM bytes per launch, or None when the record is stale or absent."""
    if rec["src_sha"] is None or rec["src_sha"] != _src_sha(TRAFFIC_SRCS):
        return None
    return 1024.0 * (rec["fetch_kib"] * rec["fetch_factor"] + rec["write_kib"] * rec["write_factor"])


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--only", default="", help="comma list of extra workloads to run")
    ap.add_argument("--src-sha", action="store_true", help="print the kernel-source hash the traffic record keys on")
    ap.add_argument("--calibrate", action="store_true",
                    help="measure the constants of the chooser's time model and print them as one JSON line")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB once per step with tra_repartition (same blocking on both sides); "
                         "the known-size reference for the HBM traffic counters")
    return ap.parse_args()


def _copy_probe(mib: int, reps: int) -> None:
    """A plain device copy of known size through the library's re-blocking kernel."""
    import torch

    import tensor_relational_algebra_amd as tra
    n = mib * (1 << 20) // 4
    src = torch.arange(n, dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    shape = [n // 1024, 1024]
    for _ in range(reps):
        tra.tra_repartition(src, shape, [1, 1], [1, 1], dst)
    torch.cuda.synchronize()
    assert torch.equal(src[-1024:], dst[-1024:])
    print(json.dumps({"copy_probe_bytes_each_way": n * 4, "reps": reps}), flush=True)


# (name, spec, bounds, d, join, agg, in dtype, out dtype, reps): one case per constant of
# the time model, each at a size where its kernel family is the planner's pick
CALIBRATION_CASES = [
    ("latency", "i,i->i", {"i": 8}, {"i": 1}, "add", "none", "f32", "f32", 400),
    ("mfma_tile0", "sa,ahd->shd", {"s": 4096, "a": 4096, "h": 32, "d": 128}, None, "mul", "sum", "bf16", "bf16", 20),
    ("mfma_tile1", "bij,bjk->bik", {"b": 256, "i": 128, "j": 512, "k": 128}, None, "mul", "sum", "bf16", "f32", 50),
    ("mfma_tile2", "bij,bjk->bik", {"b": 2048, "i": 64, "j": 256, "k": 64}, None, "mul", "sum", "bf16", "f32", 50),
    ("valu_tile", "ij,jk->ik", {"i": 8192, "j": 256, "k": 8192}, {"i": 16, "j": 1, "k": 16}, "sqdiff", "sum",
     "f32", "f32", 10),
    ("valu_tile_small_int", "ij,jk->ik", {"i": 8192, "j": 256, "k": 8192}, {"i": 16, "j": 1, "k": 16}, "add", "max",
     "i32", "i32", 10),
    ("rowreduce_compute", "ij,kj->ik", {"i": 2000, "j": 1000, "k": 2000}, None, "mul", "sum", "f32", "f32", 10),
    ("rowreduce_stream", "hst->hs", {"h": 32, "s": 4096, "t": 4096}, None, "ident", "lse", "f32", "f32", 10),
    ("generic", "ji,jk->ik", {"i": 1000, "j": 1000, "k": 1000}, None, "mul", "sum", "f32", "f32", 3),
    ("stream", "hst,hs->hst", {"h": 32, "s": 4096, "t": 4096}, None, "exp_sub", "none", "f32", "bf16", 10),
]


def _calibrate() -> None:
    """Measure the time model's constants: per case the average time of one
    tra_execute, join terms per ns, bytes per ns, and the model's prediction."""
    import torch

    import tensor_relational_algebra_amd as tra
    from tensor_relational_algebra_amd import workloads as wl
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    out = {}
    for k, (name, spec, bounds, d, join, agg, idt, odt, reps) in enumerate(CALIBRATION_CASES):
        labels = tra.tra_canonical_labels(spec)
        d = d or {c: 1 for c in labels}
        p = tra.tra_plan(spec, bounds, d, join, agg, idt, odt)
        ops = spec.split("->")[0].split(",")
        xs = [(wl.draw(9000 + 10 * k + i, [bounds[c] for c in o], "int", idt, lo=-1000, hi=1000) if idt == "i32"
               else wl.draw(9000 + 10 * k + i, [bounds[c] for c in o], "normal", idt, std=0.1)).to(dev).reshape(-1)
              for i, o in enumerate(ops)]
        z = torch.empty(p.info.z_elems, dtype=tra._binding.TORCH_DTYPES[p.out_dtype], device=dev)
        ws = p.workspace(dev)
        f = lambda: tra.tra_execute(p, xs[0], xs[1] if len(xs) > 1 else None, z, ws)
        f()
        ms = _events_time(f, reps, stream)
        terms = 1.0
        for c in labels:
            terms *= bounds[c]
        nbytes = p.info.x_bytes + p.info.y_bytes + p.info.z_bytes
        out[name] = {"kernel": p.kernel, "tile": p.info.tile, "split": p.info.agg_split, "us": round(ms * 1e3, 2),
                     "terms_per_ns": round(terms / (ms * 1e6), 2), "bytes_per_ns": round(nbytes / (ms * 1e6), 1),
                     "predicted_us": round(tra.tra_predict_ns(p) / 1e3, 2)}
        del xs, z, ws
    # back-to-back launches from the library (no Python between them): a chain of
    # 16 one-wavefront elementwise EinSum nodes run by one tra_graph_execute
    nodes = ["n0 einsum i,i->i i=64 @X,@Y0 in=f32 out=f32"]
    nodes += [f"n{i} einsum i,i->i i=64 n{i - 1},@Y{i} in=f32 out=f32" for i in range(1, 16)]
    g = tra.tra_graph_plan("\n".join(nodes), 1, [1] * 16)
    leaves = {n: torch.zeros(64, dtype=torch.float32, device=dev) for n in ["X"] + [f"Y{i}" for i in range(16)]}
    gw = g.workspace(dev)
    gout = torch.empty(64, dtype=torch.float32, device=dev)
    f = lambda: tra.tra_graph_execute(g, leaves, gout, gw)
    f()
    ms = _events_time(f, 50, stream)
    out["latency_graph_node"] = {"us_per_node": round(ms * 1e3 / 17, 2), "nodes_per_call": 16,
                                 "note": "16 nodes + the dense write-back of the output"}
    shape = [16384, 8192]
    src = torch.empty(shape, dtype=torch.float32, device=dev).reshape(-1)
    dst = torch.empty_like(src)
    f = lambda: tra.tra_repartition(src, shape, [16, 4], [4, 16], dst)
    f()
    ms = _events_time(f, 20, stream)
    out["copy"] = {"us": round(ms * 1e3, 2), "bytes_per_ns": round(2 * src.numel() * 4 / (ms * 1e6), 1),
                   "predicted_us": round(tra.tra_predict_repartition_ns(shape, "f32") / 1e3, 2)}
    print(json.dumps({"calibration": out}), flush=True)


def _events_time(fn, reps: int, stream) -> float:
    """Average milliseconds per call of fn(), HIP events on `stream`."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / reps


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the executor has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    if args.src_sha:
        print(_src_sha(TRAFFIC_SRCS))
        return
    if args.copy_probe:
        _copy_probe(args.copy_probe, max(args.steps, 1))
        return
    if args.calibrate:
        _calibrate()
        return
    import numpy as np
    import torch

    import tensor_relational_algebra_amd as tra
    from tensor_relational_algebra_amd import workloads as wl

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    sq, mp = wl.SQDIST, wl.MAXPLUS
    B = sq.bounds
    d = sq.d
    xs_h, ys_h = sq.make_inputs()
    xm_h, ym_h = mp.make_inputs()
    xs, ys, xm, ym = (t.to(dev) for t in (xs_h, ys_h, xm_h, ym_h))
    plan_sq = tra.tra_plan(sq.spec, B, d, sq.join, sq.agg, sq.in_dtype, sq.out_dtype)
    plan_mp = tra.tra_plan(mp.spec, B, d, mp.join, mp.agg, mp.in_dtype, mp.out_dtype)
    dx, dy, dz = [d["i"], d["j"]], [d["j"], d["k"]], [d["i"], d["k"]]
    sx, sy, sz = [B["i"], B["j"]], [B["j"], B["k"]], [B["i"], B["k"]]
    # resident buffers
    xr_s = torch.empty_like(xs).reshape(-1)
    yr_s = torch.empty_like(ys).reshape(-1)
    xr_m = torch.empty_like(xm).reshape(-1)
    yr_m = torch.empty_like(ym).reshape(-1)
    zr_s = torch.empty(plan_sq.info.z_elems, dtype=torch.float32, device=dev)
    zr_m = torch.empty(plan_mp.info.z_elems, dtype=torch.int32, device=dev)
    zd_s = torch.empty(sz, dtype=torch.float32, device=dev)
    zd_m = torch.empty(sz, dtype=torch.int32, device=dev)
    ws_m = plan_mp.workspace(dev)
    sq_ms, mp_ms = [], []

    def step(time_dominant: bool = False):
        tra.to_relation(xs, dx, xr_s)
        tra.to_relation(ys, dy, yr_s)
        if time_dominant:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        tra.tra_execute(plan_sq, xr_s, yr_s, zr_s)
        if time_dominant:
            e1.record(stream)
            sq_ms.append((e0, e1))
        tra.from_relation(zr_s, sz, dz, zd_s)
        tra.to_relation(xm, dx, xr_m)
        tra.to_relation(ym, dy, yr_m)
        if time_dominant:
            e2 = torch.cuda.Event(enable_timing=True)
            e3 = torch.cuda.Event(enable_timing=True)
            e2.record(stream)
        tra.tra_execute(plan_mp, xr_m, yr_m, zr_m, ws_m)
        if time_dominant:
            e3.record(stream)
            mp_ms.append((e2, e3))
        tra.from_relation(zr_m, sz, dz, zd_m)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(time_dominant=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    terms = B["i"] * B["j"] * B["k"]
    step_ops = terms * SQDIST_FLOP_PER_TERM + terms * 2
    value = step_ops / (ms_per_step * 1e-3) / 1e9
    sq_launch_ms = float(np.mean([a.elapsed_time(b) for a, b in sq_ms]))
    mp_launch_ms = float(np.mean([a.elapsed_time(b) for a, b in mp_ms]))
    mp_packed = not ws_m[-1024:].view(torch.int32).any().item()
    achieved = terms * SQDIST_FLOP_PER_TERM / (sq_launch_ms * 1e-3)
    traffic = _traffic(TRAFFIC_SQDIST)

    out = {
        "metric": "einsum GFLOP/s & % of MFMA peak; repartition GB/s & % HBM peak (1 GPU)",
        "value": round(value, 2),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32+i32",
        "data": "synthetic",
        "config": {"workload": "pairwise squared distance + max-plus, i=k=8192, j=256, d=[16,1,1,16] "
                               "(dense->relation, join+aggregate, relation->dense)",
                   "i": B["i"], "j": B["j"], "k": B["k"], "d": [d["i"], d["j"], d["j"], d["k"]],
                   "kernel": plan_sq.kernel},
        "roofline": {"bound": "alu", "achieved": round(achieved / 1e12, 3), "peak": round(VALU_SQDIST_PEAK / 1e12, 3),
                     "unit": "TFLOP/s", "frac": round(achieved / VALU_SQDIST_PEAK, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "kernel": "k_valu_tile<sqdiff,sum>", "launch_ms": round(sq_launch_ms, 4),
                     # algorithmic bytes: X and Y once, D once
                     "algorithmic_bytes": (B["i"] * B["j"] + B["j"] * B["k"] + B["i"] * B["k"]) * 4},
        # the max-plus join: range check + packed 16-bit kernel (exact on
        # integers within +-1024) or, if an input lies outside, the 32-bit kernel
        "maxplus": {"launch_ms": round(mp_launch_ms, 4), "Gterms/s": round(terms / (mp_launch_ms * 1e-3) / 1e9, 1),
                    "path": "packed f16, exact (inputs within +-1024)" if mp_packed else "int32"},
    }

    # zero-copy check of the timed outputs on a few rows against the oracle
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = _cpu_baseline(xs_h, ys_h, xm_h, ym_h, zd_s, zd_m)
    if not args.no_extra:
        only = set(filter(None, args.only.split(",")))
        out["extra"] = _extra(tra, wl, dev, stream, only)
    print(json.dumps(out), flush=True)


def _cpu_baseline(xs_h, ys_h, xm_h, ym_h, zd_s, zd_m):
    """The oracle (as it stands) on the first `rows` output rows of both joins."""
    import numpy as np
    from oracle import ref

    rows = 8192
    n_k = zd_s.shape[1]
    idx = np.arange(rows * n_k, dtype=np.int64)
    t = time.perf_counter()
    ws = ref.einsum("ij,jk->ik", xs_h, ys_h, "sqdiff", "sum", out_index=idx)
    wm = ref.einsum("ij,jk->ik", xm_h, ym_h, "add", "max", out_index=idx)
    dt = time.perf_counter() - t
    terms = rows * n_k * xs_h.shape[1]
    # the sampled rows of the timed GPU outputs agree with the oracle
    gs = zd_s[:rows].reshape(-1).cpu().double().numpy()
    gm = zd_m[:rows].reshape(-1).cpu().numpy().astype(np.int64)
    err = float(np.abs(gs - ws).max() / np.abs(ws).max())
    assert err <= 1e-4, f"squared distance differs from the oracle: {err}"
    assert np.array_equal(gm, wm), "max-plus differs from the oracle"
    return {"value": round(terms * (SQDIST_FLOP_PER_TERM + 2) / dt / 1e9, 3), "unit": "GFLOP/s",
            "cores": int(ref.max_threads()), "kind": "oracle",
            "sample": f"first {rows} of 8192 output rows of both joins ({terms / 1e9:.2f} G terms each), "
                      f"{dt:.1f} s; GPU rows checked: rel err {err:.2e}, max-plus exact"}


def _extra(tra, wl, dev, stream, only):
    import torch
    res = {}

    def want(name):
        return not only or name in only

    def timed_execute(plan, x, y, reps=10):
        z = torch.empty(plan.info.z_elems, dtype=tra._binding.TORCH_DTYPES[plan.out_dtype], device=dev)
        ws = plan.workspace(dev)
        for _ in range(2):
            tra.tra_execute(plan, x, y, z, ws)
        return _events_time(lambda: tra.tra_execute(plan, x, y, z, ws), reps, stream), z

    if want("matmul"):
        for base in (wl.MATMUL_F32, wl.MATMUL_I32):
            x, y = (t.to(dev) for t in base.make_inputs())
            for d4 in wl.MATMUL_D4:
                dm = wl.matmul_d(d4)
                p = tra.tra_plan(base.spec, base.bounds, dm, base.join, base.agg, base.in_dtype, base.out_dtype)
                xr = tra.to_relation(x, [dm["i"], dm["j"]])
                yr = tra.to_relation(y, [dm["j"], dm["k"]])
                ms, _ = timed_execute(p, xr, yr, reps=50)
                res[f"matmul_{base.in_dtype}_{'x'.join(map(str, d4))}"] = {
                    "us": round(ms * 1e3, 2), "GFLOP/s": round(2 * 256 ** 3 / ms / 1e6, 1), "kernel": p.kernel,
                    "split": p.info.agg_split}

    if want("contract4"):
        c = wl.CONTRACT4
        a, b = (t.to(dev) for t in c.make_inputs())
        p = tra.tra_plan(c.spec, c.bounds, c.d, c.join, c.agg, c.in_dtype, c.out_dtype)
        ar = tra.to_relation(a, [c.d[l] for l in "abef"])
        br = tra.to_relation(b, [c.d[l] for l in "cfed"])
        ms, _ = timed_execute(p, ar, br, reps=50)
        fl = 2 * 64 ** 4 * 32 ** 2
        res["contract4"] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(fl / ms / 1e9, 1),
                            "frac_bf16_mfma_peak": round(fl / (ms * 1e-3) / BF16_MFMA_PEAK, 4), "kernel": p.kernel}

    if want("gemm25d"):
        g = wl.GEMM25D
        x, a = (t.to(dev) for t in g.make_inputs())
        p = tra.tra_plan(g.spec, g.bounds, g.d, g.join, g.agg, g.in_dtype, g.out_dtype)
        xr = tra.to_relation(x, [g.d["i"], g.d["j"]])
        ar = tra.to_relation(a, [g.d["j"], g.d["k"]])
        del x, a
        ms, yr = timed_execute(p, xr, ar, reps=10)
        fl = 2 * 16384 * 8192 * 8192
        res["gemm25d"] = {"ms": round(ms, 4), "TFLOP/s": round(fl / ms / 1e9, 1),
                          "frac_bf16_mfma_peak": round(fl / (ms * 1e-3) / BF16_MFMA_PEAK, 4), "kernel": p.kernel}
        shape = [16384, 8192]
        dst = torch.empty_like(yr)
        f = lambda: tra.tra_repartition(yr, shape, list(wl.GEMM25D_Y_FROM), list(wl.GEMM25D_Y_TO), dst)
        f()
        ms = _events_time(f, 20, stream)
        nbytes = 2 * yr.numel() * 4
        res["gemm25d_repartition"] = {"us": round(ms * 1e3, 2), "GB/s": round(nbytes / ms / 1e6, 1),
                                      "frac_hbm_peak": round(nbytes / (ms * 1e-3) / HBM_PEAK, 4)}
        del xr, ar, yr, dst
        # backward products under the forward's blocking: dX = dY A^T, dA = X^T dY
        for name, spec, inputs in (("gemm25d_bwd_dX", "ik,jk->ij", ("ik", "jk")), ("gemm25d_bwd_dA", "ij,ik->jk", ("ij", "ik"))):
            pb = tra.tra_plan(spec, g.bounds, g.d, "mul", "sum", "bf16", "f32")
            ops = [wl.draw(1000 * 6 + t, [g.bounds[c] for c in lab], "normal", "bf16", std=0.02).to(dev)
                   for t, lab in enumerate(inputs)]
            rels = [tra.to_relation(o, [g.d[c] for c in lab]) for o, lab in zip(ops, inputs)]
            del ops
            ms, zb = timed_execute(pb, rels[0], rels[1], reps=10)
            res[name] = {"ms": round(ms, 4), "TFLOP/s": round(fl / ms / 1e9, 1),
                         "frac_bf16_mfma_peak": round(fl / (ms * 1e-3) / BF16_MFMA_PEAK, 4), "kernel": pb.kernel,
                         "operands": "X^T" if spec.startswith("ij,ik") else "Y^T"}
            del rels, zb

    if want("mha"):
        res["mha"] = _mha(tra, wl, dev, stream)
    if want("mha_fused"):
        res["mha_fused"] = _mha(tra, wl, dev, stream, fuse=True)
    if want("mha_overlap"):
        res["mha_overlap"] = _mha(tra, wl, dev, stream, overlap=True)
    if want("mha_time"):
        res["mha_time"] = _mha(tra, wl, dev, stream, time_model=True)
    if want("mha_fused_time"):
        res["mha_fused_time"] = _mha(tra, wl, dev, stream, fuse=True, time_model=True)
    if want("mha_bwd"):
        res["mha_bwd"] = _mha_backward(tra, wl, dev, stream)
        # the softmax Jacobian in the dAttn product's epilogue (opt-in, for comparison)
        res["mha_bwd_product_chain"] = _mha_backward(tra, wl, dev, stream, fuse=True)
    torch.cuda.empty_cache()
    return res


def _mha(tra, wl, dev, stream, fuse=False, time_model=False, overlap=False):
    """The attention layer as an EinGraph, d chosen for P = 256; per-node time
    (its input repartitions included) against the node's own roof.  With
    fuse=True the scores -> softmax -> weighted-sum chain runs as one kernel,
    timed on the weighted-sum node (the scores and softmax nodes enqueue nothing)."""
    import torch
    case = wl.MHA
    desc = case.graph_desc()
    flags = (tra.GRAPH_FUSE_ATTENTION if fuse else 0) | (tra.GRAPH_CHOOSE_TIME if time_model else 0) | \
        (tra.GRAPH_OVERLAP_COPIES if overlap else 0)
    g = tra.tra_graph_plan_ex(desc, 256, None, flags)
    inputs = {k: v.to(dev) for k, v in case.make_inputs().items()}
    ws = g.workspace(dev)
    out = torch.empty(g.info.out_elems, dtype=torch.float32, device=dev)
    names = [l.split()[0] for l in desc.splitlines()]
    s, a, h, dh = case.s, case.a, case.h, case.dh
    gemm = 2.0 * s * a * h * dh          # every projection and the output projection
    attn_fl = 2.0 * h * s * s * dh       # scores and weighted sum
    flops = {"Q_proj": gemm, "K_proj": gemm, "V_proj": gemm, "Scores": attn_fl, "O": attn_fl, "Output": gemm}
    # bytes the HBM-bound nodes must move at least: scores write fp32 S; softmax reads
    # S once (one pass per row) and writes bf16 Attn; weighted sum reads Attn
    sbytes = {"Scores": 4.0 * h * s * s, "Attn": 4.0 * h * s * s + 2.0 * h * s * s, "O": 2.0 * h * s * s}
    if fuse:
        # the fused node does the scores and the weighted sum; nothing is HBM-bound
        flops = dict(flops, O=2 * attn_fl, Scores=0.0)
        sbytes = {}
    for _ in range(2):
        tra.tra_graph_execute(g, inputs, out, ws)
    reps = 5
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(reps)]
    for r in range(reps):
        ev[r][0].record(stream)
        for i in range(len(names)):
            tra.tra_graph_run_node(g, i, inputs, out if i == len(names) - 1 else None, ws)
            ev[r][i + 1].record(stream)
    torch.cuda.synchronize()
    nodes = {}
    total = 0.0
    for i, n in enumerate(names):
        ms = sum(ev[r][i].elapsed_time(ev[r][i + 1]) for r in range(reps)) / reps
        total += ms
        e = {"us": round(ms * 1e3, 1), "d": g.node_d(i)}
        if n in flops and flops[n] > 0:
            e["TFLOP/s"] = round(flops[n] / ms / 1e9, 1)
            e["frac_bf16_mfma_peak"] = round(flops[n] / (ms * 1e-3) / BF16_MFMA_PEAK, 4)
        if n in sbytes:
            e["GB/s"] = round(sbytes[n] / ms / 1e6, 1)
            e["frac_hbm_peak"] = round(sbytes[n] / (ms * 1e-3) / HBM_PEAK, 4)
        nodes[n] = e
    total_fl = sum(flops.values())
    # the whole layer as one tra_graph_execute call (copies on a side stream
    # when overlapped; the per-node figures above run each node in order)
    graph_ms = _events_time(lambda: tra.tra_graph_execute(g, inputs, out, ws), reps, stream)
    r = {"ms": round(total, 3), "graph_ms": round(graph_ms, 3), "TFLOP/s": round(total_fl / total / 1e9, 1),
         "nodes": nodes,
         "repartitions": g.info.n_repartitions, "fused_chains": g.info.n_fused,
         "workspace_GB": round(g.info.workspace_bytes / 1e9, 2),
         "chooser": "time model" if time_model else "pages (numbers moved, P = 256)",
         "copies": "side stream, overlapped" if overlap else "in order"}
    if time_model and not fuse:
        r["predicted_ms"] = round(g.info.cost / 1e6, 3)
    return r


def _mha_backward(tra, wl, dev, stream, fuse=False):
    """Backward EinSums of the attention layer (dense layouts), per step and in
    total, each step against its own roof: the products against the bf16 matrix-core
    peak, the [h,s,t] elementwise steps against HBM."""
    import torch
    case = wl.MHA
    s, a, h, dh = case.s, case.a, case.h, case.dh
    layer = tra.AttentionLayer(s, a, h, dh, fuse_product_chain=fuse)
    inputs = {k: v.to(dev) for k, v in case.make_inputs().items()}
    ws = layer.workspace(dev)
    saved = layer.forward(inputs, ws)
    g = case.make_output_gradient().to(dev)
    grads = layer.backward(saved, g, ws)
    proj, attn = 2.0 * s * a * h * dh, 2.0 * h * s * s * dh
    flops = {n: proj for n in ("dO", "dW_O", "dW_Q", "dQ", "dW_K", "dK", "dW_V", "dV")}
    flops.update({n: attn for n in ("dAttn", "dV_proj", "dQ_proj", "dK_proj")})
    hst = float(h * s * s)
    names = list(layer.backward_launches)
    if layer.fuse_product_chain:
        # dScores = Attn * (dO.V^T - Rows) in the product's epilogue
        flops["dScores"] = attn
        sbytes = {}
    else:
        # dScores runs chained with dAttn_c: reads dAttn (fp32) and Attn (bf16), writes bf16
        sbytes = {"dScores": 8 * hst}
    reps = 5
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(reps)]
    for r in range(reps):
        k = iter(range(1, len(names) + 1))
        ev[r][0].record(stream)
        grads = layer.backward(saved, g, ws, on_step=lambda n: ev[r][next(k)].record(stream), out=grads)
    torch.cuda.synchronize()
    steps, total = {}, 0.0
    for i, n in enumerate(names):
        ms = sum(ev[r][i].elapsed_time(ev[r][i + 1]) for r in range(reps)) / reps
        total += ms
        e = {"us": round(ms * 1e3, 1), "kernel": layer.plans[n].kernel}
        chained = [a for a, b in tra.attention.CHAINED.items() if b == n]
        if chained and layer.fuse_product_chain:
            e["kernel"] = layer.plans["dAttn"].kernel
            e["chained_with"] = ["dAttn", chained[0]]
        elif chained:
            e["chained_with"] = chained[0]
        if n in flops:
            e["TFLOP/s"] = round(flops[n] / ms / 1e9, 1)
            e["frac_bf16_mfma_peak"] = round(flops[n] / (ms * 1e-3) / BF16_MFMA_PEAK, 4)
        if n in sbytes:
            e["GB/s"] = round(sbytes[n] / ms / 1e6, 1)
            e["frac_hbm_peak"] = round(sbytes[n] / (ms * 1e-3) / HBM_PEAK, 4)
        steps[n] = e
    fl = sum(flops.values())
    return {"ms": round(total, 3), "TFLOP/s": round(fl / total / 1e9, 1), "steps": steps}


if __name__ == "__main__":
    main()
