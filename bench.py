"""Benchmark of the extended-EinSum / TRA hot path on one MI355X.

Workload (one step): the 2.5D-blocked product Y = X A of the page "ColossalAI
2.5D 张量并行深度解析" (section on partitioning Y = XA) with X 16384 x 8192 and
A 8192 x 8192 (bf16, N(0, 0.02) inputs, fp32 accumulate and output): X cut
into depth*q = 16 row blocks and q = 4 column blocks, A into 4 x 4 blocks, so
the TRA partition vector over (i, k, j) is [16, 4, 4].  One step is
  join + aggregation (tra_execute: 256 key-matched block products folded
  4 per output block) and
  the re-cut of Y from [16, 4] to [4, 16] blocks for the next layer
  (tra_repartition),
with X and A already resident in HBM in their relation layout (the initial
dense -> relation copy is timed once, apart, and reported as layout_ms).
Plans are made once, before timing (host only).

value = the product's 2*16384*8192*8192 flop per step / step time (GFLOP/s).

The JSON line also carries:
  roofline              the product's kernel against the bf16 matrix-core peak,
                        timed with HIP events on its stream;
  roofline_repartition  the re-cut against HBM bandwidth;
  parity                the timed output on sampled rows against the oracle;
  cpu_baseline          the CPU oracle on those rows;
  extra                 the other workloads measured in the same run (pairwise
                        squared distance and max-plus, partitioned matmul,
                        four-index contraction, the product's backward, the
                        attention EinGraph), each against its own roof.
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

# HBM traffic per launch of a kernel, from two rocprofv3 --pmc runs (FETCH_SIZE,
# then WRITE_SIZE, KiB per dispatch, mean over the kernel's dispatches), scaled by
# what the same counters read for a plain 1 GiB same-blocking copy
# (`bench.py --copy-probe 1024`).  A record holds only while the kernel's sources
# hash to `src_sha`; otherwise the kernel has changed since the counters were taken
# and `traffic` is reported as null.
COMMON_SRCS = ("tensor_relational_algebra_amd/csrc/device_common.h",
               "tensor_relational_algebra_amd/csrc/tra_internal.h",
               "tensor_relational_algebra_amd/csrc/plan.h")
TRAFFIC_SRCS = {
    "sqdist": ("tensor_relational_algebra_amd/csrc/k_valu_tile.hip",) + COMMON_SRCS,
    "gemm": ("tensor_relational_algebra_amd/csrc/k_mfma4k.hip", "tensor_relational_algebra_amd/csrc/mfma_common.h")
    + COMMON_SRCS,
    "recut": ("tensor_relational_algebra_amd/csrc/k_simple.hip",) + COMMON_SRCS,
}
# squared distance: `bench.py --steps 3 --warmup 1 --no-cpu-baseline --only sqdist`;
# the blocked GEMM and its re-cut: `bench.py --steps 3 --warmup 1 --no-cpu-baseline
# --no-extra`.  The copy calibration was taken in the same session: FETCH_SIZE read
# 524,336 KiB and WRITE_SIZE 1,048,619 KiB for the 1,048,576 KiB copy, hence factors
# 2.0 and 1.0.
TRAFFIC = {
    "sqdist": {"src_sha": "e60d668d8529fb0d", "fetch_kib": 40698.5, "write_kib": 262144.0,
               "fetch_factor": 2.0, "write_factor": 1.0,
               "profile": "profiles/valu_tile_sqdist_8192x256x8192_hbm_traffic.md"},
    "gemm": {"src_sha": "be99c0e01da4d16d", "fetch_kib": 1573102.0, "write_kib": 524294.8,
             "fetch_factor": 2.0, "write_factor": 1.0,
             "profile": "profiles/mfma4k_gemm25d_16384x8192x8192_hbm_traffic.md"},
    "recut": {"src_sha": "27b277ed94e55d19", "fetch_kib": 262179.3, "write_kib": 524290.8,
              "fetch_factor": 2.0, "write_factor": 1.0,
              "profile": "profiles/mfma4k_gemm25d_16384x8192x8192_hbm_traffic.md"},
}


def _src_sha(paths) -> str:
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(name: str) -> "float | None":
    """Calibrated HBM bytes per launch, or None when the record is stale or absent."""
    rec = TRAFFIC[name]
    if rec["src_sha"] is None or rec["src_sha"] != _src_sha(TRAFFIC_SRCS[name]):
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
    ap.add_argument("--src-sha", action="store_true", help="print the kernel-source hashes the traffic records key on")
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
    ("mfma_tile3", "sa,ahd->shd", {"s": 4096, "a": 4096, "h": 32, "d": 128}, None, "mul", "sum", "bf16", "bf16", 20),
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


def _events_time_flushed(fn, reps: int, stream, scratch) -> float:
    """Average milliseconds of fn() over `reps` calls, HIP events on `stream`
    around each call, with a read-modify-write pass over `scratch` (>= 1 GiB)
    before each so that no call finds its inputs in the 256 MB Infinity Cache."""
    import torch
    evs = []
    for _ in range(reps):
        scratch.add_(1)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / reps


def _measured_roofs(tra, dev, stream) -> dict:
    """The machine's own ceilings beside the published ones: back-to-back bf16
    matrix-core products on register operands (one wave per SIMD), once with
    one operand pair and once with random operands that change from product
    to product as in a real product, and a 1 GiB same-blocking copy through
    tra_repartition."""
    import torch
    wg, iters = 1024, 20000
    out = torch.empty(wg * 256, dtype=torch.float32, device=dev)
    loops = {}
    for key, mode in (("mfma_loop", 0), ("mfma_loop_random_operands", 1), ("mfma16_loop_random_operands", 2)):
        it = iters if mode < 2 else iters // 4
        fl = (2.0 * 32 * 32 * 16 * 8 if mode < 2 else 2.0 * 16 * 16 * 32 * 64) * 4 * it * wg
        tra.tra_probe_mfma_loop(wg, 100, out, mode)
        ms = _events_time(lambda: tra.tra_probe_mfma_loop(wg, it, out, mode), 3, stream)
        what = (f"{wg} workgroups x 4 waves, {it} rounds of 8 independent 32x32x16 bf16 products"
                + (", 8 random operand pairs" if mode else ", one operand pair")) if mode < 2 else \
            f"{wg} workgroups x 4 waves, {it} rounds of 64 independent 16x16x32 bf16 products, 8 random operand pairs"
        loops[key] = {"TFLOP/s": round(fl / ms / 1e9, 1), "frac_of_published": round(fl / (ms * 1e-3) / BF16_MFMA_PEAK, 4),
                      "what": what}
    n = 1 << 28
    src = torch.zeros(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    shape = [n // 1024, 1024]
    cp = lambda: tra.tra_repartition(src, shape, [1, 1], [1, 1], dst)
    cp()
    cms = _events_time(cp, 5, stream)
    return {**loops,
            "copy": {"GB/s": round(2.0 * n * 4 / cms / 1e6, 1), "frac_of_published": round(2.0 * n * 4 / (cms * 1e-3) / HBM_PEAK, 4),
                     "what": "1 GiB read + 1 GiB written, tra_repartition between identical blockings"}}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _sample_rows(n_rows: int, n_blocks: int, per_block: int, seed: int):
    """`per_block` distinct rows in each of `n_blocks` equal row blocks, seeded."""
    import numpy as np
    rng = np.random.default_rng(seed)
    b = n_rows // n_blocks
    return np.sort(np.concatenate([k * b + rng.choice(b, size=per_block, replace=False) for k in range(n_blocks)]))


def rel_errors(got, want, floor: float = 1e-2) -> dict:
    """Max-norm relative error max|g - r| / max|r| (the gate) and the element-wise
    relative error |g - r| / |r| over elements with |r| >= floor * max|r|."""
    import numpy as np
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    big = float(np.abs(want).max()) if want.size else 0.0
    diff = np.abs(got - want)
    mask = np.abs(want) >= floor * big
    return {"maxnorm": float(diff.max() / big) if big > 0 else float(diff.max(initial=0.0)),
            "elementwise_floored": float((diff[mask] / np.abs(want[mask])).max()) if mask.any() else 0.0,
            "floor": floor, "elements": int(want.size)}


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the executor has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    if args.src_sha:
        print(json.dumps({k: _src_sha(v) for k, v in TRAFFIC_SRCS.items()}))
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

    g = wl.GEMM25D
    B = g.bounds
    shape_y = [B["i"], B["k"]]
    x_h, a_h = g.make_inputs()
    plan = tra.tra_plan(g.spec, B, g.d, g.join, g.agg, g.in_dtype, g.out_dtype)
    dx, da = [g.d["i"], g.d["j"]], [g.d["j"], g.d["k"]]
    x, a = x_h.to(dev), a_h.to(dev)
    xr = torch.empty(x.numel(), dtype=x.dtype, device=dev)
    ar = torch.empty(a.numel(), dtype=a.dtype, device=dev)
    # the initial partition of the inputs (dense -> relation), timed apart
    # after one untimed call
    lay = lambda: (tra.to_relation(x, dx, xr), tra.to_relation(a, da, ar))
    lay()
    layout_ms = _events_time(lay, 3, stream)
    del x, a
    yr = torch.empty(plan.info.z_elems, dtype=torch.float32, device=dev)
    y2 = torch.empty_like(yr)
    ws = plan.workspace(dev)
    y_from, y_to = list(wl.GEMM25D_Y_FROM), list(wl.GEMM25D_Y_TO)
    gemm_ev, recut_ev = [], []

    def step(rec: bool = False):
        if rec:
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
        tra.tra_execute(plan, xr, ar, yr, ws)
        if rec:
            e[1].record(stream)
        tra.tra_repartition(yr, shape_y, y_from, y_to, y2)
        if rec:
            e[2].record(stream)
            gemm_ev.append((e[0], e[1]))
            recut_ev.append((e[1], e[2]))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(rec=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    flops = 2.0 * B["i"] * B["j"] * B["k"]
    value = flops / (ms_per_step * 1e-3) / 1e9
    gemm_ms = float(np.mean([p.elapsed_time(q) for p, q in gemm_ev]))
    recut_ms = float(np.mean([p.elapsed_time(q) for p, q in recut_ev]))
    achieved = flops / (gemm_ms * 1e-3)
    recut_bytes = 2.0 * yr.numel() * 4
    recut_rate = recut_bytes / (recut_ms * 1e-3)
    traffic = _traffic("gemm")
    traffic_recut = _traffic("recut")

    out = {
        "metric": "einsum GFLOP/s & % of MFMA peak; repartition GB/s & % HBM peak (1 GPU)",
        "value": round(value, 1),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "2.5D-blocked GEMM Y = X A, X 16384x8192, A 8192x8192, bf16 in, fp32 accumulate "
                               "and out, TRA partition (i,k,j) = [16,4,4] (depth 4, q 4), then Y re-cut from "
                               "[16,4] to [4,16] blocks; inputs resident as relations",
                   "i": B["i"], "j": B["j"], "k": B["k"], "d_ikj": [g.d["i"], g.d["k"], g.d["j"]],
                   "y_from": y_from, "y_to": y_to, "kernel": plan.kernel, "tile": plan.info.tile,
                   "agg_split": plan.info.agg_split},
        "roofline": {"bound": "mfma", "achieved": round(achieved / 1e12, 2), "peak": round(BF16_MFMA_PEAK / 1e12, 1),
                     "unit": "TFLOP/s", "frac": round(achieved / BF16_MFMA_PEAK, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "kernel": {4: "k_mfma4k_bf16", 3: "k_mfma4_bf16"}.get(plan.info.tile, "k_mfma_bf16"), "launch_ms": round(gemm_ms, 4),
                     "flop_per_launch": flops,
                     # algorithmic bytes: X and A read once, Y written once
                     "algorithmic_bytes": (B["i"] * B["j"] + B["j"] * B["k"]) * 2 + B["i"] * B["k"] * 4},
        "roofline_repartition": {"bound": "hbm", "achieved": round(recut_rate / 1e9, 1),
                                 "peak": round(HBM_PEAK / 1e9, 1), "unit": "GB/s",
                                 "frac": round(recut_rate / HBM_PEAK, 4),
                                 "traffic": None if traffic_recut is None else round(traffic_recut),
                                 "kernel": "k_repartition_p2", "launch_ms": round(recut_ms, 4),
                                 "algorithmic_bytes": recut_bytes},
        "layout_ms": round(layout_ms, 4),
    }

    # the timed output (re-cut to [4,16]) on sampled rows against the oracle
    rows = _sample_rows(B["i"], g.d["i"], 4, seed=5005)
    y_dense = tra.from_relation(y2, shape_y, y_to)
    got = y_dense[torch.from_numpy(rows).to(dev)].cpu().double().numpy()
    del y_dense
    if not args.no_cpu_baseline:
        out["cpu_baseline"], want = _cpu_baseline(x_h, a_h, rows, g)
        err = rel_errors(got.reshape(-1), want)
        err["rows"] = len(rows)
        out["parity"] = err
        assert err["maxnorm"] <= 2e-2, f"blocked GEMM differs from the oracle: {err}"
    if not args.no_extra:
        only = set(filter(None, args.only.split(",")))
        del xr, ar, yr, y2
        torch.cuda.empty_cache()
        if not only or "roofs" in only:
            out["measured_roofs"] = _measured_roofs(tra, dev, stream)
        out["extra"] = _extra(tra, wl, dev, stream, only)
    print(json.dumps(out), flush=True)


def _cpu_baseline(x_h, a_h, rows, g):
    """The oracle (as it stands) on the sampled output rows of the blocked GEMM."""
    import numpy as np
    from oracle import ref

    n_k = g.bounds["k"]
    idx = (rows[:, None] * n_k + np.arange(n_k)[None, :]).reshape(-1)
    t = time.perf_counter()
    want = ref.einsum(g.spec, x_h, a_h, g.join, g.agg, out_index=idx)
    dt = time.perf_counter() - t
    fl = 2.0 * len(rows) * n_k * g.bounds["j"]
    return ({"value": round(fl / dt / 1e9, 3), "unit": "GFLOP/s", "cores": int(ref.max_threads()),
             "cpu_model": _cpu_model(), "kind": "oracle",
             "sample": f"{len(rows)} of 16384 output rows of the blocked GEMM (4 seeded rows in each of the 16 row "
                       f"blocks), every column: {fl / 1e9:.1f} GFLOP in {dt:.1f} s"}, want)


def _sqdist(tra, wl, dev, stream, scratch, check_rows: int = 256):
    """Pairwise squared distance and max-plus, 8192 x 256 x 8192, d = [16,1,1,16];
    each join timed alone (inputs resident as relations, caches flushed between
    calls), the squared distance against the vector-ALU ceiling."""
    import numpy as np
    import torch
    from oracle import ref
    res = {}
    for case in (wl.SQDIST, wl.MAXPLUS):
        B, d = case.bounds, case.d
        x_h, y_h = case.make_inputs()
        p = tra.tra_plan(case.spec, B, d, case.join, case.agg, case.in_dtype, case.out_dtype)
        xr = tra.to_relation(x_h.to(dev), [d["i"], d["j"]])
        yr = tra.to_relation(y_h.to(dev), [d["j"], d["k"]])
        z = torch.empty(p.info.z_elems, dtype=tra._binding.TORCH_DTYPES[p.out_dtype], device=dev)
        ws = p.workspace(dev)
        f = lambda: tra.tra_execute(p, xr, yr, z, ws)
        f()
        ms = _events_time_flushed(f, 10, stream, scratch)
        terms = B["i"] * B["j"] * B["k"]
        zd = tra.from_relation(z, [B["i"], B["k"]], [d["i"], d["k"]])
        rows = _sample_rows(B["i"], d["i"], check_rows // d["i"], seed=2000 + case.wid)
        idx = (rows[:, None] * B["k"] + np.arange(B["k"])[None, :]).reshape(-1)
        want = ref.einsum(case.spec, x_h, y_h, case.join, case.agg, out_index=idx)
        got = zd[torch.from_numpy(rows).to(dev)].cpu().reshape(-1)
        if case.join == "sqdiff":
            achieved = terms * SQDIST_FLOP_PER_TERM / (ms * 1e-3)
            traffic = _traffic("sqdist")
            err = rel_errors(got.double().numpy(), want)
            assert err["maxnorm"] <= 1e-4, f"squared distance differs from the oracle: {err}"
            res["sqdist"] = {
                "ms": round(ms, 4), "TFLOP/s": round(achieved / 1e12, 2), "kernel": p.kernel,
                "roofline": {"bound": "alu", "achieved": round(achieved / 1e12, 3),
                             "peak": round(VALU_SQDIST_PEAK / 1e12, 3), "unit": "TFLOP/s",
                             "frac": round(achieved / VALU_SQDIST_PEAK, 4),
                             "traffic": None if traffic is None else round(traffic),
                             "kernel": "k_valu_tile<sqdiff,sum>",
                             "algorithmic_bytes": (B["i"] * B["j"] + B["j"] * B["k"] + B["i"] * B["k"]) * 4},
                "parity": dict(err, rows=len(rows))}
        else:
            exact = bool(np.array_equal(got.numpy().astype(np.int64), want))
            assert exact, "max-plus differs from the oracle"
            packed = not ws[-1024:].view(torch.int32).any().item()
            res["maxplus"] = {"ms": round(ms, 4), "Gterms/s": round(terms / (ms * 1e-3) / 1e9, 1),
                              "kernel": p.kernel,
                              "path": "packed f16, exact (inputs within +-1024)" if packed else "int32",
                              "parity": {"exact": exact, "rows": len(rows)}}
        del xr, yr, z, zd, ws
    return res


def _extra(tra, wl, dev, stream, only):
    import torch
    res = {}

    def want(name):
        return not only or name in only

    # a read-modify-write pass over 1 GiB between timed calls of the small
    # workloads, so that their inputs never sit in the 256 MB Infinity Cache
    scratch = torch.zeros(1 << 28, dtype=torch.float32, device=dev)

    def timed_execute(plan, x, y, reps=10, flush=False):
        z = torch.empty(plan.info.z_elems, dtype=tra._binding.TORCH_DTYPES[plan.out_dtype], device=dev)
        ws = plan.workspace(dev)
        for _ in range(2):
            tra.tra_execute(plan, x, y, z, ws)
        f = lambda: tra.tra_execute(plan, x, y, z, ws)
        if flush:
            return _events_time_flushed(f, reps, stream, scratch), z
        return _events_time(f, reps, stream), z

    if want("sqdist"):
        res.update(_sqdist(tra, wl, dev, stream, scratch))

    if want("ragged"):
        # the squared distance at 8000 x 256 x 8000 (no tile divides 8000;
        # relation blocks of 500): masked edge tiles on the same kernel
        c = wl.SQDIST.scaled({"i": 8000, "j": 256, "k": 8000}, wl.SQDIST.d)
        x_h, y_h = c.make_inputs()
        p = tra.tra_plan(c.spec, c.bounds, c.d, c.join, c.agg, c.in_dtype, c.out_dtype)
        xr = tra.to_relation(x_h.to(dev), [c.d["i"], c.d["j"]])
        yr = tra.to_relation(y_h.to(dev), [c.d["j"], c.d["k"]])
        ms, _ = timed_execute(p, xr, yr, reps=10, flush=True)
        terms = 8000 * 256 * 8000
        res["sqdist_8000"] = {"ms": round(ms, 4), "TFLOP/s": round(terms * SQDIST_FLOP_PER_TERM / ms / 1e9, 2),
                              "kernel": p.kernel,
                              "frac_alu": round(terms * SQDIST_FLOP_PER_TERM / (ms * 1e-3) / VALU_SQDIST_PEAK, 4)}
        if "sqdist" in res:
            res["sqdist_8000"]["time_vs_8192"] = round(ms / res["sqdist"]["ms"], 3)
        del xr, yr

    if want("matmul"):
        for base in (wl.MATMUL_F32, wl.MATMUL_I32):
            x, y = (t.to(dev) for t in base.make_inputs())
            for d4 in wl.MATMUL_D4:
                dm = wl.matmul_d(d4)
                p = tra.tra_plan(base.spec, base.bounds, dm, base.join, base.agg, base.in_dtype, base.out_dtype)
                xr = tra.to_relation(x, [dm["i"], dm["j"]])
                yr = tra.to_relation(y, [dm["j"], dm["k"]])
                ms, _ = timed_execute(p, xr, yr, reps=50, flush=True)
                res[f"matmul_{base.in_dtype}_{'x'.join(map(str, d4))}"] = {
                    "us": round(ms * 1e3, 2), "GFLOP/s": round(2 * 256 ** 3 / ms / 1e6, 1), "kernel": p.kernel,
                    "split": p.info.agg_split}

    if want("contract4"):
        import numpy as np
        from oracle import ref
        c = wl.CONTRACT4
        a_h, b_h = c.make_inputs()
        p = tra.tra_plan(c.spec, c.bounds, c.d, c.join, c.agg, c.in_dtype, c.out_dtype)
        ar = tra.to_relation(a_h.to(dev), [c.d[l] for l in "abef"])
        br = tra.to_relation(b_h.to(dev), [c.d[l] for l in "cfed"])
        ms, zr = timed_execute(p, ar, br, reps=50, flush=True)
        ms_warm, _ = timed_execute(p, ar, br, reps=50)
        fl = 2 * 64 ** 4 * 32 ** 2
        zd = tra.from_relation(zr, [64] * 4, [c.d[l] for l in "abcd"]).reshape(-1)
        idx = np.sort(np.random.default_rng(3003).choice(zd.numel(), size=1 << 14, replace=False))
        ref_vals = ref.einsum(c.spec, a_h, b_h, c.join, c.agg, out_index=idx)
        err = rel_errors(zd[torch.from_numpy(idx).to(dev)].cpu().double().numpy(), ref_vals)
        assert err["maxnorm"] <= 2e-2, f"four-index contraction differs from the oracle: {err}"
        res["contract4"] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(fl / ms / 1e9, 1),
                            "frac_bf16_mfma_peak": round(fl / (ms * 1e-3) / BF16_MFMA_PEAK, 4), "kernel": p.kernel,
                            "us_cache_warm": round(ms_warm * 1e3, 2), "split": p.info.agg_split,
                            "parity": err}

    if want("gemm25d_bwd"):
        g = wl.GEMM25D
        fl = 2 * 16384 * 8192 * 8192
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
        # the default: the softmax Jacobian in the dAttn product's epilogue
        res["mha_bwd"] = _mha_backward(tra, wl, dev, stream)
        # for comparison: the product writes the fp32 dAttn, the chain follows
        res["mha_bwd_three_launches"] = _mha_backward(tra, wl, dev, stream, fuse=False)
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


def _mha_backward(tra, wl, dev, stream, fuse=True):
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
    names = []
    grads = layer.backward(saved, g, ws, on_step=names.append, out=grads)
    assert names == list(layer.backward_launches)
    if layer.fuse_product_chain:
        # dScores = Attn * (dO.V^T - Rows) in the product's epilogue
        flops["dScores"] = attn
        sbytes = {}
    else:
        # dScores runs chained with dAttn_c: reads dAttn (fp32) and Attn (bf16), writes bf16
        sbytes = {"dScores": 8 * hst}
    import gc
    gc.collect()
    torch.cuda.synchronize()
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
