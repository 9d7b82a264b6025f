"""ctypes binding of libtra (include/tra.h): argument marshalling only.

Every function here converts Python / torch arguments to the C ABI, calls the
library, and turns a negative status into ``TraError``.  All computation runs
in the library's HIP kernels; there is no Python or CPU fallback, and a
missing library raises at the first call.  torch supplies device memory and
the current HIP stream.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence, Tuple, Union

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# TRA_LIBRARY names another build of the library (the sanitizer run of the CPU
# suite loads an ASan/UBSan build of the host code this way)
LIB_PATH = os.environ.get("TRA_LIBRARY") or os.path.join(_PKG, "_build", "libtra.so")

DTYPES = {"f32": 0, "bf16": 1, "i32": 2}
TORCH_DTYPES = {0: torch.float32, 1: torch.bfloat16, 2: torch.int32}
DTYPE_OF_TORCH = {torch.float32: 0, torch.bfloat16: 1, torch.int32: 2}
JOINS = {"mul": 0, "sqdiff": 1, "add": 2, "ident": 3, "exp_sub": 4, "sub": 5}
AGGS = {"none": 0, "sum": 1, "max": 2, "min": 3, "lse": 4}
KERNELS = {0: "generic", 1: "elemwise", 2: "rowreduce", 3: "valu_tile", 4: "mfma_bf16", 5: "empty"}


class TraError(RuntimeError):
    def __init__(self, code: int, what: str, detail: str):
        super().__init__(f"{what} (status {code}): {detail}")
        self.code = code


class PlanInfo(ctypes.Structure):
    _fields_ = [("n_tasks", ctypes.c_int64), ("n_groups", ctypes.c_int64), ("n_agg", ctypes.c_int64),
                ("agg_split", ctypes.c_int64), ("x_elems", ctypes.c_int64), ("y_elems", ctypes.c_int64),
                ("z_elems", ctypes.c_int64), ("x_bytes", ctypes.c_size_t), ("y_bytes", ctypes.c_size_t),
                ("z_bytes", ctypes.c_size_t), ("workspace_bytes", ctypes.c_size_t), ("kernel", ctypes.c_int32),
                ("n_labels", ctypes.c_int32), ("labels", ctypes.c_char * 32), ("tile", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libtra.so (built in-tree by ``build()``); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libtra is not built ({LIB_PATH} missing); run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        sig = {
            "tra_plan": ([ctypes.c_char_p, P, P, I, I, I, I, I, ctypes.c_float, P], I),
            "tra_plan_info": ([P, P], I),
            "tra_plan_destroy": ([P], I),
            "tra_execute": ([P, P, P, P, P, ctypes.c_size_t, P], I),
            "tra_execute_static": ([P, P, P, P, P], I),
            "tra_probe_mfma_loop": ([I, I, I, P, P], I),
            "tra_static_scratch_bytes": ([], ctypes.c_size_t),
            "tra_execute_chain": ([P, P, P, P, P, P, P], I),
            "tra_execute_contract_chain": ([P, P, P, P, P, P, P, P, P], I),
            "tra_repartition": ([P, I, P, P, I, P, P, P], I),
            "tra_canonical_labels": ([ctypes.c_char_p, ctypes.c_char_p, I], I),
            "tra_d_from_operand_form": ([ctypes.c_char_p, P, I, P, I], I),
            "tra_cost": ([ctypes.c_char_p, P, P, I, P], I),
            "tra_choose": ([ctypes.c_char_p, I, P, I, P], I),
            "tra_choose_ex": ([ctypes.c_char_p, I, I, I64, P, I, P], I),
            "tra_choose_cache_stats": ([P, P], I),
            "tra_choose_cache_clear": ([], I),
            "tra_graph_plan_cap": ([ctypes.c_char_p, I, I, I64, P], I),
            "tra_predict_ns": ([P, P], I),
            "tra_predict_repartition_ns": ([P, I, I, P], I),
            "tra_graph_plan": ([ctypes.c_char_p, I, P, I, P], I),
            "tra_graph_plan_ex": ([ctypes.c_char_p, I, P, I, I, P], I),
            "tra_graph_info": ([P, P], I),
            "tra_graph_node_d": ([P, I, P, I], I),
            "tra_graph_leaf": ([P, I, ctypes.c_char_p, I, P, P], I),
            "tra_graph_node_output": ([P, I, P, P, P, P, P], I),
            "tra_graph_run_node": ([P, I, P, I, P, P, ctypes.c_size_t, P], I),
            "tra_graph_execute": ([P, P, I, P, P, ctypes.c_size_t, P], I),
            "tra_graph_destroy": ([P], I),
            "tra_status_string": ([I], ctypes.c_char_p),
            "tra_last_error": ([], ctypes.c_char_p),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(rc: int) -> int:
    if rc < 0:
        L = lib()
        raise TraError(rc, L.tra_status_string(rc).decode(), L.tra_last_error().decode())
    return rc


def _i64(v: Sequence[int]):
    return (ctypes.c_int64 * len(v))(*[int(a) for a in v])


def _i32(v: Sequence[int]):
    return (ctypes.c_int32 * len(v))(*[int(a) for a in v])


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def tra_canonical_labels(spec: str) -> str:
    buf = ctypes.create_string_buffer(64)
    _check(lib().tra_canonical_labels(spec.encode(), buf, 64))
    return buf.value.decode()


def _ordered(spec: str, v: Union[Dict[str, int], Sequence[int]]) -> List[int]:
    if isinstance(v, dict):
        return [int(v[c]) for c in tra_canonical_labels(spec)]
    return [int(a) for a in v]


def tra_d_from_operand_form(spec: str, d_ops: Sequence[int]) -> List[int]:
    n = len(tra_canonical_labels(spec))
    out = (ctypes.c_int32 * n)()
    _check(lib().tra_d_from_operand_form(spec.encode(), _i32(d_ops), len(d_ops), out, n))
    return list(out)


def tra_cost(spec: str, bounds, d) -> int:
    b, dd = _ordered(spec, bounds), _ordered(spec, d)
    c = ctypes.c_int64()
    _check(lib().tra_cost(spec.encode(), _i64(b), _i32(dd), len(b), ctypes.byref(c)))
    return c.value


class Plan:
    """Owns a tra_plan_t handle and a copy of its tra_plan_info_t."""

    def __init__(self, handle: int, spec: str, in_dtype: int, out_dtype: int):
        self.handle = handle
        self.spec = spec
        self.in_dtype = in_dtype
        self.out_dtype = out_dtype
        info = PlanInfo()
        _check(lib().tra_plan_info(handle, ctypes.byref(info)))
        self.info = info

    @property
    def kernel(self) -> str:
        return KERNELS[self.info.kernel]

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.tra_plan_destroy(self.handle)
            self.handle = None

    def workspace(self, device) -> Optional[torch.Tensor]:
        n = self.info.workspace_bytes
        return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def tra_plan(spec: str, bounds, d, join: str = "mul", agg: str = "sum", in_dtype: str = "f32",
             out_dtype: str = "f32", post_scale: float = 1.0) -> Plan:
    b, dd = _ordered(spec, bounds), _ordered(spec, d)
    h = ctypes.c_void_p()
    _check(lib().tra_plan(spec.encode(), _i64(b), _i32(dd), len(b), JOINS[join], AGGS[agg], DTYPES[in_dtype],
                          DTYPES[out_dtype], float(post_scale), ctypes.byref(h)))
    return Plan(h.value, spec, DTYPES[in_dtype], DTYPES[out_dtype])


def _dev_ptr(t: Optional[torch.Tensor], what: str, numel: int, dtype: Optional[int]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{what} has {t.numel()} elements, the plan needs {numel}")
    if dtype is not None and DTYPE_OF_TORCH.get(t.dtype) != dtype:
        raise ValueError(f"{what} has dtype {t.dtype}, the plan needs {TORCH_DTYPES[dtype]}")
    return t.data_ptr()


def tra_execute(plan: Plan, x: torch.Tensor, y: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Run the plan on device relations x (and y); returns z (allocated if None)."""
    inf = plan.info
    px = _dev_ptr(x, "x", inf.x_elems, plan.in_dtype)
    py = _dev_ptr(y, "y", inf.y_elems, plan.in_dtype) if inf.y_elems else None
    if z is None:
        z = torch.empty(inf.z_elems, dtype=TORCH_DTYPES[plan.out_dtype], device=x.device)
    pz = _dev_ptr(z, "z", inf.z_elems, plan.out_dtype)
    if workspace is None and inf.workspace_bytes:
        workspace = plan.workspace(x.device)
    pw = workspace.data_ptr() if workspace is not None else None
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().tra_execute(plan.handle, px, py, pz, pw, wb, _stream(stream)))
    return z


def tra_execute_static(plan: Plan, x: torch.Tensor, y: Optional[torch.Tensor], z: torch.Tensor,
                       stream=None) -> torch.Tensor:
    """tra_execute with the plan's scratch in the library's fixed per-device
    array (no workspace argument; nothing allocated); z is required."""
    inf = plan.info
    px = _dev_ptr(x, "x", inf.x_elems, plan.in_dtype)
    py = _dev_ptr(y, "y", inf.y_elems, plan.in_dtype) if inf.y_elems else None
    pz = _dev_ptr(z, "z", inf.z_elems, plan.out_dtype)
    _check(lib().tra_execute_static(plan.handle, px, py, pz, _stream(stream)))
    return z


def tra_probe_mfma_loop(workgroups: int, iters: int, out: torch.Tensor, distinct_operands: int = 0,
                        stream=None) -> None:
    """Matrix-core loop for the measured ceiling (see include/tra.h): 0 one
    operand pair, 1 random operands, 2 random operands on 16x16x32 products."""
    _dev_ptr(out, "out", workgroups * 256, DTYPES["f32"])
    _check(lib().tra_probe_mfma_loop(int(workgroups), int(iters), int(distinct_operands), out.data_ptr(),
                                     _stream(stream)))


def tra_static_scratch_bytes() -> int:
    return int(lib().tra_static_scratch_bytes())


def tra_execute_chain(plan_a: Plan, plan_b: Plan, xa: torch.Tensor, ya: Optional[torch.Tensor],
                      xb: torch.Tensor, z: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """z = plan_b(xb, plan_a(xa, ya)) in one pass (the intermediate is never written)."""
    ia, ib = plan_a.info, plan_b.info
    pxa = _dev_ptr(xa, "xa", ia.x_elems, plan_a.in_dtype)
    pya = _dev_ptr(ya, "ya", ia.y_elems, plan_a.in_dtype) if ia.y_elems else None
    pxb = _dev_ptr(xb, "xb", ib.x_elems, plan_b.in_dtype)
    if z is None:
        z = torch.empty(ib.z_elems, dtype=TORCH_DTYPES[plan_b.out_dtype], device=xa.device)
    pz = _dev_ptr(z, "z", ib.z_elems, plan_b.out_dtype)
    _check(lib().tra_execute_chain(plan_a.handle, plan_b.handle, pxa, pya, pxb, pz, _stream(stream)))
    return z


def tra_execute_contract_chain(plan_c: Plan, plan_a: Plan, plan_b: Plan, xc: torch.Tensor, yc: torch.Tensor,
                               ya: torch.Tensor, xb: torch.Tensor, z: Optional[torch.Tensor] = None,
                               stream=None) -> torch.Tensor:
    """z = plan_b(xb, plan_a(plan_c(xc, yc), ya)) in the product's epilogue."""
    ic, ia, ib = plan_c.info, plan_a.info, plan_b.info
    pxc = _dev_ptr(xc, "xc", ic.x_elems, plan_c.in_dtype)
    pyc = _dev_ptr(yc, "yc", ic.y_elems, plan_c.in_dtype)
    pya = _dev_ptr(ya, "ya", ia.y_elems, plan_a.in_dtype)
    pxb = _dev_ptr(xb, "xb", ib.x_elems, plan_b.in_dtype)
    if z is None:
        z = torch.empty(ib.z_elems, dtype=TORCH_DTYPES[plan_b.out_dtype], device=xc.device)
    pz = _dev_ptr(z, "z", ib.z_elems, plan_b.out_dtype)
    _check(lib().tra_execute_contract_chain(plan_c.handle, plan_a.handle, plan_b.handle, pxc, pyc, pya, pxb, pz,
                                            _stream(stream)))
    return z


def tra_repartition(src: torch.Tensor, bounds: Sequence[int], d_from: Sequence[int], d_to: Sequence[int],
                    dst: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Re-cut a device relation of the tensor `bounds` from d_from to d_to."""
    n = 1
    for b in bounds:
        n *= int(b)
    dt = DTYPE_OF_TORCH[src.dtype]
    if dst is None:
        dst = torch.empty(n, dtype=src.dtype, device=src.device)
    ps = _dev_ptr(src, "src", n, dt)
    pd = _dev_ptr(dst, "dst", n, dt)
    r = len(bounds)
    _check(lib().tra_repartition(_i64(bounds), r, _i32(d_from), _i32(d_to), dt, ps, pd, _stream(stream)))
    return dst


def to_relation(dense: torch.Tensor, d: Sequence[int], out: Optional[torch.Tensor] = None, stream=None):
    """Dense row-major tensor -> relation under d (the initial partition)."""
    return tra_repartition(dense.reshape(-1), list(dense.shape), [1] * dense.dim(), d, out, stream)


def from_relation(rel: torch.Tensor, shape: Sequence[int], d: Sequence[int], out: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """Relation under d -> dense row-major tensor of `shape`."""
    return tra_repartition(rel.reshape(-1), list(shape), d, [1] * len(shape), out, stream).reshape(shape)


CHOOSE_TIME = 1


def tra_choose(graph_desc: str, p: int, flags: int = 0, mem_cap: int = 0) -> Tuple[List[List[int]], int]:
    """Partition vectors for every node of an EinGraph (see include/tra.h);
    flags=CHOOSE_TIME selects the measured time model (cost in ns); mem_cap > 0
    bounds the workspace live at every node's step (bytes)."""
    cap = 24 * max(1, graph_desc.count("\n") + 1)
    out = (ctypes.c_int32 * cap)()
    cost = ctypes.c_int64()
    _check(lib().tra_choose_ex(graph_desc.encode(), int(p), int(flags), int(mem_cap), out, cap, ctypes.byref(cost)))
    res, pos = [], 0
    for line in graph_desc.splitlines():
        f = line.split()
        if not f or f[0].startswith("#"):
            continue
        spec = f[2]
        n = len(spec.split("->")[1]) if f[1] == "softmax" else len(tra_canonical_labels(spec))
        res.append(list(out[pos:pos + n]))
        pos += n
    return res, cost.value


class GraphInfo(ctypes.Structure):
    _fields_ = [("n_nodes", ctypes.c_int32), ("n_leaves", ctypes.c_int32), ("workspace_bytes", ctypes.c_size_t),
                ("out_elems", ctypes.c_int64), ("out_dtype", ctypes.c_int32), ("cost", ctypes.c_int64),
                ("n_repartitions", ctypes.c_int32), ("n_fused", ctypes.c_int32)]


class Graph:
    """Owns a tra_graph_t handle (see tra_graph_plan in include/tra.h)."""

    def __init__(self, handle: int):
        self.handle = handle
        info = GraphInfo()
        _check(lib().tra_graph_info(handle, ctypes.byref(info)))
        self.info = info
        self.leaves = []
        for i in range(info.n_leaves):
            name = ctypes.create_string_buffer(64)
            n, dt = ctypes.c_int64(), ctypes.c_int32()
            _check(lib().tra_graph_leaf(handle, i, name, 64, ctypes.byref(n), ctypes.byref(dt)))
            self.leaves.append((name.value.decode(), n.value, TORCH_DTYPES[dt.value]))

    def node_d(self, node: int) -> List[int]:
        buf = (ctypes.c_int32 * 32)()
        n = _check(lib().tra_graph_node_d(self.handle, node, buf, 32))
        return list(buf[:n])

    def workspace(self, device) -> Optional[torch.Tensor]:
        n = self.info.workspace_bytes
        return torch.empty(n, dtype=torch.uint8, device=device) if n else None

    def node_output(self, node: int, workspace: torch.Tensor) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
        """Views of node `node`'s output relation (and a softmax node's
        logsumexp, else None) inside `workspace`, valid after
        tra_graph_run_node of that node until a later node reuses the bytes."""
        off, n, dt = ctypes.c_size_t(), ctypes.c_int64(), ctypes.c_int32()
        lse, n_lse = ctypes.c_size_t(), ctypes.c_int64()
        _check(lib().tra_graph_node_output(self.handle, node, ctypes.byref(off), ctypes.byref(n), ctypes.byref(dt),
                                           ctypes.byref(lse), ctypes.byref(n_lse)))
        tdt = TORCH_DTYPES[dt.value]
        size = torch.empty(0, dtype=tdt).element_size()
        out = workspace[off.value:off.value + n.value * size].view(tdt)
        lse_view = workspace[lse.value:lse.value + n_lse.value * 4].view(torch.float32) if n_lse.value else None
        return out, lse_view

    def _leaf_ptrs(self, inputs: Dict[str, torch.Tensor]):
        ptrs = []
        for name, n, dt in self.leaves:
            t = inputs[name]
            ptrs.append(_dev_ptr(t, name, n, DTYPE_OF_TORCH[dt]))
        return (ctypes.c_void_p * len(ptrs))(*ptrs)

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.tra_graph_destroy(self.handle)
            self.handle = None


GRAPH_FUSE_ATTENTION = 1
GRAPH_CHOOSE_TIME = 2
GRAPH_OVERLAP_COPIES = 4


def tra_choose_cache_stats() -> Tuple[int, int]:
    """(hits, misses) of the chooser's DP memo."""
    h, m = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().tra_choose_cache_stats(ctypes.byref(h), ctypes.byref(m)))
    return h.value, m.value


def tra_choose_cache_clear() -> None:
    _check(lib().tra_choose_cache_clear())


def tra_graph_plan_cap(graph_desc: str, p: int = 256, flags: int = 0, mem_cap: int = 0) -> Graph:
    """tra_graph_plan_ex with the DP run under a workspace cap (bytes; 0 = none)."""
    h = ctypes.c_void_p()
    _check(lib().tra_graph_plan_cap(graph_desc.encode(), int(p), int(flags), int(mem_cap), ctypes.byref(h)))
    return Graph(h.value)


def tra_predict_ns(plan: Plan) -> int:
    """The time model's prediction for one tra_execute of the plan, in ns."""
    ns = ctypes.c_int64()
    _check(lib().tra_predict_ns(plan.handle, ctypes.byref(ns)))
    return ns.value


def tra_predict_repartition_ns(bounds: Sequence[int], dtype: str) -> int:
    """The time model's prediction for one tra_repartition of the tensor, in ns."""
    ns = ctypes.c_int64()
    _check(lib().tra_predict_repartition_ns(_i64(bounds), len(bounds), DTYPES[dtype], ctypes.byref(ns)))
    return ns.value


def tra_graph_plan(graph_desc: str, p: int = 256, d_all: Optional[Sequence[int]] = None) -> Graph:
    h = ctypes.c_void_p()
    if d_all is None:
        _check(lib().tra_graph_plan(graph_desc.encode(), int(p), None, 0, ctypes.byref(h)))
    else:
        _check(lib().tra_graph_plan(graph_desc.encode(), int(p), _i32(d_all), len(d_all), ctypes.byref(h)))
    return Graph(h.value)


def tra_graph_plan_ex(graph_desc: str, p: int = 256, d_all: Optional[Sequence[int]] = None,
                      flags: int = 0) -> Graph:
    """tra_graph_plan with option flags (GRAPH_FUSE_ATTENTION)."""
    h = ctypes.c_void_p()
    if d_all is None:
        _check(lib().tra_graph_plan_ex(graph_desc.encode(), int(p), None, 0, int(flags), ctypes.byref(h)))
    else:
        _check(lib().tra_graph_plan_ex(graph_desc.encode(), int(p), _i32(d_all), len(d_all), int(flags),
                                       ctypes.byref(h)))
    return Graph(h.value)


def tra_graph_execute(g: Graph, inputs: Dict[str, torch.Tensor], out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Run every node; `inputs` maps graph-input names (without '@') to dense device tensors."""
    dev = next(iter(inputs.values())).device
    if out is None:
        out = torch.empty(g.info.out_elems, dtype=TORCH_DTYPES[g.info.out_dtype], device=dev)
    po = _dev_ptr(out, "out", g.info.out_elems, g.info.out_dtype)
    if workspace is None:
        workspace = g.workspace(dev)
    pw = workspace.data_ptr() if workspace is not None else None
    wb = workspace.numel() if workspace is not None else 0
    _check(lib().tra_graph_execute(g.handle, g._leaf_ptrs(inputs), len(g.leaves), po, pw, wb, _stream(stream)))
    return out


def tra_graph_run_node(g: Graph, node: int, inputs: Dict[str, torch.Tensor], out: Optional[torch.Tensor],
                       workspace: Optional[torch.Tensor], stream=None) -> None:
    po = out.data_ptr() if out is not None else None
    pw = workspace.data_ptr() if workspace is not None else None
    wb = workspace.numel() if workspace is not None else 0
    _check(lib().tra_graph_run_node(g.handle, int(node), g._leaf_ptrs(inputs), len(g.leaves), po, pw, wb,
                                    _stream(stream)))
