"""Static check of the gfx950 code the matrix-core kernels compile to.

The matrix-core and fused-attention kernels issue their LDS fragment reads as
raw ``ds_read`` instructions and wait for them with an explicit
``s_waitcnt lgkmcnt(n)``: the compiler does not know those registers are
still being filled.  If register allocation ever copies or spills such a
register before the wait (a phi across a branch, a loop back-edge, a tuple
that has to be re-packed), the copy takes stale data and the results are
silently wrong.  This test compiles the kernels to AMD assembly on the host
and checks every kernel for an instruction that reads, or overwrites, a VGPR
whose LDS read is still in flight.

LDS operations retire in issue order, so ``s_waitcnt lgkmcnt(n)`` completes all
but the newest n.  The scan follows straight-line order (a label keeps the state
of the fall-through path) and counts every other LDS operation (writes too) and
scalar memory loads as in-flight entries.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

from tensor_relational_algebra_amd import build as tra_build

HIPCC = tra_build.HIPCC
KERNEL_SOURCES = ["k_mfma.hip", "k_mfma4k.hip", "k_attention.hip"]

_LDS_READ = re.compile(r"(ds_read\S*|ds_load\S*)\s+(?:v\[(\d+):(\d+)\]|v(\d+))")
_WAIT = re.compile(r"s_waitcnt.*lgkmcnt\((\d+)\)")
_STORE_PREFIXES = ("global_store", "buffer_store", "scratch_store", "ds_write", "ds_store", "flat_store")


def _regs(operand: str) -> set[int]:
    out: set[int] = set()
    for a, b in re.findall(r"\bv\[(\d+):(\d+)\]", operand):
        out |= set(range(int(a), int(b) + 1))
    for a in re.findall(r"\bv(\d+)\b", operand):
        out.add(int(a))
    return out


def scan_function(body: str) -> list[str]:
    """Instructions of one kernel that touch a VGPR whose LDS read has not been waited for."""
    queue: list[set[int]] = []
    bad: list[str] = []
    for raw in body.split("\n"):
        line = raw.split(";")[0].strip()
        if not line or line.startswith(".") or line.endswith(":"):
            continue
        op = line.split()[0]
        pending = set().union(*queue) if queue else set()
        parts = line.split(None, 1)
        ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
        m = _LDS_READ.match(line)
        if m:
            if any(_regs(o) & pending for o in ops):        # its address, or its destination
                bad.append(line)
            queue.append(set(range(int(m.group(2)), int(m.group(3)) + 1)) if m.group(2) else {int(m.group(4))})
            continue
        if op.startswith("ds_"):
            # any other LDS operation (a write, an atomic) counts against lgkmcnt
            # and reads its register operands when issued
            if any(_regs(o) & pending for o in ops):
                bad.append(line)
            queue.append(set())
            continue
        if op.startswith(("s_load", "s_buffer_load")):
            queue.append(set())
            continue
        w = _WAIT.match(line)
        if w:
            n = int(w.group(1))
            queue = queue[len(queue) - n:] if n < len(queue) else queue
            continue
        if op.startswith("s_") or op.startswith("global_load_lds") or not pending:
            continue
        if op.startswith(_STORE_PREFIXES):
            srcs, dst = ops, []
        else:
            srcs, dst = ops[1:], ops[:1]
        if any(_regs(o) & pending for o in srcs) or any(_regs(o) & pending for o in dst):
            bad.append(line)
    return bad


_MFMA = re.compile(r"(v_mfma\S*)\s+(a\[\d+:\d+\]|v\[\d+:\d+\]),\s*(v\[\d+:\d+\]),\s*(v\[\d+:\d+\])")


def mfma_operand_hazards(body: str, need: int = 2) -> list[str]:
    """Matrix-core products whose A or B operand register was written by a
    vector-ALU instruction fewer than `need` wait states before.  Products
    issued from inline asm are invisible to the compiler's hazard handling;
    their operands must come from memory reads (waited for by s_waitcnt), or
    be separated from a vector-ALU write by wait states."""
    since: dict[int, int] = {}   # register -> wait states since its last vector-ALU write
    bad: list[str] = []
    for raw in body.split("\n"):
        line = raw.split(";")[0].strip()
        if not line or line.startswith(".") or line.endswith(":"):
            continue
        op = line.split()[0]
        m = _MFMA.match(line)
        if m:
            if any(since.get(r, need) < need for r in _regs(m.group(3)) | _regs(m.group(4))):
                bad.append(line)
        elif op.startswith("v_"):
            parts = line.split(None, 1)
            dst = parts[1].split(",")[0] if len(parts) > 1 else ""
            for r in _regs(dst):
                since[r] = -1
        n = 1
        if op == "s_nop":
            n = int(line.split()[1], 0) + 1
        for r in since:
            since[r] += n
    return bad


def scan_assembly(text: str) -> dict[str, list[str]]:
    pieces = re.split(r"\n(_Z\S+):[^\n]*\n", text)
    out = {}
    for k in range(1, len(pieces), 2):
        out[pieces[k]] = scan_function(pieces[k + 1].split(".Lfunc_end")[0])
    return out


def test_scanner_flags_a_copy_of_an_in_flight_register():
    body = """
        ds_read_b128 v[10:13], v2
        ds_read_b128 v[14:17], v3
        s_waitcnt lgkmcnt(1)
        v_mov_b32_e32 v40, v10
        v_mov_b32_e32 v41, v14
        s_waitcnt lgkmcnt(0)
        v_mov_b32_e32 v42, v15
        ds_read_b64_tr_b16 v[20:21], v4
        v_add_u32_e32 v20, 1, v5
    """
    bad = scan_function(body)
    assert bad == ["v_mov_b32_e32 v41, v14", "v_add_u32_e32 v20, 1, v5"]
    # LDS writes count against lgkmcnt too: a wait for "14 outstanding" after a
    # read and 14 younger writes covers the read; an LDS write of a register whose
    # read is in flight is caught
    body = "ds_read_b128 v[76:79], v67\n" + "ds_write_b32 v70, v68\n" * 14 + \
        "s_waitcnt lgkmcnt(14)\nglobal_store_dwordx4 v[72:73], v[76:79], off\n" + \
        "ds_read_b32 v90, v1\nds_write_b32 v2, v90\n"
    assert scan_function(body) == ["ds_write_b32 v2, v90"]


def test_operand_hazard_scanner():
    body = """
        ds_read_b128 v[10:13], v2
        s_waitcnt lgkmcnt(0)
        v_mfma_f32_16x16x32_bf16 a[0:3], v[10:13], v[10:13], a[0:3]
        v_mov_b32_e32 v11, v5
        v_mfma_f32_16x16x32_bf16 a[4:7], v[10:13], v[20:23], a[4:7]
        v_mov_b32_e32 v21, v5
        s_nop 1
        v_mfma_f32_16x16x32_bf16 a[8:11], v[12:15], v[20:23], a[8:11]
    """
    assert mfma_operand_hazards(body) == ["v_mfma_f32_16x16x32_bf16 a[4:7], v[10:13], v[20:23], a[4:7]"]


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("source", KERNEL_SOURCES)
def test_no_register_is_used_before_its_lds_read_lands(source, tmp_path):
    src = os.path.join(tra_build.CSRC, source)
    out = tmp_path / (source + ".s")
    cmd = [HIPCC] + [f for f in tra_build.HIP_FLAGS if f not in ("-fPIC", "-Wall")] + \
        ["--cuda-device-only", "-S", src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    text = out.read_text()
    found = scan_assembly(text)
    assert found, "no kernels found in the assembly"
    offenders = {name: lines[:3] for name, lines in found.items() if lines}
    assert not offenders, offenders
    # products issued from inline asm: no operand fresh from a vector-ALU write
    pieces = re.split(r"\n(_Z\S+):[^\n]*\n", text)
    hazards = {pieces[k]: mfma_operand_hazards(pieces[k + 1].split(".Lfunc_end")[0])[:3]
               for k in range(1, len(pieces), 2)}
    hazards = {k: v for k, v in hazards.items() if v}
    assert not hazards, hazards
