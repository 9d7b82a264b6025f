"""Build libtra.so (HIP kernels for gfx950 + the C-ABI host code) in-tree.

Sources: csrc/*.hip are compiled by hipcc for gfx950, csrc/*.cpp (host-only
planner and chooser) by g++; everything is linked into
tensor_relational_algebra_amd/_build/libtra.so.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "_build")
LIB = os.path.join(OUT, "libtra.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_FLAGS = ["-O3", f"--offload-arch={ARCH}", "-fPIC", "-std=c++17", "-Wall",
             # packed fp32 VALU ops are kept out of every kernel
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", INCLUDE, "-I", CSRC]
CXX_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    if src.endswith(".hip"):
        cmd = [HIPCC] + HIP_FLAGS + ["-c", src, "-o", obj]
    else:
        cmd = ["g++"] + CXX_FLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OUT, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(LIB)
    return LIB


SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined"]


def build_sanitized(out_dir: str) -> str:
    """libtra with its host code (csrc/*.cpp: parser, planner, chooser, graph
    executor) built by g++ under AddressSanitizer and UndefinedBehaviorSanitizer,
    linked with the device objects of the last build() (built first if absent).
    Only the host code is instrumented; the kernels are the normal ones."""
    if not os.path.exists(LIB):
        build()
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.cpp"))):
        obj = os.path.join(out_dir, os.path.basename(src) + ".san.o")
        subprocess.run(["g++"] + SAN_FLAGS + ["-fPIC", "-std=c++17", "-Wall", "-Wextra", "-I", INCLUDE,
                                              "-I", CSRC, "-c", src, "-o", obj], check=True)
        objs.append(obj)
    dev_objs = sorted(glob.glob(os.path.join(OUT, "*.hip.o")))
    lib = os.path.join(out_dir, "libtra_san.so")
    subprocess.run(["g++", "-shared", "-fsanitize=address,undefined", "-o", lib] + objs + dev_objs +
                   ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
