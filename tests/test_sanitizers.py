"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library's host code (the einsum-spec and graph-description parsers, the
planner, the chooser and the graph executor's planning) and the oracle's C
code are rebuilt with -fsanitize=address,undefined, and the CPU tests that
drive them run again in a child process against those builds.  Any
out-of-bounds access, use after free or undefined behaviour aborts the child
and fails this test.  No kernel is launched.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUITES = ["tests/test_abi_cpu.py", "tests/test_chooser_time.py", "tests/test_graph_memory.py",
          "tests/test_oracle_definition.py", "tests/test_oracle_tra.py", "tests/test_oracle_chooser.py"]


def _runtime(name: str) -> str:
    return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()


def test_cpu_suite_under_address_and_undefined_sanitizers(tmp_path):
    from oracle import build as oracle_build
    from tensor_relational_algebra_amd import build as tra_build
    asan = _runtime("libasan.so")
    if not os.path.isabs(asan):
        pytest.fail("gcc has no AddressSanitizer runtime")
    lib = tra_build.build_sanitized(str(tmp_path))
    olib = oracle_build.build_sanitized(str(tmp_path))
    env = dict(os.environ)
    env.update({
        "TRA_LIBRARY": lib,
        "TRA_ORACLE_LIBRARY": olib,
        # python itself is not instrumented: the runtime must be loaded first
        "LD_PRELOAD": asan,
        # the interpreter's own allocations are not ours to audit
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "OMP_NUM_THREADS": "2",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider"] +
                       SUITES, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, f"sanitized CPU suite failed (status {r.returncode}):\n{tail}"
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
