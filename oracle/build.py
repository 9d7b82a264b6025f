"""Build the C part of the oracle (test infrastructure) with gcc + OpenMP."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "einsum_ref.c")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile einsum_ref.c into oracle/_build/liboracle.so and return its path."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    os.makedirs(OUT_DIR, exist_ok=True)
    tmp = LIB + ".tmp"
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11",
                    "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"], check=True)
    os.replace(tmp, LIB)
    return LIB


def build_sanitized(out_dir: str) -> str:
    """The same library built with AddressSanitizer and UndefinedBehaviorSanitizer
    (host code only), for the sanitizer run of the CPU suite."""
    os.makedirs(out_dir, exist_ok=True)
    lib = os.path.join(out_dir, "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fPIC", "-shared", "-fopenmp", "-std=c11",
                    "-Wall", "-Wextra", "-o", lib, SRC, "-lm"], check=True)
    return lib


if __name__ == "__main__":
    print(build())
