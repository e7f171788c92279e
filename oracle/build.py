"""Build the double-precision CPU oracle (test infrastructure only).

gcc -O2, OpenMP, no fast-math (fast-math would break -inf masking and the Gumbel tails).
build_sanitized: the same source under AddressSanitizer and UndefinedBehaviorSanitizer.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "hs_oracle.c")
LIB = os.path.join(HERE, "libhs_oracle.so")
CLANG = "/opt/rocm/llvm/bin/clang"


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
           "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def build_sanitized(out_dir: str) -> str:
    """The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer into out_dir
    (clang, serial: the OpenMP pragmas are ignored). A process that loads it needs clang's ASan
    runtime loaded first (LD_PRELOAD); point HS_ORACLE_LIBRARY at the result."""
    os.makedirs(out_dir, exist_ok=True)
    lib = os.path.join(out_dir, "libhs_oracle.so")
    cmd = [CLANG, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
           "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-Wall", "-Wno-unknown-pragmas", "-o", lib, SRC,
           "-lm"]
    subprocess.run(cmd, check=True)
    return lib


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(sys.argv[sys.argv.index("--sanitize") + 1]))
    else:
        print(build(force="--lazy" not in sys.argv))
