"""Build libhs.so (HIP, gfx950) in-tree with hipcc.

Flags: -O3, -ffp-contract=off (every kernel variant rounds identically), packed fp32
disabled, no fast-math (it would break -inf masking).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libhs.so")
# The benchmark's ceilings (plain streaming read, Philox word rate): a library of its own.
MICRO_LIB = os.path.join(HERE, "libhs_micro.so")
MICRO_SOURCE = os.path.join("micro", "hs_micro.hip")
SOURCES = ["hs_kernels.hip", "hs_kernels_scr.hip", "hs_kernels_pivot.hip",
           "hs_kernels_pivot_scr.hip", "hs_kernels_rows.hip", "hs_kernels_rows_scr.hip",
           "hs_filter.hip", "hs_api.hip"]
HEADERS = ["hs_device.hpp", "hs_internal.hpp", "hs_sample_kernel.hpp"]
ARCH = os.environ.get("HS_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found")
    return p


def flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
            "-fno-fast-math", "-mllvm", "-pragma-unroll-threshold=100000", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I" + os.path.join(os.path.dirname(HERE), "include"), "-I" + CSRC, "-Wall"]


def _inputs():
    srcs = [os.path.join(CSRC, s) for s in SOURCES + HEADERS + [MICRO_SOURCE]]
    srcs.append(os.path.join(os.path.dirname(HERE), "include", "hs.h"))
    return srcs


def up_to_date() -> bool:
    if not os.path.exists(LIB):
        return False
    t = os.path.getmtime(LIB)
    return all(os.path.getmtime(s) <= t for s in _inputs())


def build(force: bool = True, verbose: bool = False) -> str:
    if not force and up_to_date() and os.path.exists(MICRO_LIB):
        return LIB
    objs = []
    procs = []
    for s in SOURCES:
        obj = os.path.join(CSRC, s.replace(".hip", ".o"))
        cmd = [hipcc()] + flags() + ["-c", os.path.join(CSRC, s), "-o", obj]
        if verbose:
            print(" ".join(cmd))
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                      text=True))
        objs.append(obj)
    micro_obj = os.path.join(CSRC, "micro", "hs_micro.o")
    cmd = [hipcc()] + flags() + ["-c", os.path.join(CSRC, MICRO_SOURCE), "-o", micro_obj]
    procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                  text=True))
    for p in procs:
        out, _ = p.communicate()
        lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if p.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + "\n".join(lines))
        if verbose and lines:
            print("\n".join(lines))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    tmp = MICRO_LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, micro_obj]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, MICRO_LIB)
    os.remove(micro_obj)
    return LIB


def build_sanitized(out_dir: str, verbose: bool = False) -> str:
    """Host code only (no device code objects) under AddressSanitizer and
    UndefinedBehaviorSanitizer, into out_dir/libhs.so: the argument checks, launch planning and
    workspace layout, which run on the CPU before any device call. Kernels are not in it, so
    any call that reaches a launch fails. A process that loads it needs clang's ASan runtime
    loaded first (LD_PRELOAD); point HS_LIBRARY at the result."""
    os.makedirs(out_dir, exist_ok=True)
    san = ["--cuda-host-only", "-O1", "-g", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    objs, procs = [], []
    for s in SOURCES:
        obj = os.path.join(out_dir, s.replace(".hip", ".o"))
        cmd = [hipcc()] + flags() + san + ["-c", os.path.join(CSRC, s), "-o", obj]
        if verbose:
            print(" ".join(cmd))
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                      text=True))
        objs.append(obj)
    for p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + out)
    # Host-only objects refer to their device-code bundles by name: give each an empty
    # offload bundle (the magic string and a zero entry count), so the library loads and
    # registers no kernels.
    names = set()
    for o in objs:
        out = subprocess.run(["nm", "-u", o], check=True, capture_output=True, text=True).stdout
        names.update(l.split()[-1] for l in out.splitlines() if "__hip_fatbin_" in l)
    stub = os.path.join(out_dir, "empty_bundles.c")
    with open(stub, "w") as f:
        for n in sorted(names):
            f.write('__attribute__((aligned(8))) const char %s[32] = '
                    '"__CLANG_OFFLOAD_BUNDLE__";\n' % n)
    stub_obj = stub[:-2] + ".o"
    subprocess.run(["gcc", "-c", "-fPIC", "-o", stub_obj, stub], check=True)
    lib = os.path.join(out_dir, "libhs.so")
    subprocess.run([hipcc(), "--cuda-host-only", "-shared", "-fPIC", "-o", lib] + objs +
                   [stub_obj], check=True, capture_output=not verbose)
    return lib


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(sys.argv[sys.argv.index("--sanitize") + 1], "-v" in sys.argv))
    else:
        print(build(force=True, verbose="-v" in sys.argv))
