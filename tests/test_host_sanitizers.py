"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer, without a GPU.

The oracle and the library's host side (the C-ABI's argument checks, the launch planner, the
workspace layout) are rebuilt with both sanitizers: the library host-only, with no device
code. The CPU test suite then runs against those builds in a child process with clang's ASan
runtime preloaded; any out-of-bounds access, use after free or undefined behaviour in that code
ends the child with an error report."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASAN_RT = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))

pytestmark = pytest.mark.skipif(os.environ.get("HS_SANITIZED_RUN") == "1",
                                reason="already inside the sanitized run")


def _undefined(lib):
    return subprocess.run(["nm", "-u", lib], check=True, capture_output=True, text=True).stdout


def test_cpu_suite_under_sanitizers(tmp_path):
    if not ASAN_RT:
        pytest.skip("clang's ASan runtime is not installed")
    sys.path.insert(0, ROOT)
    from logit_transform_amd import build as lib_build
    from oracle import build as oracle_build
    lib = lib_build.build_sanitized(str(tmp_path))
    olib = oracle_build.build_sanitized(str(tmp_path))
    for f in (lib, olib):
        u = _undefined(f)
        assert "__asan_report_load" in u and "__ubsan_handle_" in u, "%s is not instrumented" % f
    # reports go to files (pytest's output capture would swallow them when the child dies)
    logs = str(tmp_path / "report")
    env = dict(os.environ, HS_LIBRARY=lib, HS_ORACLE_LIBRARY=olib, HS_SANITIZED_RUN="1",
               LD_PRELOAD=ASAN_RT[-1],
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:halt_on_error=1:"
                            "log_path=" + logs,
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:log_path=" + logs)

    def reports():
        text = ""
        for f in sorted(glob.glob(logs + "*")):
            with open(f) as fh:
                text += fh.read()[-4000:]
        return text

    # the child runs with the sanitizer runtime and loads the two sanitized builds
    probe = ("import ctypes, logit_transform_amd as hs\n"
             "from oracle import oracle as O\n"
             "ctypes.CDLL(None).__asan_init\n"
             "print(hs.load()._name)\n"
             "print(O.lib()._name)\n")
    r = subprocess.run([sys.executable, "-c", probe], env=env, cwd=ROOT, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:] + reports()
    assert r.stdout.split() == [lib, olib], r.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "tests", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider"], env=env, cwd=ROOT, capture_output=True,
                       text=True, timeout=1200)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:] + reports()
    assert " passed" in r.stdout and not reports()
