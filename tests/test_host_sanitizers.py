"""The library's host-side code (argument validation, layout arithmetic, the host pack and
unpack helpers, the chain's arena layout) built with AddressSanitizer and
UndefinedBehaviorSanitizer, and the CPU ABI tests (tests/test_abi_cpu.py) run against that
build in a child process (CPU only; no device code is built or run).

The build compiles every library source with the sanitizers on its host side only (the
device code is built as usual and never launched here); the child process preloads the sanitizer runtime and loads the sanitized
library in place of the in-tree one (FRT_LIBRARY).  Any sanitizer report fails the run
(no recovery), and its text is checked for reports as well.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "host_sanitized")
HIPCC = "/opt/rocm/bin/hipcc"


def _runtime():
    libs = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return libs[-1] if libs else None


SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _build():
    """The library with the sanitizers on its host side (device code built as usual, never
    run here), objects compiled in parallel as the in-tree build does."""
    import concurrent.futures
    from gemm_chains_amd import build as b
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, "libfrt_host_sanitized.so")

    def compile_one(src):
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC] + b.FLAGS + ["-g"] + SAN_FLAGS + ["-c", os.path.join(b.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        return obj
    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, b.SOURCES))
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + SAN_FLAGS + ["-o", lib] + objs,
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return lib


@pytest.mark.skipif(not (os.path.exists(HIPCC) and _runtime()), reason="needs hipcc and the clang ASan runtime")
def test_abi_tests_pass_under_address_and_ub_sanitizers():
    lib = _build()
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle_" in syms, "the build is not instrumented"
    env = dict(os.environ, LD_PRELOAD=_runtime(), FRT_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in out
