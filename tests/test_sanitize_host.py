"""The host-side C and C++ under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's host code (argument checks, row tables, the swap planner, the
ring's bookkeeping, the acknowledgement log, the Appendix E predictor, the
paged and partition checks) and the oracle are rebuilt with
``-fsanitize=address,undefined`` on the host side only (no GPU code is
instrumented), and every CPU-tier test runs again in a child process that
loads those builds, with the sanitizer runtime preloaded and any report made
fatal.  The GPU tier is not run this way: sanitized GPU code is not available
on the MI355X machines.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# sanitizer options of the host pass only; each -fsanitize= right after its -Xarch_host
HOST_SANITIZE = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                 "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -shared-libsan").split()


def asan_runtime():
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.timeout(900)
def test_cpu_tier_under_asan_and_ubsan(tmp_path):
    if os.environ.get("KVSTREAM_LIB") or os.environ.get("KV_ORACLE_LIB"):
        pytest.skip("already running against another build")
    rt = asan_runtime()
    if rt is None or shutil.which(HIPCC) is None:
        pytest.skip("no clang sanitizer runtime or hipcc here")
    csrc = os.path.join(ROOT, "kv_cache_streaming_amd", "csrc")
    srcs = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith(".hip"))
    lib = str(tmp_path / "libkvstream.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-std=c++17", "-fPIC", "-shared", *HOST_SANITIZE,
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-I", os.path.join(ROOT, "include"), "-I", csrc, "-o", lib, *srcs,
                    "-L/opt/rocm/lib", "-lhsa-runtime64", "-pthread"],
                   check=True, capture_output=True)
    orc = str(tmp_path / "liboracle.so")
    subprocess.run([CLANG, "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC",
                    "-shared", "-Wall", "-Werror", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-shared-libsan", "-o", orc,
                    os.path.join(ROOT, "oracle", "oracle.c")], check=True, capture_output=True)
    env = dict(os.environ, KVSTREAM_LIB=lib, KV_ORACLE_LIB=orc, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the child loads the sanitized builds (not the in-tree ones)
    probe = ("import ctypes, kv_cache_streaming_amd as kv, oracle; "
             "l = oracle.load(); "
             "assert kv.LIB_PATH == %r and hasattr(ctypes.CDLL(kv.LIB_PATH), '__asan_init'); "
             "assert hasattr(l, '__asan_init')") % lib
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "tests", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=800)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
