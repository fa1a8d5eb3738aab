"""The boundary on the GPU from C: a C99 program (tests/c_abi_device.c) that
allocates device and pinned host memory with the HIP runtime's C API and
drives the library through include/kvstream.h alone -- a ragged multi-token
pack, a move of the packed block and its unpack, a staged swap-out, and a
staging ring's push, flush and restore.  Every result it writes must equal
the oracle's on the caches the program itself generated."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from gpu_util import note

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
DIMS = (3, 3, 2, 64, 100)          # L, B, H, D, Smax as in c_abi_device.c
START, COUNT = [0, 10, 99], [100, 45, 1]
STEPS = 5


@pytest.fixture(scope="module")
def outputs(tmp_path_factory):
    from libload import build_module
    b = build_module()
    assert os.path.exists(b.LIB), "build the library first"
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    d = tmp_path_factory.mktemp("cabi_dev")
    exe = str(d / "c_abi_device")
    libdir = os.path.dirname(b.LIB)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror=implicit-function-declaration",
                    "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", "-o", exe, os.path.join(HERE, "c_abi_device.c"),
                    "-L", libdir, "-lkvstream", "-L/opt/rocm/lib", "-lamdhip64",
                    f"-Wl,-rpath,{libdir}", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    note(f"c_abi_device dims={DIMS} start={START} count={COUNT} ring steps={STEPS}")
    r = subprocess.run([exe, str(d)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert r.stdout.strip().endswith("done"), r.stdout
    calls = dict(line.split(" ", 1) for line in r.stdout.splitlines()
                 if line.startswith("kv_"))
    files = {f[:-4]: np.fromfile(str(d / f), dtype=np.uint16)
             for f in os.listdir(d) if f.endswith(".bin")}
    return calls, files


def test_every_call_succeeds(outputs):
    calls, _ = outputs
    for name in ("kv_layout_init", "kv_pack_tokens", "kv_copy_packed", "kv_unpack_tokens",
                 "kv_swap_create",
                 "kv_swap_out", "kv_swap_destroy", "kv_ring_create", "kv_ring_push",
                 "kv_ring_flush", "kv_ring_restore", "kv_ring_destroy"):
        assert calls.get(name) == "0", (name, calls.get(name))


def test_pack_unpack_from_c(outputs):
    _, f = outputs
    L, B, H, D, S = DIMS
    K, V = f["k"].reshape(L, B, H, D // 8, S, 8), f["v"].reshape(L, B, H, S, D)
    want = oracle.pack(DIMS, K, V, 0, L, START, COUNT)
    assert np.array_equal(f["pack"], want)
    assert np.array_equal(f["copy"], want)          # kv_copy_packed of the packed block
    zk, zv = np.zeros_like(K), np.zeros_like(V)
    oracle.unpack(DIMS, zk, zv, 0, L, START, COUNT, want)
    assert np.array_equal(f["unpack_k"], zk.ravel())
    assert np.array_equal(f["unpack_v"], zv.ravel())


def test_swap_out_from_c(outputs):
    _, f = outputs
    L, B, H, D, S = DIMS
    K, V = f["k"].reshape(L, B, H, D // 8, S, 8), f["v"].reshape(L, B, H, S, D)
    assert np.array_equal(f["swap"], oracle.swap_out(DIMS, K, V, 0, L, START, COUNT))


def test_ring_from_c(outputs):
    _, f = outputs
    L, B, H, D, S = DIMS
    K, V = f["k"].reshape(L, B, H, D // 8, S, 8), f["v"].reshape(L, B, H, S, D)
    pos = f["ring_pos"].view(np.int32).reshape(STEPS, B)
    slots = [oracle.pack(DIMS, K, V, 0, L, [int(p) for p in pos[j]], [1] * B)
             for j in range(STEPS)]
    host = oracle.ring_host(slots)
    assert np.array_equal(f["ring"], host)
    zk, zv = np.zeros_like(K), np.zeros_like(V)
    oracle.ring_restore(DIMS, zk, zv, pos, host)
    assert np.array_equal(f["restore_k"], zk.ravel())
    assert np.array_equal(f["restore_v"], zv.ravel())
