"""The boundary is a C ABI: a C99 program (tests/c_abi_check.c) includes
include/kvstream.h, links the library and gets the host-only answers from C."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def program(tmp_path_factory):
    from libload import build_module
    b = build_module()
    if not os.path.exists(b.LIB):
        b.build()
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp("cabi") / "c_abi_check")
    libdir = os.path.dirname(b.LIB)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror=implicit-function-declaration",
                    "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", "-o", exe, os.path.join(HERE, "c_abi_check.c"),
                    "-L", libdir, "-lkvstream", f"-Wl,-rpath,{libdir}"], check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    return dict(line.split(" ", 1) for line in out.strip().splitlines())


def test_layout_and_sizes_from_c(program):
    assert program["layout_init"] == "0"
    assert int(program["k_bytes"]) == 48 * 8 * 25 * 64 * 1024 * 2
    # 2 x B x S x H x D x P x N with B=8, S=1000, H=25, D=64, P=2, N=48
    assert int(program["pack_bytes"]) == 2 * 8 * 1000 * 25 * 64 * 2 * 48
    assert program["pack_bytes_uniform"] == program["pack_bytes"]
    assert program["bad_layout"] == "-1" and program["error_message_set"] == "1"


def test_paged_partition_schedule_and_acks_from_c(program):
    assert program["paged_init"] == "0"
    assert int(program["paged_pack_bytes"]) == 2 * 8 * 1000 * 25 * 64 * 2 * 48
    # layers 8..15 x heads 36..71 x all 8 rows of the OPT-66B slice
    assert int(program["stream_bytes"]) == 2 * 8 * 36 * 128 * 2 * sum(range(300, 308))
    assert program["swap_pays"] == "1" and program["swap_pays_sides"] == "10.0 8.0"
    # microbatch 1 has worker 1's ack missing: the restart is microbatch 1, step 0
    assert program["restart_point"] == "1 0"
    assert program["version"] == "1"
    # nothing timed yet: an all-zero window; a NULL output is KV_EINVAL
    assert program["profile_window"] == "0 0.0 0 -1"
