"""Host-side logic of bench.py: the one-GPU refusal and the matching of the
committed counter summaries to the kernels they were taken on."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    sys.path.insert(0, ROOT)
    import bench as b
    return b


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout


def _summary(tmp_path, kernel, digest, algorithmic, traffic):
    p = tmp_path / f"traffic_{kernel}_w.txt"
    p.write_text("# header: ignored\n"
                 "kernel                   n    fetch_KiB    write_KiB   scaled_bytes\n"
                 f"{kernel}  3  1.0  2.0  {traffic}\n\n"
                 f"kernel: {kernel}\nkernels_sha256_16: {digest}\n"
                 f"traffic_bytes_per_launch: {traffic}\n"
                 f"algorithmic_bytes_per_launch: {algorithmic}\n")
    return str(p)


def test_counter_summary_matching(bench, tmp_path, monkeypatch):
    src = os.path.join(ROOT, "kv_cache_streaming_amd", "csrc", "kernels.hip")
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    path = _summary(tmp_path, "pack_tiles", digest, 1000, 1234)
    monkeypatch.setattr(bench, "counters_file", lambda w, k: path)
    assert bench.read_counters("w", "pack_tiles", 1000) == 1234.0
    # another launch size, another kernel or another kernel source: no figure
    assert bench.read_counters("w", "pack_tiles", 1001) is None
    assert bench.read_counters("w", "unpack_tiles", 1000) is None
    stale = _summary(tmp_path, "pack_tiles", "0" * 16, 1000, 1234)
    monkeypatch.setattr(bench, "counters_file", lambda w, k: stale)
    assert bench.read_counters("w", "pack_tiles", 1000) is None
    monkeypatch.setattr(bench, "counters_file", lambda w, k: str(tmp_path / "absent.txt"))
    assert bench.read_counters("w", "pack_tiles", 1000) is None


def test_committed_summaries_are_well_formed(bench):
    """Every committed summary names its kernel, carries a source digest and a
    traffic figure no smaller than the algorithmic bytes it was scaled to."""
    files = [f for f in os.listdir(os.path.join(ROOT, "profiles")) if f.startswith("traffic_")]
    assert files
    for f in files:
        fields = {}
        for line in open(os.path.join(ROOT, "profiles", f)):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
        kernel = f[len("traffic_"):].rsplit("_", 1)[0]
        assert fields["kernel"] == kernel, f
        assert len(fields["kernels_sha256_16"]) == 16, f
        traffic = float(fields["traffic_bytes_per_launch"])
        algo = int(fields["algorithmic_bytes_per_launch"])
        assert 0.99 * algo <= traffic <= 1.5 * algo, f
