"""bench.py's output line on the GPU: one JSON line with every field the
benchmark contract names, the roofline object for the dominant kernel and
the oracle's CPU baseline, and internally consistent figures."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(600)
def test_headline_line():
    print("[gpu-case] bench.py --steps 2 --warmup 1 --no-detail", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2",
                        "--warmup", "1", "--no-detail", "--cpu-baseline-seconds", "2"],
                       capture_output=True, text=True, timeout=540, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["vs_baseline"] is None
    assert d["config"]["workload"] == "gqa-100k"
    # value: the host-link bytes of a step over its time
    link = d["detail"]["link_bytes_per_step"]
    assert abs(d["value"] - link / (d["ms_per_step"] / 1000) / 1e9) <= 0.01 * d["value"]
    rf = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in rf, key
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    k = d["detail"]["kernels"][rf["kernel"]]
    assert abs(rf["achieved"] - k["algorithmic_bytes_per_launch"] / (k["avg_us"] * 1e3)) \
        <= 0.01 * rf["achieved"]
    assert 0 < rf["frac"] < 1
    cpu = d["cpu_baseline"]
    for key in ("value", "unit", "cores", "kind", "sample"):
        assert key in cpu, key
    assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0
    parts = d["metric_parts"]
    assert parts["swap_host_link_GBps"] == d["value"] and parts["pack_unpack_GBps"] == rf["achieved"]
    assert abs(parts["pack_unpack_payload_GBps"] - rf["achieved"] / 2) <= 0.1
    if rf["traffic"]:
        assert abs(parts["pack_unpack_counter_traffic_GBps"] -
                   rf["traffic"] / (rf["avg_us"] * 1e3)) <= 0.01 * rf["achieved"]
    # the pages' context figures beside this link's measured rate
    ctx = d["context"]
    assert ctx["pages_opt175b_2048_token_kv_ms_estimate_8_links"] == 17.6
    assert ctx["same_9_GiB_at_this_link_GBps"] == d["detail"]["link_directions"]["d2h"]["GBps"]
    assert abs(ctx["same_9_GiB_ms_one_link"] - 9 * 2 ** 30 / (ctx["same_9_GiB_at_this_link_GBps"]
                                                              * 1e9) * 1000) <= 0.1
