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


def test_oracle_pieces_partition_the_selection(bench):
    """The all-cores CPU figure cuts each call into pieces: every selected
    (row, token) lands in exactly one piece, and nothing else does."""
    import numpy as np
    rng = np.random.default_rng(5)
    for B, threads in ((1, 16), (4, 16), (8, 3), (5, 1)):
        start = rng.integers(0, 50, B)
        count = rng.integers(0, 40, B)
        count[0] = 0                              # an empty row
        seen = {}
        for st, ct in bench.oracle_pieces(B, start, count, threads):
            live = [b for b in range(B) if ct[b] > 0]
            assert len(live) == 1                 # one row per piece
            b = live[0]
            for s in range(st[b], st[b] + ct[b]):
                assert (b, s) not in seen
                seen[(b, s)] = True
        want = {(b, int(s)) for b in range(B) for s in range(start[b], start[b] + count[b])}
        assert set(seen) == want


def test_all_cores_leg_moves_the_whole_call(bench):
    """Run through the threaded leg, the oracle's pieces leave the destination
    cache exactly as one whole-call pack + unpack does, and count its bytes."""
    import numpy as np
    import oracle
    dims = (3, 4, 2, 16, 40)
    L, B, H, D, S = dims
    n = L * B * H * D * S
    rng = np.random.default_rng(11)
    src = [rng.integers(0, 1 << 16, n, dtype=np.uint16) for _ in range(2)]
    start, count = [3, 0, 10, 1], [20, 0, 30, 39]
    want = [np.zeros(n, np.uint16), np.zeros(n, np.uint16)]
    oracle.unpack(dims, want[0], want[1], 1, 2, start, count,
                  oracle.pack(dims, src[0], src[1], 1, 2, start, count))
    got = [np.zeros(n, np.uint16), np.zeros(n, np.uint16)]
    r = bench.cpu_all_cores(oracle, dims, [("pair", src, got, 1, 2, start, count)], 60.0, 1)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
    payload = 2 * 2 * H * D * sum(count) * 2      # K and V, 2 layers, 2 bytes each
    assert r["cores"] >= 1 and r["value"] > 0
    assert f"{2 * payload / 1e9:.3f} GB" in r["sample"]


def test_all_cores_leg_keeps_order_where_calls_meet(bench, monkeypatch):
    """Calls that write the same elements stay in order (the later one wins,
    as run one after another); calls on disjoint elements share a group."""
    import numpy as np
    import oracle
    # a pool of 8 threads whatever this host has: group sizes depend on it
    monkeypatch.setattr(bench.os, "sched_getaffinity", lambda pid: set(range(8)))
    dims = (2, 3, 2, 8, 32)
    L, B, H, D, S = dims
    n = L * B * H * D * S
    rng = np.random.default_rng(3)
    s1 = [rng.integers(0, 1 << 16, n, dtype=np.uint16) for _ in range(2)]
    s2 = [rng.integers(0, 1 << 16, n, dtype=np.uint16) for _ in range(2)]
    start, count = [0, 4, 8], [16, 16, 16]
    pairs = [("first", s1, None, 0, 2, start, count), ("second", s2, None, 0, 2, start, count)]
    # eight single-token calls at distinct positions: disjoint, so one group
    steps = [(f"step{j}", s1, None, 0, 2, [20 + j] * B, [1] * B) for j in range(8)]
    got = [np.zeros(n, np.uint16), np.zeros(n, np.uint16)]
    want = [np.zeros(n, np.uint16), np.zeros(n, np.uint16)]
    for name, src, _, l0, nl, st, ct in pairs + steps:
        oracle.unpack(dims, want[0], want[1], l0, nl, st, ct,
                      oracle.pack(dims, src[0], src[1], l0, nl, st, ct))
    run = [(name, src, got, l0, nl, st, ct) for name, src, _, l0, nl, st, ct in pairs + steps]
    r = bench.cpu_all_cores(oracle, dims, run, 60.0, 1)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
    assert "(1 pass(es), 3 groups)" in r["sample"]


def test_committed_counters_match_the_headline_kernels(bench):
    """The committed counter summary of the headline workload's dominant
    kernel was taken on the current kernel source, so the bench line carries
    HBM traffic (not null)."""
    path = bench.counters_file("gqa-100k", "pack_tiles")
    fields = dict(line.split(":", 1) for line in open(path) if ":" in line and
                  not line.startswith("#"))
    alg = int(fields["algorithmic_bytes_per_launch"])
    assert bench.read_counters("gqa-100k", "pack_tiles", alg) is not None


def test_long_context_defaults(bench):
    """The 100K-context step's link configuration: prompt on DMA engine 0
    through two handles, row swap on the link-copy kernel (16 workgroups)
    through whole-image banks, the prompt's copies after the row's."""
    w = "gqa-100k"
    assert bench.DEFAULT_TRANSPORT[w] == "engine"
    assert bench.DEFAULT_ROW_TRANSPORT[w] == "auto"
    assert bench.DEFAULT_PROMPT_ENGINES[w] == "0,0"
    assert bench.DEFAULT_ROW_LINK_BLOCKS[w] == 16
    assert bench.DEFAULT_ROW_BANK_MIB[w] == 0 and bench.DEFAULT_ROW_FIRST[w] is True
    args = sys.argv
    try:
        sys.argv = ["bench.py"]
        a = bench.parse_args()
    finally:
        sys.argv = args
    assert a.workload == w and a.gpus == 1


@pytest.mark.parametrize("workload", ["gpt2-small-tiny", "opt-66b-16l"])
def test_naive_copies_land_where_the_pack_puts_them(bench, monkeypatch, workload):
    """The naive side of buffered_vs_naive on the CPU: the runtime's copies
    become memmoves between host tensors and the library's pack becomes the
    oracle's, so every per-piece and per-head copy must stay inside its
    buffers and the three host images must equal the oracle's pack of the
    step (OPT-66B: the full-size shape, 156,672 copies)."""
    import ctypes
    import types

    import numpy as np
    import torch

    import oracle
    import synth
    w = synth.WORKLOADS[workload]
    L, B, H, D, S = w.dims
    rng = np.random.default_rng(5)
    n = L * B * H * D * S
    K = rng.integers(0, 1 << 16, size=n, dtype=np.uint16)
    V = rng.integers(0, 1 << 16, size=n, dtype=np.uint16)
    k, v = torch.from_numpy(K.view(np.int16)), torch.from_numpy(V.view(np.int16))
    live = [k, v]

    def inside(p, nb):
        return any(t.data_ptr() <= p and p + nb <= t.data_ptr() + t.numel() * 2 for t in live)

    def copy1(dst, src, nb, kind, s):
        assert kind == 2 and inside(src, nb) and inside(dst, nb)
        ctypes.memmove(dst, src, nb)
        return 0

    def copy2(dst, dpitch, src, spitch, width, height, kind, s):
        assert kind == 2
        for i in range(height):
            assert inside(src + i * spitch, width) and inside(dst + i * dpitch, width)
            ctypes.memmove(dst + i * dpitch, src + i * spitch, width)
        return 0

    class Fn:                     # accepts the restype/argtypes the bench sets
        def __init__(self, f):
            self.f = f

        def __call__(self, *a):
            return self.f(*a)

    class FakeStream:
        cuda_stream = 1

        def synchronize(self):
            pass

    class FakeTorch:
        cuda = types.SimpleNamespace(Stream=FakeStream, synchronize=lambda: None)

        def __getattr__(self, name):
            return getattr(torch, name)

        @staticmethod
        def empty(*a, **kw):
            kw.pop("device", None)
            kw.pop("pin_memory", None)
            t = torch.empty(*a, **kw)
            live.append(t)
            return t

    pos = [int(p) for p in rng.integers(0, S, size=B)]
    want = oracle.pack(w.dims, K.reshape(L, B, H, D // 8, S, 8), V.reshape(L, B, H, S, D),
                       0, L, pos, [1] * B)

    def pack(lay, k_, v_, l0, nl, start, count, st, nbytes, s):
        st.numpy().view(np.uint16)[:] = want

    lay = types.SimpleNamespace(L=L, B=B, H=H, D=D, Smax=S, k_bytes=2 * n, v_bytes=2 * n)
    fkv = types.SimpleNamespace(
        _lib=types.SimpleNamespace(hipMemcpyAsync=Fn(copy1), hipMemcpy2DAsync=Fn(copy2),
                                   hipPeekAtLastError=Fn(lambda: 0)),
        kv_pack_tokens=pack, kv_pack_bytes=lambda lay_, nl, c, u: 2 * nl * B * H * D * 2 * u)
    monkeypatch.setattr(bench, "_pinned", lambda t, nb: FakeTorch.empty((nb + 1) // 2,
                                                                        dtype=torch.int16))
    step = types.SimpleNamespace(torch=FakeTorch(), lay=lay, positions=[pos])
    r = bench.buffered_vs_naive(step, fkv, (k, v), reps=1, keep_image=True)
    assert r["copies_per_step"] == {"buffered": 1, "per_piece": L * B * H * (D // 8 + 1),
                                    "per_head": 2 * L * B * H}
    assert r["host_images_equal"]
    assert np.array_equal(r["image"].numpy().view(np.uint16), want)
