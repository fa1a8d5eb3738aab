"""Library calls captured into a HIP graph replay bit for bit.

A launch-bound loop of decode-step packs is what a caller would capture
once and replay.  Every call enqueues only kernels whose row ranges travel
in the kernel arguments, so a capture holds each call's ranges by value and
needs no device metadata.  The caches change between replays (eager writes
on the program's own stream, with synchronizations in between), and every
replay is checked against the oracle on the new contents.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import dev, host, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    import kv_cache_streaming_amd as kv
    return kv


def test_pack_and_unpack_replay_from_a_graph(kv):
    import torch
    dims = (4, 3, 2, 64, 48)
    L, B, H, D, S = dims
    lay = kv.kv_layout_init(L, B, H, D, S, 0)
    K, V = synth.cache_pair(dims, 41)
    dk, dv = dev(K), dev(V)
    steps = 6
    pos = [[10 + j + 5 * b for b in range(B)] for j in range(steps)]
    slot = kv.kv_pack_bytes(lay, L, None, 1)
    st = torch.zeros(steps * slot // 2, dtype=torch.int16, device="cuda")
    start, count = [3, 0, 10], [20, 0, 33]          # tile kernel, an empty row
    pb = kv.kv_pack_bytes(lay, 2, count)
    st2 = torch.zeros(pb // 2, dtype=torch.int16, device="cuda")
    uk, uv = torch.zeros_like(dk), torch.zeros_like(dv)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    note(f"graph capture dims={dims} steps={steps} ranges start={start} count={count}")
    with torch.cuda.graph(g, stream=s, capture_error_mode="relaxed"):
        for j in range(steps):
            kv.kv_pack_tokens(lay, dk, dv, 0, L, pos[j], None, st[j * slot // 2:], slot, s)
        kv.kv_pack_tokens(lay, dk, dv, 1, 2, start, count, st2, pb, s)
        kv.kv_unpack_tokens(lay, uk, uv, 1, 2, start, count, st2, pb, s)
    torch.cuda.synchronize()
    for rep in range(3):
        K, V = synth.cache_pair(dims, 50 + rep, bits=True)
        dk.copy_(dev(K))
        dv.copy_(dev(V))
        uk.zero_()
        uv.zero_()
        torch.cuda.synchronize()
        note(f"graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        got = host(st)
        for j in range(steps):
            want = oracle.pack(dims, K, V, 0, L, pos[j], [1] * B)
            assert np.array_equal(got[j * slot // 2:(j + 1) * slot // 2], want), (rep, j)
        want = oracle.pack(dims, K, V, 1, 2, start, count)
        assert np.array_equal(host(st2), want), rep
        ek, ev = np.zeros_like(K), np.zeros_like(V)
        oracle.unpack(dims, ek, ev, 1, 2, start, count, want)
        assert np.array_equal(host(uk), ek) and np.array_equal(host(uv), ev), rep
