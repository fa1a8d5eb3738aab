"""State replication and recovery on one GPU (DejaVu summary, Failure
detection and recovery, Fig 10: the data leg).

Two microbatches replicate their prompt KV (swap-out to pinned host memory)
and every decode step (staging ring flushed to pinned host memory).  Each
worker acknowledges the steps whose flush has landed.  After a "failure" --
the device caches overwritten from the host, with unflushed steps lost -- the
restart point comes from the acknowledgements, the caches are rebuilt from the
replicas (prompt swap-in + ring restore of the durable prefix) and must equal,
bit for bit, what the oracle builds from the same replica bytes; decoding then
resumes at the restart step.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import dev, empty, host, note, pinned, pinned_host_view

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    import kv_cache_streaming_amd as kv
    return kv


def test_replicate_fail_restore_resume(kv):
    import torch
    dims = (4, 3, 2, 64, 64)
    L, B, H, D, S = dims
    M, prompt, T, R = 2, 20, 21, 4
    note(f"replication dims={dims} microbatches={M} steps={T} R={R}")
    lay = kv.kv_layout_init(*dims, 0)
    rng = np.random.default_rng(123)
    caches = [synth.cache_pair(dims, 900 + j) for j in range(M)]
    dk = [dev(c[0]) for c in caches]
    dv = [dev(c[1]) for c in caches]
    copy = torch.cuda.Stream()
    # prompt replicas
    rows = [prompt] * B
    pbytes = kv.kv_pack_bytes(lay, L, rows)
    eng = kv.KvSwap(lay, torch.empty(pbytes // 2, dtype=torch.int16, device="cuda"),
                    torch.empty(pbytes // 2, dtype=torch.int16, device="cuda"), pbytes, copy)
    prep = [pinned(pbytes // 2) for _ in range(M)]
    done = torch.cuda.Event()
    for j in range(M):
        eng.swap_out(dk[j], dv[j], 0, L, [0] * B, rows, prep[j], pbytes, None, done)
    # decode rings
    slot = kv.kv_pack_bytes(lay, L, None, 1)
    rhost = [pinned(T * slot // 2) for _ in range(M)]
    rings = [kv.KvRing(lay, R, torch.empty(R * slot // 2, dtype=torch.int16, device="cuda"),
                       torch.empty(R * slot // 2, dtype=torch.int16, device="cuda"), rhost[j],
                       copy_stream=copy) for j in range(M)]
    log = kv.KvAckLog(1, M)
    one = [1] * B
    staged = [[] for _ in range(M)]       # what each step wrote (the "model" output)
    for t in range(T):
        pos = [prompt + t] * B
        for j in range(M):
            # the step's new K/V at position prompt+t, written through an unpack
            new = rng.integers(0, 1 << 16, size=oracle.pack_elems(dims, L, one),
                               dtype=np.uint32).astype(np.uint16)
            staged[j].append(new)
            st = dev(new)
            kv.kv_unpack_tokens(lay, dk[j], dv[j], 0, L, pos, one, st)
            rings[j].push(dk[j], dv[j], pos)
            durable = rings[j].durable_steps
            if durable > 0:
                log.ack(0, j, durable - 1)
    torch.cuda.synchronize()
    for j in range(M):                    # the flushes issued so far have landed
        d = rings[j].durable_steps
        assert d == (T // R) * R, d
        log.ack(0, j, d - 1)
    done.synchronize()
    # failure: device state lost (unflushed ring steps are gone with it)
    for j in range(M):
        dk[j].fill_(0x1DEA)
        dv[j].fill_(0x1DEA)
    j0, t0 = log.restart_point()
    assert (j0, t0) == oracle.restart_point(1, M, [(0, j, (T // R) * R - 1) for j in range(M)])
    assert (j0, t0) == (0, (T // R) * R)
    # recovery from the replicas
    for j in range(M):
        eng.swap_in(dk[j], dv[j], 0, L, [0] * B, rows, prep[j], pbytes)
        rings[j].restore_steps(dk[j], dv[j], t0)
        assert rings[j].steps == t0
    torch.cuda.synchronize()
    for j in range(M):
        ek = np.full(L * B * H * D * S, 0x1DEA, np.uint16)
        ev = ek.copy()
        oracle.unpack(dims, ek, ev, 0, L, [0] * B, rows, pinned_host_view(prep[j]))
        positions = [[prompt + t] * B for t in range(t0)]
        oracle.ring_restore(dims, ek, ev, positions, pinned_host_view(rhost[j]))
        assert np.array_equal(host(dk[j]), ek), f"microbatch {j} K after recovery"
        assert np.array_equal(host(dv[j]), ev), f"microbatch {j} V after recovery"
        # the replica's decode slots are exactly what each step wrote
        img = pinned_host_view(rhost[j])
        for t in range(t0):
            assert np.array_equal(img[t * (slot // 2):(t + 1) * (slot // 2)], staged[j][t])
    # resume: the ring continues at the restart step
    for j in range(M):
        rings[j].push(dk[j], dv[j], [prompt + t0] * B)
        assert rings[j].steps == t0 + 1
        rings[j].flush(None, done)
    done.synchronize()
    for j in range(M):
        want = oracle.pack(dims, host(dk[j]), host(dv[j]), 0, L, [prompt + t0] * B, one)
        img = pinned_host_view(rhost[j])
        assert np.array_equal(img[t0 * (slot // 2):(t0 + 1) * (slot // 2)], want)
        assert rings[j].durable_steps == t0 + 1
        rings[j].close()
    eng.close()


@pytest.mark.parametrize("same_stream", [True, False])
def test_restore_steps_waits_for_unflushed_pack(kv, same_stream):
    """A partial restore issued right after a push whose pack has not run yet
    (held back by a bounded spin on its stream), with no host synchronisation
    in between: the restore loads the replica into the bank that pack writes,
    so the load must wait for it, or the restored step 0 would carry the
    unflushed step's bytes.  Each-step gather; the pushes' stream is the
    restore's own, or another one."""
    import torch
    dims = (3, 2, 2, 64, 40)
    L, B, H, D, S = dims
    R = 4
    note(f"restore_steps after an unflushed pack dims={dims} R={R} same_stream={same_stream}")
    lay = kv.kv_layout_init(*dims, 0)
    K, V = synth.cache_pair(dims, 4321)
    dk, dv = dev(K), dev(V)
    slot = kv.kv_pack_bytes(lay, L, None, 1)
    T = 2 * R + 1
    rhost = pinned(T * slot // 2)
    copy = torch.cuda.Stream()
    push_s = torch.cuda.Stream()
    restore_s = push_s if same_stream else torch.cuda.Stream()
    ring = kv.KvRing(lay, R, empty(R * slot // 2), empty(R * slot // 2), rhost, copy_stream=copy)
    positions = [[3 * t + b for b in range(B)] for t in range(T)]
    rk, rv = empty(K.size, fill=0x1DEA), empty(V.size, fill=0x1DEA)
    torch.cuda.synchronize()                     # inputs in place; none from here on
    for t in range(2 * R):                       # two banks, both flushed
        ring.push(dk, dv, positions[t], push_s)
    with torch.cuda.stream(push_s):
        torch.cuda._sleep(200_000_000)           # holds back the next pack
    ring.push(dk, dv, positions[2 * R], push_s)  # step 2R: slot 0 of bank 0, not flushed
    ring.restore_steps(rk, rv, 2 * R, restore_s)
    assert ring.steps == 2 * R
    torch.cuda.synchronize()
    slots = [oracle.pack(dims, K, V, 0, L, positions[t], [1] * B) for t in range(2 * R)]
    img = oracle.ring_host(slots)
    assert np.array_equal(pinned_host_view(rhost)[:img.size], img), "replica differs"
    ek = np.full(K.size, 0x1DEA, np.uint16)
    ev = ek.copy()
    oracle.ring_restore(dims, ek, ev, positions[:2 * R], img)
    assert np.array_equal(host(rk), ek) and np.array_equal(host(rv), ev), "restore differs"
    ring.close()
