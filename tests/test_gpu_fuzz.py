"""Seeded random cases through every copy entry point, bit for bit against
the oracle.

The hand-picked parity cases fix the shapes that matter; these draw many
more at random (head dims of every compiled vector count and odd ones,
ragged and empty rows, rows that end at Smax, layer and head sub-ranges,
both dtypes, shared and distinct page blocks, decode sequences with runs of
consecutive positions, duplicates, partial flushes and truncated restores),
so that the choice between kernels (few tokens per row or token tiles, one
step or several steps at once) and the tails of every tile are crossed many
times.  Each case prints its parameters before it runs.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import dev, empty, host, note, pinned, pinned_host_view

pytestmark = pytest.mark.gpu

CANARY = 64
VEC_COUNTS = [1, 2, 3, 4, 5, 8, 12, 16, 31, 32, 33, 64, 96, 128]   # D / 8


@pytest.fixture(scope="module")
def kv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    import kv_cache_streaming_amd as kv
    return kv


def draw_ranges(rng, B, S):
    """Per-row [start, start + count) within [0, S): one of several regimes."""
    mode = rng.choice(["few", "tiles", "mixed", "to_end"])
    start, count = [], []
    for _ in range(B):
        if mode == "few" or (mode == "mixed" and rng.random() < 0.5):
            c = int(rng.integers(0, min(S, 8) + 1))
        else:
            c = int(rng.integers(0, S + 1))
        s = S - c if mode == "to_end" else int(rng.integers(0, S - c + 1))
        start.append(s)
        count.append(c)
    return np.array(start, np.int32), np.array(count, np.int32), mode


def draw_dims(rng, max_words=3_000_000):
    while True:
        C = int(rng.choice(VEC_COUNTS))
        dims = (int(rng.integers(1, 4)), int(rng.integers(1, 7)), int(rng.integers(1, 5)),
                8 * C, int(rng.integers(1, 400)))
        if np.prod(dims) <= max_words:
            return dims


def test_pack_and_unpack_random(kv):
    import torch
    rng = np.random.default_rng(20240611)
    for case in range(400):
        dims = draw_dims(rng)
        L, B, H, D, S = dims
        dtype = int(rng.integers(0, 2))
        l0 = int(rng.integers(0, L))
        nl = int(rng.integers(1, L - l0 + 1))
        start, count, mode = draw_ranges(rng, B, S)
        note(f"fuzz pack/unpack #{case} dims={dims} dtype={dtype} layers=[{l0},+{nl}) {mode} "
             f"start={start.tolist()} count={count.tolist()}")
        K, V = synth.cache_pair(dims, 5000 + case, dtype=dtype, bits=case % 3 == 0)
        lay = kv.kv_layout_init(L, B, H, D, S, dtype)
        dk, dv = dev(K), dev(V)
        want = oracle.pack(dims, K, V, l0, nl, start, count)
        assert kv.kv_pack_bytes(lay, nl, count) == want.nbytes
        st = empty(want.size, CANARY)
        kv.kv_pack_tokens(lay, dk, dv, l0, nl, start, count, st, want.nbytes)
        torch.cuda.synchronize()
        got = host(st)
        assert np.array_equal(got[:want.size], want), f"case {case}: pack"
        assert np.all(got[want.size:] == 0x7A7A), f"case {case}: pack wrote past its bytes"
        assert np.array_equal(host(dk), K) and np.array_equal(host(dv), V), f"case {case}"
        ek = np.full(K.size, 0xC3C3, np.uint16)
        ev = np.full(V.size, 0x3C3C, np.uint16)
        gk, gv = dev(ek), dev(ev)
        packed = synth.random_bits(want.size, 9000 + case)
        oracle.unpack(dims, ek, ev, l0, nl, start, count, packed)
        kv.kv_unpack_tokens(lay, gk, gv, l0, nl, start, count, dev(packed, CANARY),
                            packed.nbytes)
        torch.cuda.synchronize()
        assert np.array_equal(host(gk), ek) and np.array_equal(host(gv), ev), f"case {case}: unpack"


def draw_part(rng, L, H, R):
    l0 = int(rng.integers(0, L))
    h0 = int(rng.integers(0, H))
    r0 = int(rng.integers(0, R))
    return (l0, int(rng.integers(1, L - l0 + 1)), h0, int(rng.integers(1, H - h0 + 1)),
            r0, int(rng.integers(1, R - r0 + 1)))


def test_stream_out_and_in_random(kv):
    """Random source and destination partitions of a model with 4 layers, 6
    heads and 6 requests: the piece, then its merge into the destination."""
    import torch
    rng = np.random.default_rng(777)
    for case in range(200):
        D = 8 * int(rng.choice(VEC_COUNTS[:10]))
        S = int(rng.integers(1, 300))
        src, dst = draw_part(rng, 4, 6, 6), draw_part(rng, 4, 6, 6)
        sdims, ddims = oracle.part_dims(src, D, S), oracle.part_dims(dst, D, S)
        start, count, mode = draw_ranges(rng, src[5], S)
        note(f"fuzz stream #{case} src={src} dst={dst} D={D} S={S} {mode} "
             f"start={start.tolist()} count={count.tolist()}")
        lay = kv.kv_layout_init(*sdims, 0)
        K, V = synth.cache_pair(sdims, 6000 + case, bits=True)
        want = oracle.stream_out(src, dst, D, S, K, V, start, count)
        nbytes = kv.kv_stream_bytes(lay, src, dst, count)
        assert nbytes == want.size * 2
        st = empty(want.size, CANARY)
        kv.kv_stream_out(lay, src, dev(K), dev(V), dst, start, count, st, nbytes)
        torch.cuda.synchronize()
        got = host(st)
        assert np.array_equal(got[:want.size], want), f"case {case}: piece"
        assert np.all(got[want.size:] == 0x7A7A), f"case {case}: wrote past the piece"
        if want.size == 0:
            continue
        # merge: the shared rows keep the source's counts at a new start; the
        # other rows get any valid range (they are not written)
        dstart = np.zeros(dst[5], np.int32)
        dcount = np.zeros(dst[5], np.int32)
        for bd in range(dst[5]):
            gr = dst[4] + bd
            if src[4] <= gr < src[4] + src[5]:
                c = int(count[gr - src[4]])
                dcount[bd] = c
                dstart[bd] = int(rng.integers(0, S - c + 1))
            else:
                dcount[bd] = int(rng.integers(0, S + 1))
                dstart[bd] = int(rng.integers(0, S - dcount[bd] + 1))
        dlay = kv.kv_layout_init(*ddims, 0)
        n = int(np.prod(ddims))
        eK, eV = np.full(n, 0x3C3C, np.uint16), np.full(n, 0x3C3C, np.uint16)
        oracle.stream_in(dst, src, D, S, eK, eV, dstart, dcount, want)
        gk, gv = empty(n, fill=0x3C3C), empty(n, fill=0x3C3C)
        kv.kv_stream_in(dlay, dst, gk, gv, src, dstart, dcount, st, nbytes)
        torch.cuda.synchronize()
        assert np.array_equal(host(gk), eK) and np.array_equal(host(gv), eV), f"case {case}: merge"


def test_paged_random(kv):
    import torch
    rng = np.random.default_rng(4242)
    for case in range(200):
        L = int(rng.integers(1, 4))
        H = int(rng.integers(1, 4))
        D = 8 * int(rng.choice(VEC_COUNTS[:12]))
        P = int(rng.choice([1, 2, 3, 5, 8, 16, 32, 64, 256]))
        B = int(rng.integers(1, 6))
        stride = int(rng.integers(1, max(2, 600 // P) + 1))
        NB = B * stride + int(rng.integers(0, 5))
        pd = (L, NB, H, D, P)
        if np.prod(pd) > 4_000_000:
            continue
        cap = stride * P
        start, count, mode = draw_ranges(rng, B, cap)
        shared = bool(rng.random() < 0.5)
        note(f"fuzz paged #{case} pool={pd} B={B} stride={stride} {mode} shared={shared} "
             f"start={start.tolist()} count={count.tolist()}")
        pg = kv.kv_paged_init(L, NB, H, D, P, 0)
        n = L * NB * H * D * P
        Kp, Vp = synth.random_bits(n, 7000 + case), synth.random_bits(n, 7100 + case)
        if shared:
            table = rng.integers(0, NB, size=(B, stride)).astype(np.int32)
        else:
            table = rng.permutation(NB)[:B * stride].reshape(B, stride).astype(np.int32)
        dtab = torch.from_numpy(np.ascontiguousarray(table)).cuda()
        l0 = int(rng.integers(0, L))
        nl = int(rng.integers(1, L - l0 + 1))
        want = oracle.pack_paged(pd, Kp, Vp, l0, nl, table, start, count)
        nbytes = kv.kv_paged_pack_bytes(pg, nl, B, count)
        assert nbytes == want.nbytes
        st = empty(want.size, CANARY)
        kv.kv_pack_paged(pg, dev(Kp), dev(Vp), l0, nl, dtab, start, count, st, nbytes)
        torch.cuda.synchronize()
        got = host(st)
        assert np.array_equal(got[:want.size], want), f"case {case}: paged pack"
        assert np.all(got[want.size:] == 0x7A7A), f"case {case}: wrote past the packed words"
        if shared:
            continue   # an unpack through shared blocks has no single answer
        packed = synth.random_bits(want.size, 7200 + case)
        eK, eV = np.full(n, 0x6B6B, np.uint16), np.full(n, 0x6B6B, np.uint16)
        oracle.unpack_paged(pd, eK, eV, l0, nl, table, start, count, packed)
        gk, gv = empty(n, fill=0x6B6B), empty(n, fill=0x6B6B)
        kv.kv_unpack_paged(pg, gk, gv, l0, nl, dtab, start, count, dev(packed, CANARY),
                           packed.nbytes)
        torch.cuda.synchronize()
        assert np.array_equal(host(gk), eK) and np.array_equal(host(gv), eV), \
            f"case {case}: paged unpack"


def draw_positions(rng, B, S, steps):
    """Decode positions: mostly every row advancing by one (runs), sometimes a
    jump or a repeat of the previous step."""
    pos = [rng.integers(0, S, size=B)]
    for _ in range(steps - 1):
        r = rng.random()
        if r < 0.65 and np.all(pos[-1] + 1 < S):
            pos.append(pos[-1] + 1)
        elif r < 0.75:
            pos.append(pos[-1].copy())
        else:
            pos.append(rng.integers(0, S, size=B))
    return [[int(x) for x in p] for p in pos]


def test_ring_random_sequences(kv):
    """Pushes with partial flushes at random points, gather mode switched
    between flushed states, a truncated restore that rewinds the ring, and a
    final restore; the host image and every restore against the oracle."""
    import torch
    rng = np.random.default_rng(99)
    for case in range(100):
        C = int(rng.choice([1, 2, 3, 8, 16, 32, 128]))
        dims = (int(rng.integers(1, 4)), int(rng.integers(1, 5)), int(rng.integers(1, 4)),
                8 * C, int(rng.integers(2, 90)))
        L, B, H, D, S = dims
        R = int(rng.integers(1, 7))
        steps = int(rng.integers(1, 40))
        transport = int(rng.choice([0, 1, 2, 3, 5]))
        positions = draw_positions(rng, B, S, steps)
        note(f"fuzz ring #{case} dims={dims} R={R} steps={steps} transport={transport}")
        pairs = [synth.cache_pair(dims, 8000 + 10 * case + i, bits=True) for i in range(2)]
        devs = [(dev(a), dev(b)) for a, b in pairs]
        lay = kv.kv_layout_init(L, B, H, D, S, 0)
        slot = kv.kv_pack_bytes(lay, L, None, 1)
        banks = [empty(R * slot // 2), empty(R * slot // 2)]
        hostbuf = pinned(steps * slot // 2 + CANARY)
        copy = torch.cuda.Stream()
        compute = torch.cuda.current_stream()
        ring = kv.KvRing(lay, R, banks[0], banks[1], hostbuf, host_bytes=steps * slot,
                         copy_stream=copy, transport=transport)
        gather = int(rng.integers(0, 2))
        ring.set_gather(gather)
        rewind_at = int(rng.integers(0, steps + 1)) if rng.random() < 0.5 else -1
        kept_pos, kept_slots = [], []
        j = 0
        while j < steps:
            pair = int(rng.integers(0, 2)) if rng.random() < 0.2 else 0
            pos = positions[j]
            kept_slots.append(oracle.pack(dims, pairs[pair][0], pairs[pair][1], 0, L, pos,
                                          [1] * B))
            kept_pos.append(pos)
            ring.push(devs[pair][0], devs[pair][1], pos, compute)
            j += 1
            if rng.random() < 0.15:
                ring.flush(compute)
                if rng.random() < 0.3:
                    gather = 1 - gather
                    ring.set_gather(gather)
            if j == rewind_at:
                # keep a prefix of the replicated steps and carry on from there
                ring.flush(compute)
                n = int(rng.integers(0, len(kept_pos) + 1))
                zk, zv = np.zeros(pairs[0][0].size, np.uint16), np.zeros(pairs[0][1].size,
                                                                          np.uint16)
                rk, rv = dev(zk), dev(zv)
                ring.restore_steps(rk, rv, n, compute)
                torch.cuda.synchronize()
                if n:
                    oracle.ring_restore(dims, zk, zv, kept_pos[:n], oracle.ring_host(kept_slots[:n]))
                assert np.array_equal(host(rk), zk) and np.array_equal(host(rv), zv), \
                    f"case {case}: restore of the first {n} steps"
                del kept_pos[n:], kept_slots[n:]
                assert ring.steps == n
        done = torch.cuda.Event()
        ring.flush(compute, done)
        done.synchronize()
        want_host = oracle.ring_host(kept_slots) if kept_slots else np.zeros(0, np.uint16)
        got_host = pinned_host_view(hostbuf)
        assert np.array_equal(got_host[:want_host.size], want_host), f"case {case}: host image"
        assert np.all(got_host[steps * slot // 2:] == 0x5C5C), f"case {case}: wrote past the image"
        zk, zv = np.zeros(pairs[0][0].size, np.uint16), np.zeros(pairs[0][1].size, np.uint16)
        rk, rv = dev(zk), dev(zv)
        if kept_pos:
            oracle.ring_restore(dims, zk, zv, kept_pos, want_host)
        ring.restore(rk, rv, compute)
        torch.cuda.synchronize()
        assert np.array_equal(host(rk), zk) and np.array_equal(host(rv), zv), f"case {case}: restore"
        ring.close()
