"""The five workloads at full size, in the bench's launch configuration.

Each test runs a workload's call sequence on its real shape (transport
KV_XFER_AUTO, two staging banks, the ring sizes of the workload) and compares
with the oracle bit for bit: whole buffers where the host can hold the
oracle's inputs, otherwise complete layers or chunks sampled from every part of
the flow (the oracle on one layer of the cache, a property the pins fix: a
multi-layer pack is the concatenation of its per-layer packs).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import note, pinned, pinned_host_view

pytestmark = pytest.mark.gpu

MiB = 1 << 20


@pytest.fixture(scope="module")
def kv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    import kv_cache_streaming_amd as kv
    return kv


@pytest.fixture(autouse=True)
def free_memory():
    """Give device memory and cached pinned host memory back after each test
    (the workloads pin tens of GB of host memory each)."""
    import gc

    import torch
    yield
    torch.cuda.synchronize()
    gc.collect()
    torch.cuda.empty_cache()
    torch._C._host_emptyCache()


def device_cache(w, seed):
    import torch
    n = w.L * w.B * w.H * w.D * w.Smax
    k = torch.empty(n, dtype=torch.int16, device="cuda")
    v = torch.empty(n, dtype=torch.int16, device="cuda")
    synth.fill_device_cache(k, seed, w.dtype)
    synth.fill_device_cache(v, seed + 1, w.dtype)
    return k, v


def layer_host(t, w, l):
    """uint16 host copy of layer l of a flat device cache tensor."""
    return t.view(w.L, -1)[l].cpu().numpy().view(np.uint16).copy()


def row_digest(t, w, l, b):
    """Two integer sums over row b of layer l of a flat device cache tensor
    (plain and position-weighted), as a fingerprint of its contents."""
    import torch
    x = t.view(w.L, w.B, -1)[l, b].view(torch.int32).to(torch.int64)
    wgt = torch.arange(x.numel(), device=x.device, dtype=torch.int64) % 65521 + 1
    return int(x.sum().item()), int((x * wgt).sum().item())


def one_layer(w):
    return (1, w.B, w.H, w.D, w.Smax)


def bank(nbytes):
    import torch
    return torch.empty((nbytes + 15) // 16 * 8, dtype=torch.int16, device="cuda")


def test_gpt2_small_tiny_full_flow(kv):
    """12 prompt-layer packs of 32 tokens, 16 decode steps into a ring of 8, restore
    into a fresh zeroed cache (round-trip identity on the decode region)."""
    import torch
    w = synth.WORKLOADS["gpt2-small-tiny"]
    note(f"workload {w.name} dims={w.dims}")
    K, V = synth.cache_pair(w.dims, w.value_seed, w.dtype)
    lay = kv.kv_layout_init(*w.dims, w.dtype)
    dk = torch.from_numpy(K.view(np.int16)).cuda()
    dv = torch.from_numpy(V.view(np.int16)).cuda()
    lens = synth.row_lengths(w)
    for l in range(w.L):
        want = oracle.pack(w.dims, K, V, l, 1, [0] * w.B, lens)
        st = torch.empty(want.size, dtype=torch.int16, device="cuda")
        kv.kv_pack_prompt_layer(lay, dk, dv, l, 0, w.prompt_len, None, st)
        torch.cuda.synchronize()
        assert np.array_equal(st.cpu().numpy().view(np.uint16), want), f"prompt layer {l}"
    pos = synth.decode_positions(w)
    slot = kv.kv_pack_bytes(lay, w.L, None, 1)
    R = w.ring_slots
    host = pinned(w.decode_steps * slot // 2)
    ring = kv.KvRing(lay, R, bank(R * slot), bank(R * slot), host, copy_stream=torch.cuda.Stream())
    for p in pos:
        ring.push(dk, dv, p)
    done = torch.cuda.Event()
    ring.flush(None, done)
    done.synchronize()
    want = oracle.ring_host([oracle.pack(w.dims, K, V, 0, w.L, p, [1] * w.B) for p in pos])
    assert np.array_equal(pinned_host_view(host), want), "ring host image"
    zk, zv = torch.zeros_like(dk), torch.zeros_like(dv)
    ring.restore(zk, zv)
    ek, ev = np.zeros_like(K), np.zeros_like(V)
    oracle.ring_restore(w.dims, ek, ev, pos, want)
    torch.cuda.synchronize()
    assert np.array_equal(zk.cpu().numpy().view(np.uint16), ek)
    assert np.array_equal(zv.cpu().numpy().view(np.uint16), ev)
    ring.close()


def test_gpt2_1p5b_full_flow(kv):
    """48 streamed prompt layers (1000 tokens), 24 decode steps flushed every 8,
    restore into a zeroed cache, microbatch swap-out/in of all 1024 positions."""
    import torch
    w = synth.WORKLOADS["gpt2-1.5b"]
    note(f"workload {w.name} dims={w.dims}")
    lay = kv.kv_layout_init(*w.dims, w.dtype)
    dk, dv = device_cache(w, w.value_seed)
    K = dk.cpu().numpy().view(np.uint16)
    V = dv.cpu().numpy().view(np.uint16)
    B = w.B
    prompt = [w.prompt_len] * B
    layer_bytes = kv.kv_pack_bytes(lay, 1, prompt)
    copy_out, copy_in = torch.cuda.Stream(), torch.cuda.Stream()
    eng = kv.KvSwap(lay, bank(layer_bytes), bank(layer_bytes), layer_bytes, copy_out)
    host = pinned(w.L * layer_bytes // 2)
    done = torch.cuda.Event()
    for l in range(w.L):
        eng.stream_prompt_layer(dk, dv, l, 0, w.prompt_len, None,
                                host.data_ptr() + l * layer_bytes, layer_bytes, None, done)
    done.synchronize()
    hv = pinned_host_view(host)
    for l in range(w.L):
        want = oracle.pack(w.dims, K, V, l, 1, [0] * B, prompt)
        assert np.array_equal(hv[l * want.size:(l + 1) * want.size], want), f"prompt layer {l}"
    # the streamed prompt loaded back as one call through one-layer banks
    # (the token worker's load in the bench step), into a sentinel cache
    ein = kv.KvSwap(lay, bank(layer_bytes), bank(layer_bytes), layer_bytes, copy_in)
    pk = torch.full_like(dk, 0x0F0F)
    pv = torch.full_like(dv, 0x0F0F)
    ein.swap_in(pk, pv, 0, w.L, [0] * B, prompt, host, w.L * layer_bytes)
    torch.cuda.synchronize()
    ek = np.full_like(K, 0x0F0F)
    ev = np.full_like(V, 0x0F0F)
    oracle.unpack(w.dims, ek, ev, 0, w.L, [0] * B, prompt, hv)
    assert np.array_equal(pk.cpu().numpy().view(np.uint16), ek), "prompt load K"
    assert np.array_equal(pv.cpu().numpy().view(np.uint16), ev), "prompt load V"
    del pk, pv, ek, ev
    ein.close()
    # decode ring, each step packed when pushed and a bank gathered at its flush
    pos = synth.decode_positions(w)
    slot = kv.kv_pack_bytes(lay, w.L, None, 1)
    R = w.ring_slots
    want = oracle.ring_host([oracle.pack(w.dims, K, V, 0, w.L, p, [1] * B) for p in pos])
    ek, ev = np.zeros_like(K), np.zeros_like(V)
    oracle.ring_restore(w.dims, ek, ev, pos, want)
    for gather in (kv.KV_RING_GATHER_EACH_STEP, kv.KV_RING_GATHER_AT_FLUSH):
        rhost = pinned(w.decode_steps * slot // 2)
        ring = kv.KvRing(lay, R, bank(R * slot), bank(R * slot), rhost, copy_stream=copy_out)
        ring.set_gather(gather)
        for p in pos:
            ring.push(dk, dv, p)
        ring.flush(None, done)
        done.synchronize()
        assert np.array_equal(pinned_host_view(rhost), want), f"ring host image (gather {gather})"
        rk, rv = torch.zeros_like(dk), torch.zeros_like(dv)
        ring.restore(rk, rv)
        torch.cuda.synchronize()
        assert np.array_equal(rk.cpu().numpy().view(np.uint16), ek), "restored K"
        assert np.array_equal(rv.cpu().numpy().view(np.uint16), ev), "restored V"
        ring.close()
        del rk, rv
    del ek, ev
    # microbatch swap-out of all 1024 positions, swap-in to a sentinel cache
    full = [w.Smax] * B
    total = kv.kv_pack_bytes(lay, w.L, full)
    sb = 256 * MiB
    eo = kv.KvSwap(lay, bank(sb), bank(sb), sb, copy_out)
    ei = kv.KvSwap(lay, bank(sb), bank(sb), sb, copy_in)
    shost = pinned(total // 2)
    eo.swap_out(dk, dv, 0, w.L, [0] * B, full, shost, total, None, done)
    done.synchronize()
    sv = pinned_host_view(shost)
    per = total // 2 // w.L
    for l in range(w.L):
        want = oracle.pack(w.dims, K, V, l, 1, [0] * B, full)
        assert np.array_equal(sv[l * per:(l + 1) * per], want), f"swap-out layer {l}"
    sk = torch.full_like(dk, 0x1357)
    svv = torch.full_like(dv, 0x2468)
    ei.swap_in(sk, svv, 0, w.L, [0] * B, full, shost, total)
    torch.cuda.synchronize()
    assert torch.equal(sk, dk) and torch.equal(svv, dv), "swap-in of every position restores the cache"
    # the isolated large slice: one pack call over every layer and position
    big = torch.empty(total // 2, dtype=torch.int16, device="cuda")
    kv.kv_pack_tokens(lay, dk, dv, 0, w.L, [0] * B, full, big, total)
    torch.cuda.synchronize()
    assert np.array_equal(big.cpu().numpy().view(np.uint16), sv), "48-layer pack in one call"
    del big
    eng.close()
    eo.close()
    ei.close()


@pytest.mark.parametrize("gather", [0, 1])
def test_opt66b_slice_decode_ring(kv, gather):
    """Ragged decode positions (len_b + j), 64 steps into a ring of 16 flushed to
    pinned host memory, restored into a second, zeroed cache; each step packed
    when pushed, or a bank's 16 steps in one pass at its flush."""
    import torch
    w = synth.WORKLOADS["opt-66b-16l"]
    note(f"workload {w.name} dims={w.dims} gather={gather}")
    lay = kv.kv_layout_init(*w.dims, w.dtype)
    dk, dv = device_cache(w, w.value_seed)
    K = dk.cpu().numpy().view(np.uint16)
    V = dv.cpu().numpy().view(np.uint16)
    pos = synth.decode_positions(w)
    assert pos.max() < w.Smax
    slot = kv.kv_pack_bytes(lay, w.L, None, 1)
    assert slot == 4_718_592
    R = w.ring_slots
    host = pinned(w.decode_steps * slot // 2)
    ring = kv.KvRing(lay, R, bank(R * slot), bank(R * slot), host, copy_stream=torch.cuda.Stream())
    ring.set_gather(gather)
    for p in pos:
        ring.push(dk, dv, p)
    done = torch.cuda.Event()
    ring.flush(None, done)
    done.synchronize()
    want = oracle.ring_host([oracle.pack(w.dims, K, V, 0, w.L, p, [1] * w.B) for p in pos])
    assert np.array_equal(pinned_host_view(host), want), "ring host image"
    rk, rv = torch.zeros_like(dk), torch.zeros_like(dv)
    ring.restore(rk, rv)
    ek, ev = np.zeros_like(K), np.zeros_like(V)
    oracle.ring_restore(w.dims, ek, ev, pos, want)
    torch.cuda.synchronize()
    assert np.array_equal(rk.cpu().numpy().view(np.uint16), ek), "restored K"
    assert np.array_equal(rv.cpu().numpy().view(np.uint16), ev), "restored V"
    ring.close()


def test_bloom_slice_microbatch_swap(kv):
    """Two device slots: swap out microbatch x-1 from slot B while microbatch x+1
    is swapped in to slot A from its host image (layer-pipelined, duplex), then
    the reverse; full 1500-token microbatches of 13.76 GB."""
    import torch
    w = synth.WORKLOADS["bloom-176b-10l"]
    note(f"workload {w.name} dims={w.dims}")
    lay = kv.kv_layout_init(*w.dims, w.dtype)
    B = w.B
    rows = [w.prompt_len] * B
    total = kv.kv_pack_bytes(lay, w.L, rows)
    assert total == 13_762_560_000
    slot_a = device_cache(w, w.value_seed)          # microbatch 0 lives in slot A
    slot_b = device_cache(w, w.value_seed + 40)     # microbatch 1 lives in slot B
    sb = 256 * MiB
    copy_out, copy_in = torch.cuda.Stream(), torch.cuda.Stream()
    eo = kv.KvSwap(lay, bank(sb), bank(sb), sb, copy_out)
    ei = kv.KvSwap(lay, bank(sb), bank(sb), sb, copy_in)
    host = [pinned(total // 2) for _ in range(2)]
    per = total // 2 // w.L
    s_a, s_b = torch.cuda.Stream(), torch.cuda.Stream()
    # initial swap-out of microbatch 0 (slot A) to host[0]
    done = torch.cuda.Event()
    eo.swap_out(slot_a[0], slot_a[1], 0, w.L, [0] * B, rows, host[0], total, s_a, done)
    done.synchronize()
    samples = (0, 7)
    ref_a = {l: (layer_host(slot_a[0], w, l), layer_host(slot_a[1], w, l)) for l in samples}
    hv0 = pinned_host_view(host[0])
    for l in samples:
        want = oracle.pack(one_layer(w), ref_a[l][0], ref_a[l][1], 0, 1, [0] * B, rows)
        assert np.array_equal(hv0[l * per:(l + 1) * per], want), f"swap-out mb0 layer {l}"
    ref_b = {l: (layer_host(slot_b[0], w, l), layer_host(slot_b[1], w, l)) for l in samples}
    # duplex round: swap out microbatch 1 from slot B to host[1] while microbatch 0
    # comes back into slot A (overwritten first with a sentinel) from host[0]
    slot_a[0].fill_(0x0BAD)
    slot_a[1].fill_(0x0BAD)
    torch.cuda.synchronize()
    d_out, d_in = torch.cuda.Event(), torch.cuda.Event()
    for l in range(w.L):
        eo.swap_out(slot_b[0], slot_b[1], l, 1, [0] * B, rows, host[1].data_ptr() + l * per * 2,
                    per * 2, s_b, d_out)
        ei.swap_in(slot_a[0], slot_a[1], l, 1, [0] * B, rows, host[0].data_ptr() + l * per * 2,
                   per * 2, s_a, d_in)
    d_out.synchronize()
    d_in.synchronize()
    torch.cuda.synchronize()
    hv1 = pinned_host_view(host[1])
    for l in samples:
        want = oracle.pack(one_layer(w), ref_b[l][0], ref_b[l][1], 0, 1, [0] * B, rows)
        assert np.array_equal(hv1[l * per:(l + 1) * per], want), f"swap-out mb1 layer {l}"
        ek = np.full_like(ref_a[l][0], 0x0BAD)
        ev = np.full_like(ref_a[l][1], 0x0BAD)
        oracle.unpack(one_layer(w), ek, ev, 0, 1, [0] * B, rows, hv0[l * per:(l + 1) * per])
        assert np.array_equal(layer_host(slot_a[0], w, l), ek), f"swap-in mb0 K layer {l}"
        assert np.array_equal(layer_host(slot_a[1], w, l), ev), f"swap-in mb0 V layer {l}"
    eo.close()
    ei.close()


def test_bloom_slice_one_call_past_4gib(kv):
    """One pack and one unpack call over all 10 layers of the BLOOM slice with
    ragged rows: a 13.9 GB packed buffer, so every offset past 4 GiB in the
    staging buffer is exercised in a single launch sequence."""
    import torch
    w = synth.WORKLOADS["bloom-176b-10l"]
    L, B, H, D, S = w.dims
    lay = kv.kv_layout_init(*w.dims, w.dtype)
    rng = np.random.default_rng(4)
    count = rng.integers(1200, S + 1, size=B).astype(np.int32)
    start = np.array([int(rng.integers(0, S - c + 1)) for c in count], np.int32)
    total = kv.kv_pack_bytes(lay, L, count)
    assert total > 1 << 32
    note(f"workload {w.name} one call of {total} bytes, start={start.tolist()} count={count.tolist()}")
    src = device_cache(w, w.value_seed + 7)
    st = torch.full((total // 2 + 64,), 0x7A7A, dtype=torch.int16, device="cuda")
    kv.kv_pack_tokens(lay, src[0], src[1], 0, L, start, count, st, total)
    torch.cuda.synchronize()
    per = total // 2 // L
    got = st.view(-1)
    assert np.all(got[total // 2:].cpu().numpy() == 0x7A7A), "wrote past the packed bytes"
    for l in (0, L // 2, L - 1):
        Kl, Vl = layer_host(src[0], w, l), layer_host(src[1], w, l)
        want = oracle.pack(one_layer(w), Kl, Vl, 0, 1, start, count)
        assert np.array_equal(got[l * per:(l + 1) * per].cpu().numpy().view(np.uint16), want), \
            f"pack layer {l}"
    dst = (torch.full_like(src[0], 0x1F1F), torch.full_like(src[1], 0x1F1F))
    del src
    kv.kv_unpack_tokens(lay, dst[0], dst[1], 0, L, start, count, st, total)
    torch.cuda.synchronize()
    for l in (0, L - 1):
        ek = np.full(B * H * D * S, 0x1F1F, np.uint16)
        ev = ek.copy()
        oracle.unpack(one_layer(w), ek, ev, 0, 1, start, count,
                      got[l * per:(l + 1) * per].cpu().numpy().view(np.uint16))
        assert np.array_equal(layer_host(dst[0], w, l), ek), f"unpack K layer {l}"
        assert np.array_equal(layer_host(dst[1], w, l), ev), f"unpack V layer {l}"


@pytest.mark.parametrize("transport", [1, 0, 5])
def test_swap_through_banks_past_1gib(kv, transport):
    """Swap-out and swap-in of every GPT-2-1.5B layer and position through
    1.5 GiB banks (30 layers per chunk): each link copy of a chunk is cut into
    launches of at most 1 GiB, in both directions with the kernel transport."""
    import torch
    w = synth.WORKLOADS["gpt2-1.5b"]
    L, B = w.L, w.B
    note(f"workload {w.name} 1.5 GiB banks transport={transport}")
    lay = kv.kv_layout_init(*w.dims, w.dtype)
    full = [w.Smax] * B
    total = kv.kv_pack_bytes(lay, L, full)
    sb = 1536 * MiB
    plan = kv.kv_swap_plan(lay, 0, L, [0] * B, full, sb)
    assert [c["layer_count"] for c in plan] == [30, 18]
    src = device_cache(w, w.value_seed + 11)
    copy_out, copy_in = torch.cuda.Stream(), torch.cuda.Stream()
    eo = kv.KvSwap(lay, bank(sb), bank(sb), sb, copy_out, transport)
    ei = kv.KvSwap(lay, bank(sb), bank(sb), sb, copy_in, transport)
    host = pinned(total // 2 + 64)
    done = torch.cuda.Event()
    eo.swap_out(src[0], src[1], 0, L, [0] * B, full, host, total, None, done)
    done.synchronize()
    hv = pinned_host_view(host)
    assert np.all(hv[total // 2:] == 0x5C5C), "wrote past the host image"
    per = total // 2 // L
    for l in (0, 29, 30, L - 1):
        want = oracle.pack(one_layer(w), layer_host(src[0], w, l), layer_host(src[1], w, l), 0, 1,
                           [0] * B, full)
        assert np.array_equal(hv[l * per:(l + 1) * per], want), f"swap-out layer {l}"
    dk, dv = torch.full_like(src[0], 0x2E2E), torch.full_like(src[1], 0x2E2E)
    ei.swap_in(dk, dv, 0, L, [0] * B, full, host, total)
    torch.cuda.synchronize()
    assert torch.equal(dk, src[0]) and torch.equal(dv, src[1]), "swap-in restores every position"
    eo.close()
    ei.close()


def test_gqa_100k_long_context(kv):
    """bf16, Smax = 100000, ragged rows: 4096-token prompt chunks per layer, 64
    ragged decode steps into a ring of 16, swap-out/in of the longest row."""
    import torch
    w = synth.WORKLOADS["gqa-100k"]
    note(f"workload {w.name} dims={w.dims}")
    lay = kv.kv_layout_init(*w.dims, w.dtype)
    B = w.B
    lens = synth.row_lengths(w)
    dk, dv = device_cache(w, w.value_seed)
    lk, lv = {}, {}

    def host_layer(l):
        if l not in lk:
            lk[l], lv[l] = layer_host(dk, w, l), layer_host(dv, w, l)
        return lk[l], lv[l]

    # chunked prompt packs: every chunk of layer 0, first and last chunks of two others
    chunk = w.chunk_tokens
    nchunks = (int(lens.max()) + chunk - 1) // chunk
    st = bank(kv.kv_pack_bytes(lay, 1, None, chunk))
    cases = [(0, c) for c in range(nchunks)] + [(59, 0), (59, nchunks - 1), (31, 0),
                                                 (31, nchunks // 2), (31, nchunks - 1)]
    for l, c in cases:
        tb = c * chunk
        tc = min(chunk, w.Smax - tb)
        start, count = oracle.prompt_ranges(B, tb, tc, lens)
        need = kv.kv_pack_bytes(lay, 1, count)
        if need == 0:
            continue
        kv.kv_pack_prompt_layer(lay, dk, dv, l, tb, tc, lens, st, need)
        torch.cuda.synchronize()
        K1, V1 = host_layer(l)
        want = oracle.pack(one_layer(w), K1, V1, 0, 1, start, count)
        got = st.cpu().numpy().view(np.uint16)[:want.size]
        assert np.array_equal(got, want), f"prompt chunk layer {l} chunk {c}"
    # decode ring, ragged positions
    pos = synth.decode_positions(w)
    assert pos.max() < w.Smax
    slot = kv.kv_pack_bytes(lay, w.L, None, 1)
    assert slot == 983_040
    R = w.ring_slots
    host = pinned(w.decode_steps * slot // 2)
    ring = kv.KvRing(lay, R, bank(R * slot), bank(R * slot), host, copy_stream=torch.cuda.Stream())
    ring.set_gather(kv.KV_RING_GATHER_AT_FLUSH)       # as the bench step runs it
    for p in pos:
        ring.push(dk, dv, p)
    done = torch.cuda.Event()
    ring.flush(None, done)
    done.synchronize()
    hv = pinned_host_view(host)
    per_layer = slot // 2 // w.L
    for l in (0, 31, 59):
        K1, V1 = host_layer(l)
        for j, p in enumerate(pos):
            want = oracle.pack(one_layer(w), K1, V1, 0, 1, p, [1] * B)
            got = hv[j * (slot // 2) + l * per_layer:j * (slot // 2) + (l + 1) * per_layer]
            assert np.array_equal(got, want), f"ring step {j} layer {l}"
    ring.close()
    # swap-out of the longest row over all 60 layers, then swap-in after the row is
    # overwritten with a sentinel
    bstar = int(np.argmax(lens))
    count = [0] * B
    count[bstar] = int(lens[bstar])
    total = kv.kv_pack_bytes(lay, w.L, count)
    per = total // 2 // w.L
    sb = 512 * MiB
    copy_out, copy_in = torch.cuda.Stream(), torch.cuda.Stream()
    eo = kv.KvSwap(lay, bank(sb), bank(sb), sb, copy_out)
    ei = kv.KvSwap(lay, bank(sb), bank(sb), sb, copy_in)
    shost = pinned(total // 2)
    eo.swap_out(dk, dv, 0, w.L, [0] * B, count, shost, total, None, done)
    done.synchronize()
    sv = pinned_host_view(shost)
    for l in (0, 31, 59):
        K1, V1 = host_layer(l)
        want = oracle.pack(one_layer(w), K1, V1, 0, 1, [0] * B, count)
        assert np.array_equal(sv[l * per:(l + 1) * per], want), f"row swap-out layer {l}"
    # every layer of the image: the row's own region of each layer is a cache
    # of one row, so the oracle packs it from that region alone
    row_dims = (1, 1, w.H, w.D, w.Smax)
    for l in range(w.L):
        Kr = dk.view(w.L, B, -1)[l, bstar].cpu().numpy().view(np.uint16)
        Vr = dv.view(w.L, B, -1)[l, bstar].cpu().numpy().view(np.uint16)
        want = oracle.pack(row_dims, Kr, Vr, 0, 1, [0], [count[bstar]])
        assert np.array_equal(sv[l * per:(l + 1) * per], want), f"row swap-out layer {l}"
    # the row as it was (device copy) and digests of every other row of every
    # layer, to compare after the swap-in
    saved_k = dk.view(w.L, B, -1)[:, bstar, :].clone()
    saved_v = dv.view(w.L, B, -1)[:, bstar, :].clone()
    others = [b for b in range(B) if b != bstar]
    digest_before = [row_digest(t, w, l, b) for t in (dk, dv) for l in range(w.L) for b in others]
    dk.view(w.L, B, -1)[:, bstar, :].fill_(0x7E7E)
    dv.view(w.L, B, -1)[:, bstar, :].fill_(0x7E7E)
    ei.swap_in(dk, dv, 0, w.L, [0] * B, count, shost, total)
    torch.cuda.synchronize()
    # the swapped row is back in every layer: its tokens [0, len) from the
    # image, the positions past len still the sentinel; no other row changed
    n = count[bstar]
    for t, saved in ((dk, saved_k), (dv, saved_v)):
        got = t.view(w.L, B, -1)[:, bstar, :]
        if t is dk:   # K row region: [H, D/8, Smax, 8], positions on the third axis
            g4 = got.view(w.L, w.H * w.D // 8, w.Smax, 8)
            s4 = saved.view(w.L, w.H * w.D // 8, w.Smax, 8)
            assert torch.equal(g4[:, :, :n], s4[:, :, :n]), "row swap-in K, tokens"
            assert bool((g4[:, :, n:] == 0x7E7E).all()), "row swap-in K wrote past len"
        else:         # V row region: [H, Smax, D]
            g3 = got.view(w.L, w.H, w.Smax, w.D)
            s3 = saved.view(w.L, w.H, w.Smax, w.D)
            assert torch.equal(g3[:, :, :n], s3[:, :, :n]), "row swap-in V, tokens"
            assert bool((g3[:, :, n:] == 0x7E7E).all()), "row swap-in V wrote past len"
    del saved_k, saved_v
    digest_after = [row_digest(t, w, l, b) for t in (dk, dv) for l in range(w.L) for b in others]
    assert digest_after == digest_before, "row swap-in touched another row"
    for l in (0, 31, 59):
        K1, V1 = host_layer(l)
        ek = K1.copy().reshape(B, -1)
        ev = V1.copy().reshape(B, -1)
        ek[bstar] = 0x7E7E
        ev[bstar] = 0x7E7E
        ek, ev = ek.reshape(-1), ev.reshape(-1)
        oracle.unpack(one_layer(w), ek, ev, 0, 1, [0] * B, count, sv[l * per:(l + 1) * per])
        assert np.array_equal(layer_host(dk, w, l), ek), f"row swap-in K layer {l}"
        assert np.array_equal(layer_host(dv, w, l), ev), f"row swap-in V layer {l}"
    eo.close()
    ei.close()
