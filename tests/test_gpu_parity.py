"""HIP path vs the oracle, bit for bit, at sizes the oracle finishes in seconds.

Every comparison is element by element (np.array_equal on raw 16-bit words).
Shapes span several token tiles with ragged tails, every compiled head-dim
variant (D/8 = 1, 2, 3 (generic), 4, 8, 16, 32, 64, 128), empty rows, rows at
the end of the cache, random bit patterns (NaN payloads, Inf, +-0, subnormals)
and both kernels (few tokens per row and tiled).  Canaries after every staging
buffer and sentinels around every unpacked region check that nothing outside
the defined bytes is written.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import dev, empty, host, note, pinned, pinned_host_view

pytestmark = pytest.mark.gpu

CANARY = 64   # words after every staging buffer


@pytest.fixture(scope="module")
def kv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    import kv_cache_streaming_amd as kv
    return kv


def random_ranges(rng, B, S, max_count=None):
    start = rng.integers(0, S, size=B)
    count = []
    for s in start:
        hi = S - int(s)
        if max_count is not None:
            hi = min(hi, max_count)
        count.append(int(rng.integers(0, hi + 1)))
    return [int(x) for x in start], count


def check_pack_unpack(kv, dims, l0, nl, start, count, seed, bits=True, dtype=0):
    import torch
    L, B, H, D, S = dims
    note(f"pack/unpack dims={dims} layers=[{l0},+{nl}) start={start} count={count} seed={seed}")
    K, V = synth.cache_pair(dims, seed, dtype=dtype, bits=bits)
    lay = kv.kv_layout_init(L, B, H, D, S, dtype)
    dk, dv = dev(K), dev(V)
    want = oracle.pack(dims, K, V, l0, nl, start, count)
    assert kv.kv_pack_bytes(lay, nl, count) == want.nbytes
    st = empty(want.size, CANARY)
    kv.kv_pack_tokens(lay, dk, dv, l0, nl, start, count, st, want.nbytes)
    torch.cuda.synchronize()
    got = host(st)
    assert np.array_equal(got[:want.size], want), "pack differs from the oracle"
    assert np.all(got[want.size:] == 0x7A7A), "pack wrote past kv_pack_bytes"
    assert np.array_equal(host(dk), K) and np.array_equal(host(dv), V), "pack wrote a cache"
    # unpack into sentinel caches; the oracle does the same on host copies
    sk = np.full(K.size, 0xC3C3, np.uint16)
    sv = np.full(V.size, 0x3C3C, np.uint16)
    ek, ev = sk.copy(), sv.copy()
    oracle.unpack(dims, ek, ev, l0, nl, start, count, want)
    dk2, dv2 = dev(sk), dev(sv)
    kv.kv_unpack_tokens(lay, dk2, dv2, l0, nl, start, count, st, want.nbytes)
    torch.cuda.synchronize()
    assert np.array_equal(host(dk2), ek) and np.array_equal(host(dv2), ev), "unpack differs"
    assert np.array_equal(host(st)[:want.size], want), "unpack wrote its staging input"


@pytest.mark.parametrize("D", [8, 16, 24, 32, 64, 72, 96, 128, 200, 256, 320, 512, 776, 1024])
def test_tiled_ranges_every_head_dim(kv, D):
    """Multi-token ranges (tile kernel), several tiles and a ragged tail per row.
    Head sizes of 9, 12, 25, 40 and 97 vectors take the kernels' generic
    variants (one vector per thread up to 32 vectors, four above), whose
    tiles do not divide 256 or 1024 vectors evenly."""
    rng = np.random.default_rng(D)
    C = D // 8
    tile = max(1, 1024 // C)
    S = 2 * tile + 37 if D <= 256 else 3 * tile + 5
    dims = (3, 3, 2, D, S)
    start = [0, 5, S - (tile + 11)]
    count = [S, min(tile + 29, S - 5), tile + 11]
    check_pack_unpack(kv, dims, 1, 2, start, count, seed=D)
    for it in range(3):
        st, ct = random_ranges(rng, 3, S)
        ct[0] = max(ct[0], 9)        # keep the tile kernel selected
        st[0] = min(st[0], S - ct[0])
        check_pack_unpack(kv, dims, 0, 3, st, ct, seed=D * 10 + it)


@pytest.mark.parametrize("D", [8, 16, 24, 64, 96, 128, 320, 1024])
def test_few_tokens_every_head_dim(kv, D):
    """Decode-like ranges (at most 8 tokens per row: the small kernel)."""
    rng = np.random.default_rng(100 + D)
    dims = (4, 5, 3, D, 40)
    for it in range(4):
        st, ct = random_ranges(rng, 5, 40, max_count=8)
        check_pack_unpack(kv, dims, 0, 4, st, ct, seed=200 + D + it)
    # one token per row at the last position
    check_pack_unpack(kv, dims, 0, 4, [39] * 5, [1] * 5, seed=7)


def test_empty_and_degenerate(kv):
    import torch
    dims = (2, 3, 2, 16, 12)
    check_pack_unpack(kv, dims, 0, 2, [0, 0, 0], [0, 12, 0], seed=1)
    check_pack_unpack(kv, dims, 1, 1, [11, 0, 5], [1, 0, 7], seed=2)
    # zero layers and zero tokens enqueue nothing and succeed
    L, B, H, D, S = dims
    lay = kv.kv_layout_init(L, B, H, D, S, 0)
    K, V = synth.cache_pair(dims, 3)
    dk, dv = dev(K), dev(V)
    st = empty(16)
    kv.kv_pack_tokens(lay, dk, dv, 0, 0, [0] * B, [1] * B, st, 32)
    kv.kv_pack_tokens(lay, dk, dv, 0, 2, [0] * B, [0] * B, st, 32)
    torch.cuda.synchronize()
    assert np.all(host(st) == 0x7A7A)


def test_empty_rows_around_the_moved_ones(kv):
    """The grids cover only the rows from the first to the last that move a
    token: empty rows before, inside and after that span, over several
    layers, with the tile kernel and the few-token kernel (D/8 = 3, the
    generic variant)."""
    dims = (3, 9, 3, 24, 80)
    z = [0] * 9
    check_pack_unpack(kv, dims, 0, 3, [0, 0, 5, 0, 7, 0, 0, 0, 0],
                      [0, 0, 70, 0, 33, 0, 0, 0, 0], seed=31)
    check_pack_unpack(kv, dims, 0, 3, [3] + z[1:], [77] + z[1:], seed=32)       # first row only
    check_pack_unpack(kv, dims, 1, 2, z[:8] + [79], z[:8] + [1], seed=33)      # last row only
    check_pack_unpack(kv, dims, 0, 3, [0, 10, 0, 0, 0, 0, 0, 20, 0],
                      [0, 4, 0, 0, 0, 0, 0, 8, 0], seed=34)
    check_pack_unpack(kv, dims, 2, 1, z[:4] + [60] + z[5:], z[:4] + [20] + z[5:], seed=35)


@pytest.mark.parametrize("D", [16, 24, 128, 1024])
def test_ragged_rows_both_tile_grids(kv, D):
    """Rows of very different lengths (a grid of the rows' own tiles: one row
    of 2000 tokens beside rows of 10-40 and an empty one) and nearly equal
    ones (the dense grid), over several layers and head dims."""
    dims = (3, 5, 3, D, 2100)
    check_pack_unpack(kv, dims, 0, 3, [50, 7, 0, 300, 2000], [2000, 10, 0, 40, 17], seed=41)
    check_pack_unpack(kv, dims, 1, 2, [0, 3, 9, 1, 2], [1500, 1490, 1497, 1500, 1466], seed=42)


@pytest.mark.parametrize("S", [512, 520])
@pytest.mark.parametrize("base", [0, 1664])
def test_value_runs_on_cache_pages(kv, S, base):
    """Rows that start in mid-page of the value cache: rows a whole number
    of 4 KiB pages long (Smax = 512, D = 128) or with the page offset moving
    from head to head (Smax = 520), a value cache that is a view based on a
    page boundary or 1664 bytes past one, dense and ragged grids; pack and
    unpack against the oracle, and nothing outside the cache view written."""
    import torch
    dims = (2, 4, 3, 128, S)
    L, B, H, D, _ = dims
    lay = kv.kv_layout_init(L, B, H, D, S, 0)
    for seed, start, count in ((51, [5, 100, 17, 0], [400, 300, 411, 500]),
                               (52, [3, 0, 250, 9], [500, 0, 7, 260])):
        note(f"value runs S={S} base={base} start={start} count={count}")
        K, V = synth.cache_pair(dims, seed)
        want = oracle.pack(dims, K, V, 0, L, start, count)
        dk = dev(K)
        # the value cache as a view starting `base` bytes past a 4 KiB boundary
        vbuf = torch.empty(V.size + 4096, dtype=torch.int16, device="cuda")
        off = ((base - vbuf.data_ptr()) % 4096) // 2     # int16 words
        assert (vbuf.data_ptr() + 2 * off) % 4096 == base
        dv = vbuf[off:off + V.size]
        dv.copy_(torch.from_numpy(V.view(np.int16)))
        st = empty(want.size, CANARY)
        kv.kv_pack_tokens(lay, dk, dv, 0, L, start, count, st, want.nbytes)
        torch.cuda.synchronize()
        assert np.array_equal(host(st)[:want.size], want), "pack differs from the oracle"
        sk, sv = np.full(K.size, 0xC3C3, np.uint16), np.full(V.size, 0x3C3C, np.uint16)
        ek, ev = sk.copy(), sv.copy()
        oracle.unpack(dims, ek, ev, 0, L, start, count, want)
        dk2 = dev(sk)
        vbuf.fill_(0x3C3C)
        kv.kv_unpack_tokens(lay, dk2, vbuf[off:off + V.size], 0, L, start, count, st,
                            want.nbytes)
        torch.cuda.synchronize()
        got_v = host(vbuf)
        assert np.array_equal(host(dk2), ek), "unpack: key cache differs"
        assert np.array_equal(got_v[off:off + V.size], ev), "unpack: value cache differs"
        assert np.all(got_v[:off] == 0x3C3C) and np.all(got_v[off + V.size:] == 0x3C3C), \
            "unpack wrote outside the value cache"


def test_maximum_rows(kv):
    """KV_MAX_ROWS = 256 rows in one call (the row table travels in the kernel
    arguments): ragged and empty rows with the tile kernel, one token per row
    with the small kernel, and a ring of 256-row decode steps gathered at
    flush."""
    rng = np.random.default_rng(256)
    dims = (2, kv.KV_MAX_ROWS, 2, 16, 40)
    L, B, H, D, S = dims
    st, ct = random_ranges(rng, B, S)
    ct[0], st[0] = S, 0
    ct[1], ct[2] = 0, 9
    st[2] = min(st[2], S - 9)
    check_pack_unpack(kv, dims, 0, L, st, ct, seed=256)
    check_pack_unpack(kv, dims, 1, 1, [int(x) for x in rng.integers(0, S, size=B)], [1] * B,
                      seed=257)
    pos = [[int(p0) + j for p0 in rng.integers(0, S - 10, size=B)] for j in range(10)]
    for j in range(1, 10):
        pos[j] = [p + j for p in pos[0]]
    run_ring(kv, dims, 4, pos, seed=258, gather=1)


def test_fp16_and_bf16_values(kv):
    dims = (2, 2, 3, 64, 300)
    check_pack_unpack(kv, dims, 0, 2, [0, 17], [300, 250], seed=5, bits=False, dtype=0)
    check_pack_unpack(kv, dims, 0, 2, [3, 0], [290, 300], seed=6, bits=False, dtype=1)


def test_prompt_layer_chunks(kv):
    import torch
    dims = (3, 4, 2, 32, 700)
    L, B, H, D, S = dims
    note(f"prompt chunks dims={dims}")
    K, V = synth.cache_pair(dims, 11)
    lay = kv.kv_layout_init(L, B, H, D, S, 0)
    dk, dv = dev(K), dev(V)
    row_len = [700, 123, 0, 333]
    chunk = 256
    for layer in range(L):
        for tb in range(0, S, chunk):
            tc = min(chunk, S - tb)
            start, count = oracle.prompt_ranges(B, tb, tc, row_len)
            want = oracle.pack(dims, K, V, layer, 1, start, count)
            st = empty(max(want.size, 1), CANARY)
            kv.kv_pack_prompt_layer(lay, dk, dv, layer, tb, tc, row_len, st, want.nbytes)
            torch.cuda.synchronize()
            got = host(st)
            assert np.array_equal(got[:want.size], want)
            assert np.all(got[max(want.size, 1):] == 0x7A7A)
            # unpack the chunk back into a sentinel cache
            ek = np.full(K.size, 0x1111, np.uint16)
            ev = np.full(V.size, 0x2222, np.uint16)
            dk2, dv2 = dev(ek), dev(ev)
            oracle.unpack(dims, ek, ev, layer, 1, start, count, want)
            kv.kv_unpack_prompt_layer(lay, dk2, dv2, layer, tb, tc, row_len, st, want.nbytes)
            torch.cuda.synchronize()
            assert np.array_equal(host(dk2), ek) and np.array_equal(host(dv2), ev)


@pytest.mark.parametrize("nbytes", [16, 4096, 4096 + 16, (1 << 20) + 48, 300 << 20])
def test_copy_packed_moves_every_byte(kv, nbytes):
    """kv_copy_packed is a plain copy: the destination equals the source
    bit for bit, and nothing past the destination range is written
    (sizes below, at and just past one workgroup's 4 KiB, and a 300 MiB
    block of many workgroups)."""
    import torch
    note(f"copy_packed {nbytes} bytes")
    words = nbytes // 2
    src = dev(synth.random_bits(words, 600 + nbytes % 997))
    dst = empty(words, extra=CANARY)
    kv.kv_copy_packed(dst, src, nbytes)
    torch.cuda.synchronize()
    got = host(dst)
    assert np.array_equal(got[:words], host(src)), "copy differs from its source"
    assert np.all(got[words:] == 0x7A7A), "copy wrote past its destination"


def test_copy_packed_refuses_bad_buffers(kv):
    """Overlapping ranges, a misaligned address and pageable host memory are
    refused before anything is enqueued (the range-inside-one-allocation
    check is the one every entry point shares; its test is below)."""
    import torch
    a = empty(1024)
    with pytest.raises(kv.KvError) as e:          # overlapping ranges of one buffer
        kv.kv_copy_packed(a[256:], a, 1024)
    assert e.value.status == kv.KV_EINVAL
    with pytest.raises(kv.KvError) as e:          # misaligned destination
        kv.kv_copy_packed(a.data_ptr() + 8, a.data_ptr() + 1024, 512)
    assert e.value.status == kv.KV_EINVAL
    h = np.zeros(512, np.uint16)                  # pageable host memory
    with pytest.raises(kv.KvError) as e:
        kv.kv_copy_packed(a, h.ctypes.data, 1024)
    assert e.value.status == kv.KV_EINVAL
    torch.cuda.synchronize()
    assert np.all(host(a) == 0x7A7A), "a refused copy wrote"


def test_error_paths(kv):
    import torch
    dims = (2, 2, 2, 16, 8)
    L, B, H, D, S = dims
    lay = kv.kv_layout_init(L, B, H, D, S, 0)
    K, V = synth.cache_pair(dims, 1)
    dk, dv = dev(K), dev(V)
    st = empty(4096)
    pageable = np.zeros(8192, np.uint16)
    note("error paths")
    with pytest.raises(kv.KvError) as e:                    # host array passed as a cache
        kv.kv_pack_tokens(lay, pageable, dv, 0, 1, [0, 0], [1, 1], st, 8192)
    assert e.value.status == kv.KV_EINVAL
    with pytest.raises(kv.KvError) as e:                    # misaligned staging
        kv.kv_pack_tokens(lay, dk, dv, 0, 1, [0, 0], [1, 1], st.data_ptr() + 2, 4096)
    assert e.value.status == kv.KV_EINVAL
    with pytest.raises(kv.KvError) as e:                    # staging overlapping the key cache
        kv.kv_pack_tokens(lay, dk, dv, 0, 1, [0, 0], [1, 1], dk, 4096)
    assert e.value.status == kv.KV_EINVAL
    with pytest.raises(kv.KvError) as e:                    # short staging
        kv.kv_pack_tokens(lay, dk, dv, 0, 1, [0, 0], [2, 2], st, 255)
    assert e.value.status == kv.KV_ESIZE
    with pytest.raises(kv.KvError) as e:                    # position >= Smax
        kv.kv_pack_tokens(lay, dk, dv, 0, 1, [8, 0], None, st, 8192)
    assert e.value.status == kv.KV_ERANGE
    torch.cuda.synchronize()
    assert np.all(host(st) == 0x7A7A), "a rejected call wrote staging"
    # swap engine: pageable host image, short host image
    b0, b1 = empty(512), empty(512)
    eng = kv.KvSwap(lay, b0, b1, 1024)
    with pytest.raises(kv.KvError) as e:
        eng.swap_out(dk, dv, 0, 2, [0, 0], [4, 4], pageable, pageable.nbytes)
    assert e.value.status == kv.KV_EINVAL
    hp = pinned(64)
    with pytest.raises(kv.KvError) as e:
        eng.swap_out(dk, dv, 0, 2, [0, 0], [4, 4], hp, 128)
    assert e.value.status == kv.KV_ESIZE
    with pytest.raises(kv.KvError) as e:                    # a bank aliasing the cache
        kv.KvSwap(lay, dk, b1, 512).swap_out(dk, dv, 0, 1, [0, 0], [1, 1], pinned(4096), 8192)
    assert e.value.status == kv.KV_EINVAL
    # ring: restore before flush, full host image, bad position
    slot = kv.kv_pack_bytes(lay, L, None, 1)
    rb0, rb1 = empty(2 * slot // 2), empty(2 * slot // 2)
    rh = pinned(3 * slot // 2)
    ring = kv.KvRing(lay, 2, rb0, rb1, rh)
    ring.push(dk, dv, [0, 1])
    with pytest.raises(kv.KvError) as e:
        ring.restore(dk, dv)
    assert e.value.status == kv.KV_EBUSY
    with pytest.raises(kv.KvError) as e:
        ring.push(dk, dv, [0, 8])
    assert e.value.status == kv.KV_ERANGE
    ring.push(dk, dv, [1, 2])
    ring.push(dk, dv, [2, 3])
    with pytest.raises(kv.KvError) as e:
        ring.push(dk, dv, [3, 4])
    assert e.value.status == kv.KV_ESIZE
    ring.flush()
    torch.cuda.synchronize()
    assert ring.steps == 3


TRANSPORTS = [0, 1, 2, 3, 4, 5]   # KV_XFER_AUTO, _KERNEL, _RUNTIME, _DMA, _DMA_OUT, _ENGINE


def run_ring(kv, dims, R, positions, seed, bits=True, mutate=False, delay_cycles=0, transport=0,
             gather=0, caches=1, options=()):
    """Push every step, flush, restore into a zero cache; compare with the oracle.
    `caches` > 1: step j reads cache pair (j // 3) % caches (runs of three steps
    per cache)."""
    import torch
    L, B, H, D, S = dims
    note(f"ring dims={dims} R={R} steps={len(positions)} mutate={mutate} delay={delay_cycles} "
         f"transport={transport} gather={gather} caches={caches}")
    pairs = [synth.cache_pair(dims, seed + 1000 * i, bits=bits) for i in range(caches)]
    K, V = pairs[0]
    lay = kv.kv_layout_init(L, B, H, D, S, 0)
    devs = [(dev(a), dev(b)) for a, b in pairs]
    dk, dv = devs[0]
    slot = kv.kv_pack_bytes(lay, L, None, 1)
    banks = [empty(R * slot // 2), empty(R * slot // 2)]
    steps = len(positions)
    hostbuf = pinned(steps * slot // 2 + CANARY)
    copy = torch.cuda.Stream()
    compute = torch.cuda.current_stream()
    ring = kv.KvRing(lay, R, banks[0], banks[1], hostbuf, host_bytes=steps * slot,
                     copy_stream=copy, transport=transport)
    if gather:
        ring.set_gather(kv.KV_RING_GATHER_AT_FLUSH)
    for opt, val in options:
        ring.set_option(opt, val)
    slots = []
    rng = np.random.default_rng(seed)
    if delay_cycles:
        with torch.cuda.stream(copy):
            torch.cuda._sleep(delay_cycles)   # a bounded spin: makes every flush copy late
    for j, pos in enumerate(positions):
        ci = (j // 3) % caches
        slots.append(oracle.pack(dims, pairs[ci][0], pairs[ci][1], 0, L, pos, [1] * B))
        ring.push(devs[ci][0], devs[ci][1], pos, compute)
        if mutate:
            assert caches == 1 and not gather
            # the cache changes between steps (new values at random places)
            idx = rng.integers(0, K.size, size=64)
            K[idx] = rng.integers(0, 1 << 16, size=64).astype(np.uint16)
            V[idx] = rng.integers(0, 1 << 16, size=64).astype(np.uint16)
            dk.copy_(torch.from_numpy(K.view(np.int16)).cuda(), non_blocking=False)
            dv.copy_(torch.from_numpy(V.view(np.int16)).cuda(), non_blocking=False)
    done = torch.cuda.Event()
    ring.flush(compute, done)
    done.synchronize()
    want_host = oracle.ring_host(slots)
    got_host = pinned_host_view(hostbuf)
    assert np.array_equal(got_host[:want_host.size], want_host), "ring host image differs"
    assert np.all(got_host[want_host.size:] == 0x5C5C), "ring wrote past its steps"
    zk, zv = np.zeros(K.size, np.uint16), np.zeros(V.size, np.uint16)
    rk, rv = dev(zk), dev(zv)
    oracle.ring_restore(dims, zk, zv, positions, want_host)
    ring.restore(rk, rv, compute)
    torch.cuda.synchronize()
    assert np.array_equal(host(rk), zk) and np.array_equal(host(rv), zv), "restore differs"
    ring.close()


@pytest.mark.parametrize("gather", [0, 1])
@pytest.mark.parametrize("transport", TRANSPORTS)
def test_ring_decode_flow(kv, transport, gather):
    dims = (3, 4, 2, 64, 50)
    pos = [[10 + j, 20 + j, 3 + j, 40 + (j % 9)] for j in range(19)]   # 2 full banks + a partial
    run_ring(kv, dims, 8, pos, seed=21, transport=transport, gather=gather)


@pytest.mark.parametrize("transport,opt,val", [(5, 1, 0), (5, 1, 3), (0, 2, 2)])
def test_ring_link_options(kv, transport, opt, val):
    dims = (3, 4, 2, 64, 50)
    pos = [[10 + j, 20 + j, 3 + j, 40 + (j % 9)] for j in range(19)]
    run_ring(kv, dims, 8, pos, seed=22, transport=transport, options=[(opt, val)])


@pytest.mark.parametrize("D,R,steps", [(128, 16, 37), (8, 5, 12), (24, 7, 15), (1024, 4, 9)])
def test_ring_gather_at_flush_runs(kv, D, R, steps):
    """Gather at flush: runs of consecutive positions packed in one pass, broken
    by a position jump (row 1 at step 6) and by the cache changing every three
    steps; the host image and the restore equal the per-step oracle."""
    dims = (2, 3, 2, D, 60)
    pos = [[j, 10 + j + (5 if j >= 6 else 0), 17 if j % 4 == 3 else 2 + j]
           for j in range(steps)]
    run_ring(kv, dims, R, pos, seed=24, gather=1, caches=2)


@pytest.mark.parametrize("gather", [0, 1])
@pytest.mark.parametrize("D,R,steps", [(1024, 16, 21), (512, 20, 23)])
def test_ring_wide_units_past_the_lds_pass(kv, D, R, steps, gather):
    """Runs of steps whose unit holds more than 1024 vectors (16 steps of a
    128-vector head, 20 of a 64-vector one) take the per-vector step kernel
    instead of the LDS pass: gathered at flush, and unpacked in runs by the
    restore in both gather modes."""
    dims = (2, 3, 2, D, 48)
    pos = [[j, 5 + j, 20 + j] for j in range(steps)]
    run_ring(kv, dims, R, pos, seed=27 + D, gather=gather)


@pytest.mark.parametrize("D", [8, 24, 64, 128])
def test_ring_gather_at_flush_many_units(kv, D):
    """Gather at flush over 105 (layer, row, head) units at ragged row
    positions: heads of 1, 3, 8 and 16 vectors, so a flush of 8 steps moves
    8-128 vectors per unit and the gather groups several units per wave with
    a partial last group; the 19 steps end in a partial bank of 3."""
    dims = (3, 5, 7, D, 40)
    pos = [[(7 * b) % 20 + j for b in range(5)] for j in range(19)]
    run_ring(kv, dims, 8, pos, seed=26, gather=1)


def test_ring_gather_at_flush_partial_flushes(kv):
    """Explicit flushes in the middle of a bank: the pending steps are gathered
    then, and later steps continue in the same bank."""
    import torch
    dims = (2, 2, 2, 64, 40)
    L, B, H, D, S = dims
    note(f"ring gather-at-flush with partial flushes dims={dims}")
    K, V = synth.cache_pair(dims, 25, bits=True)
    lay = kv.kv_layout_init(L, B, H, D, S, 0)
    dk, dv = dev(K), dev(V)
    slot = kv.kv_pack_bytes(lay, L, None, 1)
    R, steps = 6, 14
    hostbuf = pinned(steps * slot // 2 + CANARY)
    ring = kv.KvRing(lay, R, empty(R * slot // 2), empty(R * slot // 2), hostbuf,
                     host_bytes=steps * slot, copy_stream=torch.cuda.Stream())
    ring.set_gather(kv.KV_RING_GATHER_AT_FLUSH)
    pos = [[3 + j, 20 + j] for j in range(steps)]
    for j in range(steps):
        ring.push(dk, dv, pos[j])
        if j == 2:
            with pytest.raises(kv.KvError) as e:      # a pending step: the mode is fixed until a flush
                ring.set_gather(kv.KV_RING_GATHER_EACH_STEP)
            assert e.value.status == kv.KV_EBUSY
        if j in (1, 4, 9):
            ring.flush()
    done = torch.cuda.Event()
    ring.flush(None, done)
    done.synchronize()
    assert ring.steps == steps
    want = oracle.ring_host([oracle.pack(dims, K, V, 0, L, p, [1] * B) for p in pos])
    got = pinned_host_view(hostbuf)
    assert np.array_equal(got[:want.size], want)
    assert np.all(got[want.size:] == 0x5C5C)
    ring.set_gather(kv.KV_RING_GATHER_EACH_STEP)      # everything flushed: allowed
    ring.close()


@pytest.mark.parametrize("transport", TRANSPORTS)
def test_ring_duplicate_positions_last_writer_wins(kv, transport):
    dims = (2, 3, 3, 16, 6)
    pos = [[j % 6, (2 * j) % 6, 5] for j in range(11)]
    run_ring(kv, dims, 4, pos, seed=22, mutate=True, transport=transport)


def test_ring_restore_runs_keep_the_last_writer(kv):
    """Runs of consecutive positions that revisit earlier positions (each row
    cycles through 0..5): the restore applies runs in step order."""
    dims = (2, 2, 2, 64, 6)
    pos = [[j % 6, (j + 3) % 6] for j in range(17)]
    run_ring(kv, dims, 8, pos, seed=26, gather=1)


@pytest.mark.parametrize("transport", TRANSPORTS)
def test_ring_bank_reuse_waits_for_a_late_flush(kv, transport):
    """The copy stream is held back by a bounded spin; a push that reuses a bank
    must still wait for that bank's copy (else the host image would differ)."""
    dims = (2, 2, 2, 32, 64)
    pos = [[j, 63 - j] for j in range(13)]
    run_ring(kv, dims, 2, pos, seed=23, mutate=True, delay_cycles=200_000_000,
             transport=transport)


def test_ring_gather_at_flush_waits_for_a_late_flush(kv):
    dims = (2, 2, 2, 32, 64)
    pos = [[j, 40 + j] for j in range(13)]
    run_ring(kv, dims, 2, pos, seed=27, delay_cycles=200_000_000, gather=1)


def run_swap(kv, dims, l0, nl, start, count, bank_bytes, seed, delay_cycles=0, transport=0,
             options=()):
    import torch
    L, B, H, D, S = dims
    note(f"swap dims={dims} layers=[{l0},+{nl}) bank={bank_bytes} delay={delay_cycles} "
         f"transport={transport} options={options}")
    K, V = synth.cache_pair(dims, seed, bits=True)
    lay = kv.kv_layout_init(L, B, H, D, S, 0)
    dk, dv = dev(K), dev(V)
    want = oracle.pack(dims, K, V, l0, nl, start, count)
    b0, b1 = empty(bank_bytes // 2 + 8), empty(bank_bytes // 2 + 8)
    copy = torch.cuda.Stream()
    compute = torch.cuda.current_stream()
    eng = kv.KvSwap(lay, b0, b1, bank_bytes, copy, transport)
    for opt, val in options:
        eng.set_option(opt, val)
    hostbuf = pinned(want.size + CANARY)
    if delay_cycles:
        with torch.cuda.stream(copy):
            torch.cuda._sleep(delay_cycles)
    done = torch.cuda.Event()
    eng.swap_out(dk, dv, l0, nl, start, count, hostbuf, want.nbytes, compute, done)
    # overwrite the source cache right away on compute: the packs precede it there
    dk.fill_(0)
    dv.fill_(0)
    done.synchronize()
    got = pinned_host_view(hostbuf)
    assert np.array_equal(got[:want.size], want), "swap-out host image differs"
    assert np.all(got[want.size:] == 0x5C5C)
    # swap-in into sentinel caches
    ek = np.full(K.size, 0x4444, np.uint16)
    ev = np.full(V.size, 0x5555, np.uint16)
    dk2, dv2 = dev(ek), dev(ev)
    oracle.unpack(dims, ek, ev, l0, nl, start, count, want)
    if delay_cycles:
        with torch.cuda.stream(copy):
            torch.cuda._sleep(delay_cycles)
    done2 = torch.cuda.Event()
    eng.swap_in(dk2, dv2, l0, nl, start, count, hostbuf, want.nbytes, compute, done2)
    done2.synchronize()
    assert np.array_equal(host(dk2), ek) and np.array_equal(host(dv2), ev), "swap-in differs"
    eng.close()


@pytest.mark.parametrize("transport,opt,val", [
    (0, 2, 1), (0, 2, 3), (0, 2, 200), (1, 2, 12), (5, 1, 0), (5, 1, 2), (5, 1, 3), (5, 1, -1),
    (5, 2, 5)])
def test_swap_link_options(kv, transport, opt, val):
    """Per-handle link settings (KV_OPT_LINK_BLOCKS: 1, 3, 200 or 12
    link-copy workgroups; KV_OPT_DMA_ENGINE: engine 0, 2, 3 or an idle one)
    move the same bytes: row-group chunks, late copies."""
    dims = (3, 5, 2, 128, 260)
    count = [260, 0, 100, 255, 3]
    start = [0, 0, 160, 5, 257]
    per_row = [2 * 2 * 128 * 2 * c for c in count]
    run_swap(kv, dims, 0, 3, start, count, max(per_row) + 4096, seed=34,
             delay_cycles=50_000_000, transport=transport, options=[(opt, val)])


def test_link_options_rejected(kv):
    import torch
    dims = (2, 2, 2, 64, 16)
    lay = kv.kv_layout_init(*dims, 0)
    note("link option errors")
    eng = kv.KvSwap(lay, empty(4096), empty(4096), 8192, torch.cuda.Stream(), kv.KV_XFER_AUTO)
    for opt, val in ((kv.KV_OPT_DMA_ENGINE, 0), (kv.KV_OPT_LINK_BLOCKS, -1),
                     (kv.KV_OPT_LINK_BLOCKS, 1025), (99, 1)):
        with pytest.raises(kv.KvError) as ei:
            eng.set_option(opt, val)
        assert ei.value.status == kv.KV_EINVAL
    eng.close()
    eng = kv.KvSwap(lay, empty(4096), empty(4096), 8192, torch.cuda.Stream(), kv.KV_XFER_ENGINE)
    for val in (-2, 4):
        with pytest.raises(kv.KvError) as ei:
            eng.set_option(kv.KV_OPT_DMA_ENGINE, val)
        assert ei.value.status == kv.KV_EINVAL
    eng.close()


@pytest.mark.parametrize("transport", TRANSPORTS)
def test_swap_whole_layer_chunks(kv, transport):
    dims = (6, 3, 2, 64, 300)
    layer = 2 * 2 * 64 * 2 * (300 + 250 + 17)
    run_swap(kv, dims, 1, 5, [0, 50, 283], [300, 250, 17], 2 * layer, seed=31,
             transport=transport)


@pytest.mark.parametrize("transport", TRANSPORTS)
def test_swap_row_group_chunks(kv, transport):
    dims = (3, 5, 2, 128, 260)
    count = [260, 0, 100, 255, 3]
    start = [0, 0, 160, 5, 257]
    per_row = [2 * 2 * 128 * 2 * c for c in count]
    run_swap(kv, dims, 0, 3, start, count, max(per_row) + 4096, seed=32, transport=transport)


@pytest.mark.parametrize("transport", TRANSPORTS)
def test_swap_waits_for_late_copies(kv, transport):
    dims = (8, 2, 2, 32, 128)
    layer = 2 * 2 * 32 * 2 * 256
    run_swap(kv, dims, 0, 8, [0, 0], [128, 128], layer, seed=33, delay_cycles=200_000_000,
             transport=transport)


@pytest.mark.parametrize("transport", TRANSPORTS)
def test_stream_prompt_layers(kv, transport):
    import torch
    dims = (4, 3, 2, 64, 200)
    L, B, H, D, S = dims
    note(f"prompt streamer dims={dims}")
    K, V = synth.cache_pair(dims, 41)
    lay = kv.kv_layout_init(L, B, H, D, S, 0)
    dk, dv = dev(K), dev(V)
    row_len = [200, 150, 77]
    start, count = oracle.prompt_ranges(B, 0, 180, row_len)
    per_layer = oracle.pack(dims, K, V, 0, 1, start, count).size
    b0, b1 = empty(per_layer), empty(per_layer)
    copy = torch.cuda.Stream()
    eng = kv.KvSwap(lay, b0, b1, per_layer * 2, copy, transport)
    hostbuf = pinned(L * per_layer + CANARY)
    hv = pinned_host_view(hostbuf)
    done = torch.cuda.Event()
    for layer in range(L):
        dst = hostbuf.data_ptr() + layer * per_layer * 2
        eng.stream_prompt_layer(dk, dv, layer, 0, 180, row_len, dst, per_layer * 2,
                                torch.cuda.current_stream(), done)
    done.synchronize()
    for layer in range(L):
        want = oracle.pack(dims, K, V, layer, 1, start, count)
        assert np.array_equal(hv[layer * per_layer:(layer + 1) * per_layer], want)
    assert np.all(hv[L * per_layer:] == 0x5C5C)


def test_profiler_counts_launches(kv):
    import torch
    dims = (2, 2, 2, 64, 128)
    K, V = synth.cache_pair(dims, 51)
    lay = kv.kv_layout_init(*dims, 0)
    dk, dv = dev(K), dev(V)
    st = empty(2 * 2 * 2 * 64 * 256)
    kv.kv_profile_begin()
    kv.kv_pack_tokens(lay, dk, dv, 0, 2, [0, 0], [128, 128], st)
    kv.kv_pack_tokens(lay, dk, dv, 0, 2, [5, 9], None, st)
    kv.kv_unpack_tokens(lay, dk, dv, 0, 2, [0, 0], [128, 128], st)
    stats = kv.kv_profile_end()
    torch.cuda.synchronize()
    assert stats["pack_tiles"][0] == 1 and stats["pack_rows_small"][0] == 1
    assert stats["unpack_tiles"][0] == 1
    assert stats["pack_tiles"][2] == 2 * 2 * (2 * 2 * 2 * 64 * 256)
    assert all(v[1] > 0 for v in stats.values())
    win = kv.kv_profile_last_window()
    assert win["hbm_launches"] == 3 and win["link_launches"] == 0
    assert win["hbm_bytes"] == sum(v[2] for v in stats.values())
    total = sum(v[1] for v in stats.values())
    # one stream: the kernels follow one another, so their union is at most
    # their sum and at least the longest of them, and fits in the span
    assert max(v[1] for v in stats.values()) <= win["hbm_busy_ms"] <= total * (1 + 1e-6)
    assert win["hbm_busy_ms"] <= win["span_ms"] * (1 + 1e-6)
    assert win["link_busy_ms"] == 0.0 and win["link_bytes"] == 0


def test_profile_window_overlapping_streams(kv):
    """Two streams packing at once, and a ring flush's link copy: the window
    holds the union of the timed intervals of each class."""
    import torch
    dims = (4, 4, 4, 128, 1024)
    L, B, H, D, S = dims
    K, V = synth.cache_pair(dims, 53)
    lay = kv.kv_layout_init(*dims, 0)
    dk, dv = dev(K), dev(V)
    n = kv.kv_pack_bytes(lay, L, [S] * B)
    st = [empty(n // 2), empty(n // 2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    slot = kv.kv_pack_bytes(lay, L, None, 1)
    hostbuf = pinned(2 * slot // 2)
    ring = kv.KvRing(lay, 2, empty(2 * slot // 2), empty(2 * slot // 2), hostbuf,
                     copy_stream=torch.cuda.Stream(), transport=1)
    torch.cuda.synchronize()
    kv.kv_profile_begin()
    for i in range(3):
        for j in range(2):
            kv.kv_pack_tokens(lay, dk, dv, 0, L, [0] * B, [S] * B, st[j], stream=streams[j])
    ring.push(dk, dv, [3] * B)
    ring.push(dk, dv, [4] * B)      # fills the bank: one link copy
    stats = kv.kv_profile_end()
    torch.cuda.synchronize()
    win = kv.kv_profile_last_window()
    hbm = {k: v for k, v in stats.items() if not k.startswith("link_copy")}
    link = {k: v for k, v in stats.items() if k.startswith("link_copy")}
    assert win["hbm_launches"] == sum(v[0] for v in hbm.values()) == 8
    assert win["link_launches"] == sum(v[0] for v in link.values()) == 1
    assert win["hbm_bytes"] == sum(v[2] for v in hbm.values())
    assert win["link_bytes"] == 2 * slot
    assert max(v[1] for v in hbm.values()) / max(v[0] for v in hbm.values()) <= \
        win["hbm_busy_ms"] * (1 + 1e-6)
    assert win["hbm_busy_ms"] <= sum(v[1] for v in hbm.values()) * (1 + 1e-6)
    assert 0 < win["link_busy_ms"] <= win["span_ms"] * (1 + 1e-6)
    assert win["hbm_busy_ms"] <= win["span_ms"] * (1 + 1e-6)
    ring.close()


def test_staging_past_its_allocation_is_refused(kv):
    """A staging range that starts inside one device allocation and runs past
    its end is refused before anything is enqueued, whether the bytes past
    the end belong to another allocation or to none."""
    import ctypes
    import torch
    dims = (2, 2, 2, 64, 64)
    L, B, H, D, S = dims
    note("staging past the end of its allocation")
    lay = kv.kv_layout_init(L, B, H, D, S, 0)
    K, V = synth.cache_pair(dims, 5)
    dk, dv = dev(K), dev(V)
    lib = kv._lib
    lib.hipMalloc.restype = ctypes.c_int
    lib.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    lib.hipFree.restype = ctypes.c_int
    lib.hipFree.argtypes = [ctypes.c_void_p]
    size = 4 << 20
    bufs = []
    for _ in range(2):
        p = ctypes.c_void_p()
        assert lib.hipMalloc(ctypes.byref(p), size) == 0 and p.value
        bufs.append(p.value)
    try:
        # only where the runtime sizes allocations: without that the range
        # check falls back to the two ends, and this case must not run
        lib.hipMemGetAddressRange.restype = ctypes.c_int
        lib.hipMemGetAddressRange.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                              ctypes.POINTER(ctypes.c_size_t), ctypes.c_void_p]
        base, got = ctypes.c_void_p(), ctypes.c_size_t()
        if (lib.hipMemGetAddressRange(ctypes.byref(base), ctypes.byref(got), bufs[0]) != 0
                or base.value != bufs[0] or got.value < size):
            pytest.skip("the runtime does not report allocation ranges")
        need = kv.kv_pack_bytes(lay, L, None, S)
        assert need <= size
        start = bufs[0] + size - need // 2        # half the packed block fits, half does not
        with pytest.raises(kv.KvError) as e:
            kv.kv_pack_tokens(lay, dk, dv, 0, L, [0] * B, [S] * B, start, need)
        assert e.value.status == kv.KV_EINVAL
        msg = kv.kv_last_error()
        assert "past the end of its allocation" in msg or "not device memory" in msg, msg
        # the same call on the allocation's own range goes through
        kv.kv_pack_tokens(lay, dk, dv, 0, L, [0] * B, [S] * B, bufs[0], need)
        torch.cuda.synchronize()
    finally:
        torch.cuda.synchronize()
        for p in bufs:
            lib.hipFree(p)
