"""stream_out / stream_in between differing partitions on the GPU, bit for bit
against the oracle (DejaVu summary, DejaVuLib primitives, Table 1; Fast
prompt KV transfer).

Small shapes span several tiles with ragged tails and decode-sized ranges;
the full-size case repartitions the 16-layer OPT-66B slice (72 heads, ragged
lengths) held by one worker into 2 pipeline stages x 2 tensor-parallel ranks.
"""
import itertools

import numpy as np
import pytest

import oracle
import synth
from gpu_util import dev, empty, host, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    import kv_cache_streaming_amd as kv
    return kv


@pytest.fixture(autouse=True)
def free_memory():
    import gc

    import torch
    yield
    torch.cuda.synchronize()
    gc.collect()
    torch.cuda.empty_cache()


SMALL_DESTS = [(0, 10, 0, 10, 0, 20),     # holds all of the source
               (3, 1, 0, 2, 11, 5),       # one layer, low heads, upper rows
               (0, 3, 2, 5, 0, 11),       # high heads
               (4, 4, 3, 1, 12, 1),       # a single (layer, head, row)
               (5, 2, 0, 8, 0, 20),       # no shared layer: empty piece
               (2, 3, 0, 8, 9, 2)]        # rows straddling the source's first row


@pytest.mark.parametrize("D,S,counts", [(64, 700, "tiles"), (128, 300, "tiles"),
                                        (24, 200, "tiles"), (320, 180, "tiles"),
                                        (64, 40, "decode")])
def test_pieces_and_merge_small(kv, D, S, counts):
    import torch
    src = (2, 3, 1, 3, 10, 3)
    dims = oracle.part_dims(src, D, S)
    note(f"stream_out/in src={src} D={D} S={S} {counts}")
    lay = kv.kv_layout_init(*dims, 0)
    K, V = synth.cache_pair(dims, 41 + D, bits=True)
    dk, dv = dev(K), dev(V)
    rng = np.random.default_rng(D + S)
    if counts == "tiles":
        count = np.array([S - 3, 129, 0], np.int32)
        start = np.array([1, int(rng.integers(0, S - 129)), 5], np.int32)
    else:
        count = np.array([1, 2, 1], np.int32)
        start = np.array([S - 1, 7, 0], np.int32)
    for dst in SMALL_DESTS:
        want = oracle.stream_out(src, dst, D, S, K, V, start, count)
        nbytes = kv.kv_stream_bytes(lay, src, dst, count)
        assert nbytes == want.size * 2
        st = empty(want.size, extra=64)
        kv.kv_stream_out(lay, src, dk, dv, dst, start, count, st, nbytes)
        torch.cuda.synchronize()
        got = host(st)
        assert np.array_equal(got[:want.size], want), f"piece for {dst}"
        assert np.all(got[want.size:] == 0x7A7A), "wrote past the piece"
        # merge into the destination's own cache: its rows keep the source's
        # counts and start one token later where they fit
        ddims = oracle.part_dims(dst, D, S)
        if want.size == 0 or np.prod(ddims) > 40_000_000:
            continue
        dlay = kv.kv_layout_init(*ddims, 0)
        dstart = np.zeros(dst[5], np.int32)
        dcount = np.zeros(dst[5], np.int32)
        for gr in range(max(src[4], dst[4]), min(src[4] + src[5], dst[4] + dst[5])):
            b, bd = gr - src[4], gr - dst[4]
            dcount[bd] = count[b]
            dstart[bd] = start[b] + (1 if start[b] + count[b] < S else 0)
        eK = np.full(int(np.prod(ddims)), 0x3C3C, np.uint16)
        eV = eK.copy()
        oracle.stream_in(dst, src, D, S, eK, eV, dstart, dcount, want)
        gk = empty(eK.size, fill=0x3C3C)
        gv = empty(eV.size, fill=0x3C3C)
        kv.kv_stream_in(dlay, dst, gk, gv, src, dstart, dcount, st, nbytes)
        torch.cuda.synchronize()
        assert np.array_equal(host(gk), eK) and np.array_equal(host(gv), eV), f"merge into {dst}"


def test_batch_merge_of_two_sources(kv):
    """Two prompt microbatches of 3 and 2 requests merge into one token-side
    batch of 5 (batch size differs between the two sides)."""
    import torch
    D, S = 128, 520
    dst = (0, 4, 0, 6, 100, 5)
    srcs = [(0, 4, 0, 6, 100, 3), (0, 4, 0, 6, 103, 2)]
    ddims = oracle.part_dims(dst, D, S)
    note(f"batch merge dst={dst} srcs={srcs}")
    dlay = kv.kv_layout_init(*ddims, 0)
    lens = np.array([517, 3, 260, 1, 515], np.int32)
    eK = np.zeros(int(np.prod(ddims)), np.uint16)
    eV = eK.copy()
    gk, gv = empty(eK.size, fill=0), empty(eV.size, fill=0)
    for i, src in enumerate(srcs):
        dims = oracle.part_dims(src, D, S)
        lay = kv.kv_layout_init(*dims, 0)
        K, V = synth.cache_pair(dims, 90 + i)
        rows = slice(src[4] - dst[4], src[4] - dst[4] + src[5])
        count = lens[rows]
        start = np.zeros(src[5], np.int32)
        nbytes = kv.kv_stream_bytes(lay, src, dst, count)
        st = empty(nbytes // 2)
        sk, sv = dev(K), dev(V)
        kv.kv_stream_out(lay, src, sk, sv, dst, start, count, st, nbytes)
        piece = oracle.stream_out(src, dst, D, S, K, V, start, count)
        oracle.stream_in(dst, src, D, S, eK, eV, np.zeros(5, np.int32), lens, piece)
        kv.kv_stream_in(dlay, dst, gk, gv, src, np.zeros(5, np.int32), lens, st, nbytes)
        torch.cuda.synchronize()
        assert np.array_equal(host(st), piece), f"piece of {src}"
    assert np.array_equal(host(gk), eK) and np.array_equal(host(gv), eV)


def test_opt66b_slice_to_two_stages_by_two_ranks(kv):
    """The 16-layer OPT-66B slice (72 heads, 8 requests of ragged length)
    split into 4 pieces -- layers [0,8) / [8,16) x heads [0,36) / [36,72) --
    each merged into its worker's cache; sampled layers of every piece and
    every destination cache checked against the oracle on that layer."""
    import torch
    w = synth.WORKLOADS["opt-66b-16l"]
    L, B, H, D, S = w.dims
    note(f"repartition {w.name} 1 -> 2 stages x 2 ranks")
    src = (0, L, 0, H, 0, B)
    lay = kv.kv_layout_init(*w.dims, w.dtype)
    n = L * B * H * D * S
    k = torch.empty(n, dtype=torch.int16, device="cuda")
    v = torch.empty(n, dtype=torch.int16, device="cuda")
    synth.fill_device_cache(k, w.value_seed, w.dtype)
    synth.fill_device_cache(v, w.value_seed + 1, w.dtype)
    lens = synth.row_lengths(w)
    start = np.zeros(B, np.int32)
    for l0, h0 in itertools.product((0, L // 2), (0, H // 2)):
        dst = (l0, L // 2, h0, H // 2, 0, B)
        ddims = oracle.part_dims(dst, D, S)
        dlay = kv.kv_layout_init(*ddims, w.dtype)
        nbytes = kv.kv_stream_bytes(lay, src, dst, lens)
        st = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda")
        dn = int(np.prod(ddims))
        dk = torch.full((dn,), 0x1F1F, dtype=torch.int16, device="cuda")
        dvv = torch.full((dn,), 0x1F1F, dtype=torch.int16, device="cuda")
        kv.kv_stream_out(lay, src, k, v, dst, start, lens, st, nbytes)
        kv.kv_stream_in(dlay, dst, dk, dvv, src, start, lens, st, nbytes)
        torch.cuda.synchronize()
        per_layer = nbytes // 2 // (L // 2)
        for ll in (0, L // 2 - 1):
            gl = l0 + ll
            # the source's layer gl as a one-layer partition on the host
            one = (gl, 1, 0, H, 0, B)
            hk = k.view(L, -1)[gl].cpu().numpy().view(np.uint16).copy()
            hv = v.view(L, -1)[gl].cpu().numpy().view(np.uint16).copy()
            want = oracle.stream_out(one, dst, D, S, hk, hv, start, lens)
            got = st[ll * per_layer:(ll + 1) * per_layer].cpu().numpy().view(np.uint16)
            assert np.array_equal(got, want), f"piece {dst} layer {gl}"
            ek = np.full(B * (H // 2) * D * S, 0x1F1F, np.uint16)
            ev = ek.copy()
            oracle.stream_in((gl, 1, h0, H // 2, 0, B), one, D, S, ek, ev, start, lens, want)
            assert np.array_equal(dk.view(L // 2, -1)[ll].cpu().numpy().view(np.uint16), ek), \
                f"merged K {dst} layer {gl}"
            assert np.array_equal(dvv.view(L // 2, -1)[ll].cpu().numpy().view(np.uint16), ev), \
                f"merged V {dst} layer {gl}"
        del st, dk, dvv


def test_error_paths(kv):
    """Host memory in place of a cache or staging, overlapping staging and a
    short staging buffer are rejected before anything is enqueued."""
    import torch
    D, S = 64, 32
    src, dst = (0, 2, 0, 2, 0, 2), (1, 1, 1, 1, 0, 2)
    dims = oracle.part_dims(src, D, S)
    note(f"stream_out/in error paths src={src} dst={dst}")
    lay = kv.kv_layout_init(*dims, 0)
    K, V = synth.cache_pair(dims, 3)
    dk, dv = dev(K), dev(V)
    need = kv.kv_stream_bytes(lay, src, dst, [4, 4])
    st = empty(need // 2 + 64)
    pageable = np.zeros(K.size, np.uint16)
    with pytest.raises(kv.KvError) as e:                   # pageable host memory as the cache
        kv.kv_stream_out(lay, src, pageable, dv, dst, [0, 0], [4, 4], st, need)
    assert e.value.status == kv.KV_EINVAL
    with pytest.raises(kv.KvError) as e:                   # staging inside the key cache
        kv.kv_stream_out(lay, src, dk, dv, dst, [0, 0], [4, 4], dk, need)
    assert e.value.status == kv.KV_EINVAL
    with pytest.raises(kv.KvError) as e:                   # staging one vector short
        kv.kv_stream_in(lay, src, dk, dv, dst, [0, 0], [4, 4], st, need - 16)
    assert e.value.status == kv.KV_ESIZE
    with pytest.raises(kv.KvError) as e:                   # layout of another partition
        kv.kv_stream_out(lay, dst, dk, dv, src, [0, 0], [4, 4], st, need)
    assert e.value.status == kv.KV_EINVAL
    torch.cuda.synchronize()
    assert np.all(host(st) == 0x7A7A), "a rejected call wrote staging"
    assert np.array_equal(host(dk), K) and np.array_equal(host(dv), V)
