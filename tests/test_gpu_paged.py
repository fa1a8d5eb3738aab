"""Gather/scatter between a paged block-table pool and the packed format on
the GPU, bit for bit against the oracle.  Block sizes: 16 tokens (vLLM-style
pages), 256 (chunk-organised KV), 5 (not a power of two), 1; head dims with
power-of-two and odd vector counts; ragged and decode-sized ranges; block ids
outside the pool skipped; the GPT-2-1.5B shape at full size from a 16-token
page pool."""
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


def dev_table(table):
    import torch
    return torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).cuda()


CASES = [  # L, H, D, P, B, stride, ranges
    (2, 3, 64, 16, 4, 40, "tiles"),
    (2, 2, 128, 256, 3, 3, "tiles"),
    (3, 2, 24, 5, 3, 90, "tiles"),
    (2, 2, 96, 16, 3, 20, "tiles"),         # 12-vector heads: the generic one-vector tiles
    (2, 2, 320, 16, 3, 12, "tiles"),        # 40-vector heads: the generic four-vector tiles
    (2, 3, 8, 16, 3, 10, "tiles"),          # 1-vector heads
    (2, 2, 256, 16, 3, 8, "tiles"),         # 32-vector heads: four vectors per thread
    (2, 1, 1024, 16, 2, 6, "tiles"),        # 128-vector heads
    (2, 2, 64, 1, 2, 300, "tiles"),
    (2, 3, 64, 16, 5, 8, "decode"),
    (2, 3, 64, 16, 6, 10, "span"),          # empty rows before, inside and after the moved ones
    (2, 2, 24, 5, 5, 6, "span-decode"),     # only the last row moves (few-token kernel)
]


@pytest.mark.parametrize("L,H,D,P,B,stride,ranges", CASES)
def test_pack_and_unpack_match_the_oracle(kv, L, H, D, P, B, stride, ranges):
    import torch
    rng = np.random.default_rng(P * 7 + D)
    NB = B * stride + 7
    pd = (L, NB, H, D, P)
    note(f"paged pool {pd} B={B} stride={stride} {ranges}")
    pg = kv.kv_paged_init(L, NB, H, D, P, 0)
    n = L * NB * H * D * P
    Kp = synth.random_bits(n, 300 + P)
    Vp = synth.random_bits(n, 301 + P)
    dk, dv = dev(Kp), dev(Vp)
    cap = stride * P
    if ranges == "tiles":
        count = rng.integers(0, cap + 1, size=B).astype(np.int32)
        count[0] = cap - 1
        start = np.array([int(rng.integers(0, cap - c + 1)) for c in count], np.int32)
    elif ranges == "span":
        count = np.zeros(B, np.int32)
        count[1], count[B - 2] = cap - 3, 5
        start = np.array([int(rng.integers(0, cap - c + 1)) for c in count], np.int32)
    elif ranges == "span-decode":
        count = np.zeros(B, np.int32)
        count[B - 1] = 2
        start = np.zeros(B, np.int32)
        start[B - 1] = cap - 2
    else:
        count = rng.integers(1, 3, size=B).astype(np.int32)
        start = rng.integers(0, cap - 2, size=B).astype(np.int32)
    # pack: blocks may be shared between rows
    table = rng.integers(0, NB, size=(B, stride)).astype(np.int32)
    want = oracle.pack_paged(pd, Kp, Vp, 0, L, table, start, count)
    nbytes = kv.kv_paged_pack_bytes(pg, L, B, count)
    assert nbytes == want.nbytes
    st = empty(want.size, extra=48)
    kv.kv_pack_paged(pg, dk, dv, 0, L, dev_table(table), start, count, st, nbytes)
    torch.cuda.synchronize()
    got = host(st)
    assert np.array_equal(got[:want.size], want), "paged pack"
    assert np.all(got[want.size:] == 0x7A7A), "wrote past the packed words"
    assert np.array_equal(host(dk), Kp) and np.array_equal(host(dv), Vp), "pack wrote the pool"
    # unpack: distinct blocks, into a sentinel pool; one layer range not from 0
    table = rng.permutation(NB)[:B * stride].reshape(B, stride).astype(np.int32)
    l0, nl = (1, L - 1) if L > 1 else (0, 1)
    packed = synth.random_bits(2 * nl * H * D * int(count.sum()), 77)
    eK = np.full(n, 0x6B6B, np.uint16)
    eV = eK.copy()
    oracle.unpack_paged(pd, eK, eV, l0, nl, table, start, count, packed)
    gk, gv = empty(n, fill=0x6B6B), empty(n, fill=0x6B6B)
    kv.kv_unpack_paged(pg, gk, gv, l0, nl, dev_table(table), start, count, dev(packed),
                       packed.nbytes)
    torch.cuda.synchronize()
    assert np.array_equal(host(gk), eK) and np.array_equal(host(gv), eV), "paged unpack"


def test_block_ids_outside_the_pool_are_skipped(kv):
    """Tokens whose block id is -1 or >= blocks leave their packed words (and,
    unpacking, the pool) untouched; every other word is the oracle's.  The
    expectation comes from the oracle on a pool with one extra block that
    stands in for the invalid ids: filled with the canary when packing, and
    dropped after unpacking."""
    import torch
    L, H, D, P, B, stride = 2, 2, 64, 16, 3, 6
    NB = 12
    pd, xpd = (L, NB, H, D, P), (L, NB + 1, H, D, P)
    note(f"paged pool {pd} with invalid block ids")
    pg = kv.kv_paged_init(L, NB, H, D, P, 0)
    n, per_blk = L * NB * H * D * P, H * D * P
    Kp, Vp = synth.random_bits(n, 5), synth.random_bits(n, 6)
    # the selected tokens map to distinct slots (a requirement of unpack)
    table = np.array([[0, 1, -1, 2, 3, 4], [5, NB, 6, 7, 8, 9], [10, 11, 3, 4, 7, -1]], np.int32)
    start = np.array([3, 10, 0], np.int32)
    count = np.array([60, 30, 96], np.int32)
    xtable = np.where((table < 0) | (table >= NB), NB, table).astype(np.int32)

    def extend(a, fill):
        x = np.full((L, NB + 1, per_blk), fill, np.uint16)
        x[:, :NB] = a.reshape(L, NB, per_blk)
        return x.reshape(-1)

    want = oracle.pack_paged(xpd, extend(Kp, 0x7A7A), extend(Vp, 0x7A7A), 0, L, xtable, start,
                             count)
    st = empty(want.size)
    kv.kv_pack_paged(pg, dev(Kp), dev(Vp), 0, L, dev_table(table), start, count, st)
    torch.cuda.synchronize()
    assert np.array_equal(host(st), want), "pack with skipped blocks"
    packed = synth.random_bits(want.size, 8)
    xK = extend(np.full(n, 0x4E4E, np.uint16), 0)
    xV = xK.copy()
    oracle.unpack_paged(xpd, xK, xV, 0, L, xtable, start, count, packed)
    eK = xK.reshape(L, NB + 1, per_blk)[:, :NB].reshape(-1)
    eV = xV.reshape(L, NB + 1, per_blk)[:, :NB].reshape(-1)
    gk, gv = empty(n, fill=0x4E4E), empty(n, fill=0x4E4E)
    kv.kv_unpack_paged(pg, gk, gv, 0, L, dev_table(table), start, count, dev(packed))
    torch.cuda.synchronize()
    assert np.array_equal(host(gk), eK) and np.array_equal(host(gv), eV), "unpack with skipped blocks"


@pytest.mark.parametrize("P", [16, 256])
def test_gpt2_1p5b_from_a_page_pool(kv, P):
    """48 layers x 25 heads x 64 dims, 8 rows of 1000 prompt tokens in
    P-token pages scattered over the pool: every prompt layer packed from the
    pool one call per layer and all layers in one call (as the bench times
    it), and one decode step (positions 1000) unpacked into it."""
    import torch
    w = synth.WORKLOADS["gpt2-1.5b"]
    L, B, H, D = w.L, w.B, w.H, w.D
    stride = w.Smax // P
    NB = B * stride + 40
    pd = (L, NB, H, D, P)
    note(f"paged gpt2-1.5b pool {pd} P={P}")
    pg = kv.kv_paged_init(L, NB, H, D, P, 0)
    n = L * NB * H * D * P
    rng = np.random.default_rng(16)
    table = rng.permutation(NB)[:B * stride].reshape(B, stride).astype(np.int32)
    dk = torch.empty(n, dtype=torch.int16, device="cuda")
    dv = torch.empty(n, dtype=torch.int16, device="cuda")
    synth.fill_device_cache(dk, 1616, 0)
    synth.fill_device_cache(dv, 1617, 0)
    Kp, Vp = host(dk), host(dv)
    dt = dev_table(table)
    start = np.zeros(B, np.int32)
    count = np.full(B, w.prompt_len, np.int32)
    nbytes = kv.kv_paged_pack_bytes(pg, L, B, count)
    st = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda")
    for l in range(L):
        per = nbytes // 2 // L
        kv.kv_pack_paged(pg, dk, dv, l, 1, dt, start, count, st[l * per:(l + 1) * per], per * 2)
    torch.cuda.synchronize()
    want = oracle.pack_paged(pd, Kp, Vp, 0, L, table, start, count)
    assert np.array_equal(host(st), want), "prompt layers from the page pool"
    st.fill_(0x7A7A)
    kv.kv_pack_paged(pg, dk, dv, 0, L, dt, start, count, st, nbytes)
    torch.cuda.synchronize()
    assert np.array_equal(host(st), want), "all layers from the page pool in one call"
    pos = np.full(B, w.prompt_len, np.int32)
    new = synth.random_bits(2 * L * H * D * B, 17)
    kv.kv_unpack_paged(pg, dk, dv, 0, L, dt, pos, None, dev(new), new.nbytes)
    oracle.unpack_paged(pd, Kp, Vp, 0, L, table, pos, np.ones(B, np.int32), new)
    torch.cuda.synchronize()
    assert np.array_equal(host(dk), Kp) and np.array_equal(host(dv), Vp), "decode step into the pool"


def test_error_paths(kv):
    """A pageable block table, a table that is too short for the ranges,
    staging overlapping the table, and host memory as a pool are rejected
    before anything is enqueued."""
    import torch
    L, NB, H, D, P = 2, 8, 2, 64, 16
    note(f"paged error paths pool={(L, NB, H, D, P)}")
    pg = kv.kv_paged_init(L, NB, H, D, P, 0)
    n = L * NB * H * D * P
    dk, dv = dev(synth.random_bits(n, 1)), dev(synth.random_bits(n, 2))
    table = np.arange(8, dtype=np.int32).reshape(2, 4)
    dt = dev_table(table)
    need = kv.kv_paged_pack_bytes(pg, L, 2, [20, 30])
    st = empty(need // 2 + 64)
    with pytest.raises(kv.KvError) as e:                   # the table in pageable host memory
        kv.kv_pack_paged(pg, dk, dv, 0, L, table, [0, 0], [20, 30], st, need)
    assert e.value.status == kv.KV_EINVAL
    with pytest.raises(kv.KvError) as e:                   # tokens past the table's 4 blocks
        kv.kv_pack_paged(pg, dk, dv, 0, L, dt, [0, 40], [20, 30], st, need)
    assert e.value.status == kv.KV_ERANGE
    with pytest.raises(kv.KvError) as e:                   # staging on top of the value pool
        kv.kv_pack_paged(pg, dk, dv, 0, L, dt, [0, 0], [20, 30], dv, need)
    assert e.value.status == kv.KV_EINVAL
    with pytest.raises(kv.KvError) as e:                   # host memory as the key pool
        kv.kv_unpack_paged(pg, np.zeros(n, np.uint16), dv, 0, L, dt, [0, 0], [20, 30], st, need)
    assert e.value.status == kv.KV_EINVAL
    torch.cuda.synchronize()
    assert np.all(host(st) == 0x7A7A), "a rejected call wrote staging"
