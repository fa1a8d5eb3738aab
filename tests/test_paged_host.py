"""Paged-pool planning through the C ABI (host only)."""
import numpy as np
import pytest

import oracle


@pytest.fixture(scope="module")
def kv():
    from libload import kv_module
    return kv_module()


def test_descriptor_strides_and_sizes(kv):
    pg = kv.kv_paged_init(3, 10, 4, 64, 16, 1)
    assert (pg.L, pg.blocks, pg.H, pg.D, pg.block_tokens, pg.dtype) == (3, 10, 4, 64, 16, 1)
    k = np.empty((3, 10, 4, 8, 16, 8), np.uint16)
    v = np.empty((3, 10, 4, 16, 64), np.uint16)
    assert list(pg.k_strides) == [x // 2 for x in k.strides]
    assert list(pg.v_strides) == [x // 2 for x in v.strides]
    assert pg.k_bytes == k.nbytes and pg.v_bytes == v.nbytes


def test_pack_bytes_match_the_oracle(kv):
    pg = kv.kv_paged_init(5, 7, 3, 128, 4, 0)
    rng = np.random.default_rng(2)
    for _ in range(50):
        B = int(rng.integers(1, 9))
        count = rng.integers(0, 20, size=B).astype(np.int32)
        nl = int(rng.integers(0, 6))
        table = rng.integers(0, 7, size=(B, 5)).astype(np.int32)
        Kp = np.zeros(5 * 7 * 3 * 128 * 4, np.uint16)
        got = kv.kv_paged_pack_bytes(pg, nl, B, count)
        want = oracle.pack_paged((5, 7, 3, 128, 4), Kp, Kp, 0, nl, table, [0] * B, count).nbytes
        assert got == want


def test_rejects_bad_descriptors(kv):
    for args in [(0, 1, 1, 8, 1), (1, 0, 1, 8, 1), (1, 1, 1, 12, 1), (1, 1, 1, 2048, 1),
                 (1, 1, 1, 8, 0), (2**20, 2**20, 2**20, 1024, 2**20)]:
        with pytest.raises(kv.KvError) as e:
            kv.kv_paged_init(*args)
        assert e.value.status == kv.KV_EINVAL
    with pytest.raises(kv.KvError):
        kv.kv_paged_init(1, 1, 1, 8, 1, dtype=7)


def test_check_table(kv):
    pg = kv.kv_paged_init(2, 6, 2, 16, 4, 0)
    table = np.array([[0, 1, 2], [5, -1, 9]], np.int32)
    kv.kv_paged_check_table(pg, table, [0, 0], [12, 4])          # row 1 stays in block 0
    with pytest.raises(kv.KvError) as e:
        kv.kv_paged_check_table(pg, table, [0, 0], [12, 5])      # row 1 reaches block id -1
    assert e.value.status == kv.KV_ERANGE
    with pytest.raises(kv.KvError) as e:
        kv.kv_paged_check_table(pg, table, [0, 9], [0, 2])       # tokens 9..10: block 2 = id 9
    assert e.value.status == kv.KV_ERANGE
    with pytest.raises(kv.KvError) as e:
        kv.kv_paged_check_table(pg, table, [0, 11], [0, 2])      # past the table's 12 tokens
    assert e.value.status == kv.KV_ERANGE


def test_copy_checks_come_before_any_enqueue(kv):
    pg = kv.kv_paged_init(2, 6, 2, 16, 4, 0)
    with pytest.raises(kv.KvError) as e:                          # layer range
        kv.kv_pack_paged(pg, 0, 0, 1, 2, 0, [0], [1], 0, 64, stream=0, table_stride=3)
    assert e.value.status == kv.KV_ERANGE
    with pytest.raises(kv.KvError) as e:                          # token range past the table
        kv.kv_pack_paged(pg, 0, 0, 0, 1, 0, [10], [3], 0, 1 << 10, stream=0, table_stride=3)
    assert e.value.status == kv.KV_ERANGE
    with pytest.raises(kv.KvError) as e:                          # short staging
        kv.kv_unpack_paged(pg, 0, 0, 0, 2, 0, [0, 0], [2, 1], 0, 2 * 2 * 2 * 16 * 2 * 3 - 2,
                           stream=0, table_stride=3)
    assert e.value.status == kv.KV_ESIZE
    with pytest.raises(kv.KvError) as e:
        kv.kv_pack_paged(pg, 0, 0, 0, 1, 0, [0] * 257, None, 0, 1 << 20, stream=0, table_stride=1)
    assert e.value.status == kv.KV_EINVAL
