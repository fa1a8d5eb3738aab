"""stream_out / stream_in planning through the C ABI (host only): the piece
size of two partitions against the oracle, and the argument checks."""
import numpy as np
import pytest

import oracle


@pytest.fixture(scope="module")
def kv():
    from libload import kv_module
    return kv_module()


def random_part(rng, L=12, H=16, R=9):
    l0 = int(rng.integers(0, L))
    h0 = int(rng.integers(0, H))
    r0 = int(rng.integers(0, R))
    return (l0, int(rng.integers(1, L - l0 + 1)), h0, int(rng.integers(1, H - h0 + 1)),
            r0, int(rng.integers(1, R - r0 + 1)))


def test_piece_bytes_match_the_oracle(kv):
    rng = np.random.default_rng(3)
    D, S = 64, 40
    for _ in range(400):
        me, peer = random_part(rng), random_part(rng)
        lay = kv.kv_layout_init(me[1], me[5], me[3], D, S, 0)
        count = rng.integers(0, S + 1, size=me[5]).astype(np.int32)
        got = kv.kv_stream_bytes(lay, me, peer, count)
        assert got == 2 * oracle.stream_elems(me, peer, D, count)
        # the meet is symmetric: seen from the peer with the same counts on shared rows
        assert kv.kv_stream_bytes(lay, me, peer, None) == \
            2 * oracle.stream_elems(me, peer, D, np.ones(me[5], np.int32))


def test_whole_partition_is_the_pack_size(kv):
    lay = kv.kv_layout_init(4, 3, 8, 128, 100, 1)
    part = (10, 4, 16, 8, 5, 3)
    assert kv.kv_stream_bytes(lay, part, part, [7, 0, 100]) == kv.kv_pack_bytes(lay, 4, [7, 0, 100])
    assert kv.kv_stream_bytes(lay, part, (0, 10, 0, 99, 0, 99), [7, 0, 100]) == 0


def test_rejects_bad_partitions(kv):
    lay = kv.kv_layout_init(4, 3, 8, 128, 100, 0)
    good = (0, 4, 0, 8, 0, 3)
    for bad_self in [(0, 5, 0, 8, 0, 3), (0, 4, 0, 7, 0, 3), (0, 4, 0, 8, 0, 2),
                     (-1, 4, 0, 8, 0, 3), (0, 4, 0, 8, 2**31 - 2, 3)]:
        with pytest.raises(kv.KvError) as e:
            kv.kv_stream_bytes(lay, bad_self, good, None)
        assert e.value.status == -1
    for bad_peer in [(0, 0, 0, 8, 0, 3), (0, 4, 0, -1, 0, 3), (0, 4, 0, 8, -5, 3)]:
        with pytest.raises(kv.KvError):
            kv.kv_stream_bytes(lay, good, bad_peer, None)
    with pytest.raises(kv.KvError) as e:
        kv.kv_stream_bytes(lay, good, good, [1, 101, 0])
    assert e.value.status == -2
    with pytest.raises(kv.KvError) as e:
        kv.kv_stream_bytes(lay, good, good, [1, -1, 0])
    assert e.value.status == -2


def test_copy_checks_come_before_any_enqueue(kv):
    """Errors found on the host return before anything touches a device."""
    lay = kv.kv_layout_init(2, 2, 4, 64, 16, 0)
    me, peer = (0, 2, 0, 4, 0, 2), (1, 1, 2, 2, 1, 1)
    with pytest.raises(kv.KvError) as e:        # start past the end of the cache
        kv.kv_stream_out(lay, me, 0, 0, peer, [0, 15], [1, 2], 0, 1 << 20, stream=0)
    assert e.value.status == -2
    need = kv.kv_stream_bytes(lay, me, peer, [1, 2])
    assert need == 2 * 1 * 2 * 64 * 2 * 2
    with pytest.raises(kv.KvError) as e:        # staging too small for the piece
        kv.kv_stream_in(lay, me, 0, 0, peer, [0, 0], [1, 2], 0, need - 16, stream=0)
    assert e.value.status == -3
