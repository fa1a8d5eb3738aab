"""Acknowledgement log and restart point (host-only C ABI) against the oracle.

The rule (DejaVu summary, Failure detection and recovery, Fig 10, as read
here): a (microbatch, step) pair is replicated once every worker has
acknowledged it; steps run in (step, microbatch) order; the pipeline restarts
at the first pair that is not replicated.
"""
import numpy as np
import pytest

import oracle


@pytest.fixture(scope="module")
def kv():
    from libload import kv_module
    return kv_module()


def restart(kv, workers, mbs, acks):
    log = kv.KvAckLog(workers, mbs)
    for x, j, t in acks:
        log.ack(x, j, t)
    return log.restart_point()


def test_hand_worked(kv):
    acks = [(0, 0, 5), (1, 0, 4), (0, 1, 5), (1, 1, 5), (0, 2, 4), (1, 2, 4)]
    assert restart(kv, 2, 3, acks) == (0, 5)
    assert restart(kv, 1, 2, []) == (0, 0)
    assert restart(kv, 1, 1, [(0, 0, 9), (0, 0, 2)]) == (0, 10)


def test_random_ack_streams_match_the_oracle(kv):
    rng = np.random.default_rng(77)
    for it in range(200):
        workers = int(rng.integers(1, 5))
        mbs = int(rng.integers(1, 6))
        n = int(rng.integers(0, 40))
        acks = [(int(rng.integers(0, workers)), int(rng.integers(0, mbs)),
                 int(rng.integers(0, 12))) for _ in range(n)]
        assert restart(kv, workers, mbs, acks) == oracle.restart_point(workers, mbs, acks), acks


def test_errors(kv):
    with pytest.raises(kv.KvError) as e:
        kv.KvAckLog(0, 1)
    assert e.value.status == kv.KV_EINVAL
    log = kv.KvAckLog(2, 2)
    for bad in ((2, 0, 0), (0, 2, 0), (0, 0, -1), (-1, 0, 0)):
        with pytest.raises(kv.KvError) as e:
            log.ack(*bad)
        assert e.value.status == kv.KV_ERANGE
