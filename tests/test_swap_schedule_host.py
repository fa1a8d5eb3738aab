"""Appendix E break-even test (host-only C ABI) against the oracle."""
import numpy as np
import pytest

import oracle


@pytest.fixture(scope="module")
def kv():
    from libload import kv_module
    return kv_module()


def test_matches_the_oracle(kv):
    rng = np.random.default_rng(5)
    for _ in range(300):
        N = int(rng.integers(0, 3000))
        p = int(rng.integers(0, 4000))
        B = int(rng.integers(1, 64))
        t = float(rng.uniform(0.0, 0.1))
        C = float(rng.choice([12288, 589824, 917504, 4718592 / 8]))
        bw = float(rng.uniform(5e9, 1.2e11))
        got = kv.kv_swap_pays(N, t, p, B, C, bw)
        want = oracle.swap_pays(N, t, p, B, C, bw)
        assert got[0] == want[0]
        assert got[1] == want[1] and abs(got[2] - want[2]) <= 1e-9 * max(1.0, want[2])


def test_bloom_slice_on_the_measured_link(kv):
    """The BLOOM-176B slice on one MI355X stage (10 layers, 112 heads, D=128,
    fp16: C = 2*10*112*128*2 bytes per token per request), B=16, prompt 1500:
    at 55 GB/s the 13.76 GB cache of 16 x 1500 tokens takes ~0.25 s to bring
    back, so for 100 new tokens swapping pays only when a decode step is slow
    enough to hide that transfer (here: 0.5 s yes, 30 ms no)."""
    C = 2 * 10 * 112 * 128 * 2
    fast = kv.kv_swap_pays(100, 0.030, 1500, 16, C, 55e9)
    slow = kv.kv_swap_pays(100, 0.500, 1500, 16, C, 55e9)
    assert fast[0] is False and slow[0] is True


def test_rejects_bad_arguments(kv):
    with pytest.raises(kv.KvError):
        kv.kv_swap_pays(10, 0.01, 5, 0, 100.0, 1e9)
    with pytest.raises(kv.KvError):
        kv.kv_swap_pays(10, 0.01, 5, 1, 100.0, 0.0)
