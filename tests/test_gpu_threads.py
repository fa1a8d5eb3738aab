"""Two host threads drive the library at once, each with its own caches,
streams and swap handle: every pack, unpack and swap-out still equals the
oracle, and each thread reads its own last error (kv_last_error is
per-thread).  The binding's calls release the interpreter lock, so the two
threads are inside the library at the same time."""
import threading

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


def worker(kv, t, out):
    import torch
    try:
        torch.cuda.set_device(0)
        dims = (3, 4, 2, 64 if t == 0 else 128, 120)
        L, B, H, D, S = dims
        K, V = synth.cache_pair(dims, 900 + t, bits=True)
        lay = kv.kv_layout_init(*dims, 0)
        dk, dv = dev(K), dev(V)
        s = torch.cuda.Stream()
        torch.cuda.current_stream().synchronize()     # the caches are written before s reads them
        bank = kv.kv_pack_bytes(lay, 1, [S] * B)
        eng = kv.KvSwap(lay, empty(bank // 2), empty(bank // 2), bank, torch.cuda.Stream())
        rng = np.random.default_rng(950 + t)
        for it in range(12):
            count = rng.integers(0, S + 1, size=B).astype(np.int32)
            start = np.array([int(rng.integers(0, S - c + 1)) for c in count], np.int32)
            want = oracle.pack(dims, K, V, 0, L, start, count)
            st = empty(max(want.size, 8))
            rk, rv = torch.zeros_like(dk), torch.zeros_like(dv)
            torch.cuda.current_stream().synchronize()  # filled before the library's stream s
            kv.kv_pack_tokens(lay, dk, dv, 0, L, start, count, st, want.nbytes, s)
            kv.kv_unpack_tokens(lay, rk, rv, 0, L, start, count, st, want.nbytes, s)
            hostbuf = pinned(max(want.size, 8))
            done = torch.cuda.Event()
            eng.swap_out(dk, dv, 0, L, start, count, hostbuf, want.nbytes, s, done)
            done.synchronize()
            s.synchronize()
            assert np.array_equal(host(st)[:want.size], want), (t, it, "pack")
            ek, ev = np.zeros_like(K), np.zeros_like(V)
            oracle.unpack(dims, ek, ev, 0, L, start, count, want)
            assert np.array_equal(host(rk), ek) and np.array_equal(host(rv), ev), (t, it, "unpack")
            assert np.array_equal(pinned_host_view(hostbuf)[:want.size], want), (t, it, "swap")
            # a refused call: this thread's own message, whatever the other thread does
            bad = [S] * B if t == 0 else [0] * B
            with pytest.raises(kv.KvError):
                kv.kv_pack_tokens(lay, dk, dv, 0, L, bad, [1] * B if t == 0 else [-1] * B, st,
                                  want.nbytes, s)
            msg = kv.kv_last_error()
            assert ("outside" in msg) if t == 0 else ("negative count" in msg), (t, msg)
        eng.close()
        out[t] = True
    except BaseException as e:          # reported by the main thread
        out[t] = e


def test_two_threads_at_once(kv):
    import torch
    note("two host threads: pack, unpack, swap-out and errors at once")
    out = [None, None]
    threads = [threading.Thread(target=worker, args=(kv, t, out)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    torch.cuda.synchronize()
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    for t, r in enumerate(out):
        if r is not True:
            raise AssertionError(f"thread {t}: {r!r}")
