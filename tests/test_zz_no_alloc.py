"""kv_swap_out_noalloc: the swap-out that allocates nothing, through the C ABI.

Its host image must equal, bit for bit, the one kv_swap_out (the handle-based
swap engine with caller-provided banks) writes for the same region -- and the
oracle's pack of it.  Two calls in a row share the library's scratch buffer,
the second with a smaller input; a region whose single (layer, row) block
exceeds the scratch buffer is refused before anything is enqueued.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import dev, note, pinned, pinned_host_view

pytestmark = pytest.mark.gpu

CANARY = 64   # words past the image that no call may write


@pytest.fixture(scope="module")
def kv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    import kv_cache_streaming_amd as kv
    return kv


def swap_both(kv, dims, l0, nl, start, count, seed, bank_bytes):
    """Swap out one region with kv_swap_out and with kv_swap_out_noalloc; return
    both host images (with their canaries) and the oracle's pack."""
    import torch
    L, B, H, D, S = dims
    note(f"noalloc dims={dims} layers=[{l0},+{nl}) start={start} count={count}")
    K, V = synth.cache_pair(dims, seed, bits=True)
    lay = kv.kv_layout_init(*dims, 0)
    dk, dv = dev(K), dev(V)
    need = kv.kv_pack_bytes(lay, nl, count)
    words = need // 2
    ref = pinned(words + CANARY)
    got = pinned(words + CANARY)
    torch.cuda.synchronize()
    copy = torch.cuda.Stream()
    s = torch.cuda.Stream()
    eng = kv.KvSwap(lay, torch.empty(bank_bytes // 2, dtype=torch.int16, device="cuda"),
                    torch.empty(bank_bytes // 2, dtype=torch.int16, device="cuda"), bank_bytes,
                    copy)
    done = torch.cuda.Event()
    eng.swap_out(dk, dv, l0, nl, start, count, ref, need, s, done)
    kv.kv_swap_out_noalloc(lay, dk, dv, l0, nl, start, count, got, need, s)
    done.synchronize()
    s.synchronize()
    eng.close()
    want = oracle.pack(dims, K, V, l0, nl, start, count)
    return pinned_host_view(ref), pinned_host_view(got), want


def check(ref, got, want):
    n = want.size
    assert np.array_equal(ref[:n], want), "kv_swap_out differs from the oracle"
    assert np.array_equal(got[:n], ref[:n]), "kv_swap_out_noalloc differs from kv_swap_out"
    assert np.all(got[n:] == 0x5C5C), "kv_swap_out_noalloc wrote past the image"


def test_noalloc_matches_swap_out_twice(kv):
    # first call: a layer needs 327 MB, more than the 128 MiB scratch buffer,
    # so the chunks are single rows of one layer (82 MB: K and V pieces);
    # ragged rows, one of them empty
    dims = (3, 4, 8, 128, 20000)
    start, count = [0, 11, 5000, 0], [20000, 19989, 0, 7]
    ref, got, want = swap_both(kv, dims, 0, 3, start, count, seed=501, bank_bytes=96 << 20)
    check(ref, got, want)
    # second call, smaller: whole layers per chunk, other rows and layers
    dims2 = (5, 3, 4, 64, 300)
    start2, count2 = [10, 0, 299], [250, 300, 1]
    ref, got, want = swap_both(kv, dims2, 1, 3, start2, count2, seed=502, bank_bytes=8 << 20)
    check(ref, got, want)


def test_noalloc_refuses_blocks_beyond_scratch(kv):
    import torch
    # one layer of one row of 70000 tokens, 8 heads of 128: 286.7 MB > 128 MiB
    dims = (1, 1, 8, 128, 70000)
    note(f"noalloc refusal dims={dims}")
    lay = kv.kv_layout_init(*dims, 0)
    n = 8 * 128 * 70000
    dk = torch.zeros(n, dtype=torch.int16, device="cuda")
    dv = torch.zeros(n, dtype=torch.int16, device="cuda")
    need = kv.kv_pack_bytes(lay, 1, [70000])
    host = pinned(need // 2)
    with pytest.raises(kv.KvError) as ei:
        kv.kv_swap_out_noalloc(lay, dk, dv, 0, 1, [0], [70000], host, need)
    assert ei.value.status == kv.KV_ESIZE
    assert np.all(pinned_host_view(host) == 0x5C5C)
    # a region within the limit on the same cache goes through
    kv.kv_swap_out_noalloc(lay, dk, dv, 0, 1, [0], [30000], host, need)
    torch.cuda.synchronize()
    assert np.all(pinned_host_view(host)[:need // 2 * 3 // 7] == 0)
