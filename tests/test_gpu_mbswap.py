"""Microbatch swapping on two device slots (DejaVu summary, Microbatch
swapping workflow, Fig 9), bit for bit against the oracle.

Four microbatches with ragged prompts share two device caches.  Every round
the slot of the current microbatch must hold exactly its prompt plus every
token it has generated so far (swapped in from its prompt image and its ring
of step updates, while the previous microbatch computed); the round then
writes one new token per row and the schedule swaps that update out and the
microbatch two ahead in.
"""
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


@pytest.mark.parametrize("N,transport", [(4, 0), (4, 3), (4, 5), (3, 0), (2, 0)])
def test_round_robin_schedule(kv, N, transport):
    import torch
    dims = (3, 2, 2, 64, 48)
    L, B, H, D, S = dims
    steps_each = 3
    note(f"microbatch swapping dims={dims} N={N} transport={transport}")
    lay = kv.kv_layout_init(*dims, 0)
    plen = np.array([[20, 13], [7, 30], [25, 25], [1, 18]], dtype=np.int32)[:N]
    rng = np.random.default_rng(31)
    state = [synth.cache_pair(dims, 700 + x, bits=True) for x in range(N)]   # expected K, V
    copy_out, copy_in = torch.cuda.Stream(), torch.cuda.Stream()
    # prompt images, written through a swap-out of each microbatch's cache
    pbytes = [kv.kv_pack_bytes(lay, L, plen[x]) for x in range(N)]
    bank_bytes = max(pbytes)
    banks = [torch.empty(bank_bytes // 2, dtype=torch.int16, device="cuda") for _ in range(4)]
    eng_out = kv.KvSwap(lay, banks[0], banks[1], bank_bytes, copy_out, transport)
    eng_in = kv.KvSwap(lay, banks[2], banks[3], bank_bytes, copy_in, transport)
    prompt_host = [pinned(pbytes[x] // 2) for x in range(N)]
    done = torch.cuda.Event()
    for x in range(N):
        src_k, src_v = dev(state[x][0]), dev(state[x][1])
        eng_out.swap_out(src_k, src_v, 0, L, [0] * B, plen[x], prompt_host[x], pbytes[x], None, done)
        done.synchronize()
        want = oracle.pack(dims, state[x][0], state[x][1], 0, L, [0] * B, plen[x])
        assert np.array_equal(pinned_host_view(prompt_host[x]), want)
    # rings: one slot per step, flushed at once
    slot = kv.kv_pack_bytes(lay, L, None, 1)
    ring_host = [pinned(steps_each * slot // 2) for _ in range(N)]
    rings = [kv.KvRing(lay, 1, torch.empty(slot // 2, dtype=torch.int16, device="cuda"),
                       torch.empty(slot // 2, dtype=torch.int16, device="cuda"), ring_host[x],
                       copy_stream=copy_out, transport=transport) for x in range(N)]
    slots = [(empty(L * B * H * D * S, fill=0x5AA5), empty(L * B * H * D * S, fill=0x5AA5))
             for _ in range(2)]
    by_addr = {t.data_ptr(): t for pair in slots for t in pair}
    swap_stream = torch.cuda.Stream()
    m = kv.KvMbSwap(lay, slots, eng_in, rings, prompt_host, pbytes, plen, swap_stream)
    compute = torch.cuda.current_stream()
    m.start(compute)
    gen = [0] * N
    staged = [[] for _ in range(N)]
    for r in range(N * steps_each):
        x, ka, va = m.current()
        assert x == r % N
        torch.cuda.synchronize()
        k_t, v_t = by_addr[ka], by_addr[va]
        count = plen[x] + gen[x]
        got = oracle.pack(dims, host(k_t), host(v_t), 0, L, [0] * B, count)
        want = oracle.pack(dims, state[x][0], state[x][1], 0, L, [0] * B, count)
        assert np.array_equal(got, want), f"round {r}: slot does not hold microbatch {x}"
        # the step: one new token per row, written into the slot
        pos = [int(plen[x][b] + gen[x]) for b in range(B)]
        new = rng.integers(0, 1 << 16, size=oracle.pack_elems(dims, L, [1] * B),
                           dtype=np.uint32).astype(np.uint16)
        staged[x].append(new)
        kv.kv_unpack_tokens(lay, k_t, v_t, 0, L, pos, [1] * B, dev(new), stream=compute)
        oracle.unpack(dims, state[x][0], state[x][1], 0, L, pos, [1] * B, new)
        m.round(pos, compute)
        gen[x] += 1
    torch.cuda.synchronize()
    for x in range(N):
        img = pinned_host_view(ring_host[x])
        assert np.array_equal(img, np.concatenate(staged[x])), f"microbatch {x} step updates"
    m.close()
    for rg in rings:
        rg.close()
