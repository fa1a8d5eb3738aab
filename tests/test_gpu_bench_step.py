"""The benchmark's own steps, bit for bit against the oracle.

The workload tests run each call sequence on its own; here the step that
bench.py times runs as it is timed (two compute streams and one copy stream
per link direction, both directions at once, double-buffered host images,
decode steps gathered at flush, whole images in one bank-chunked call,
the workload's transport), and everything it leaves behind is checked:

* the prompt image streamed out of cache A, layer by layer;
* cache B's prompt region against the image it loaded (streamed by an
  earlier step);
* the ring's host image against the decode positions of B, and cache D's
  restored positions;
* the microbatch image swapped out of B, and cache C against the image it
  swapped in.
"""
import numpy as np
import pytest

import oracle
from gpu_util import note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bench():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    import bench as b
    return b


@pytest.fixture(autouse=True)
def free_memory():
    import gc

    import torch
    yield
    torch.cuda.synchronize()
    gc.collect()
    torch.cuda.empty_cache()
    torch._C._host_emptyCache()


def words(t):
    return t.cpu().numpy().view(np.uint16)


def host_words(t, nbytes):
    """uint16 view of the first nbytes of a pinned host buffer (torch tensor or HostBuffer)."""
    return t.numpy().view(np.uint16)[:nbytes // 2]


def check_layers(dims, K, V, count, image, layer_bytes, what):
    L, B = dims[0], dims[1]
    per = layer_bytes // 2
    for l in range(L):
        want = oracle.pack(dims, K, V, l, 1, [0] * B, count)
        assert want.size == per
        assert np.array_equal(image[l * per:(l + 1) * per], want), f"{what}, layer {l}"


@pytest.mark.timeout(900)
@pytest.mark.parametrize("transport", ["bench default", "auto"])
def test_gpt2_stream_step(bench, transport):
    import synth
    w = synth.WORKLOADS["gpt2-1.5b"]
    name = bench.DEFAULT_TRANSPORT[w.name] if transport == "bench default" else transport
    note(f"bench step {w.name} dims={w.dims} transport={name}")
    step = bench.StreamStep(w, 256 << 20, bench.TRANSPORTS[name])
    dims = w.dims
    L, B = w.L, w.B
    A = [words(t) for t in step.caches["A"]]
    for k in range(3):
        note(f"bench step {w.name}: step {k}")
        step.run()
        if k == 0:
            continue   # its inbound images were never written: nothing to compare yet
        out, inn = k % 2, (k + 1) % 2
        Bk, Bv = (words(t) for t in step.caches["B"])
        # 1: the prompt streamed out of A this step
        check_layers(dims, A[0], A[1], step.rows_prompt,
                     host_words(step.host_p[out], L * step.layer_prompt), step.layer_prompt,
                     "prompt streamed out of A")
        # 2: B's prompt region holds the image loaded this step
        check_layers(dims, Bk, Bv, step.rows_prompt,
                     host_words(step.host_p[inn], L * step.layer_prompt), step.layer_prompt,
                     "prompt loaded into B")
        # 3: the ring's host image: B's decode positions, step by step
        slots = [oracle.pack(dims, Bk, Bv, 0, L, p, [1] * B) for p in step.positions]
        ring = oracle.ring_host(slots)
        assert np.array_equal(host_words(step.ring_host, ring.nbytes), ring), "ring host image"
        # 4: D holds B's decode positions after the restore
        Dk, Dv = (words(t) for t in step.caches["D"])
        for j, p in enumerate(step.positions):
            assert np.array_equal(oracle.pack(dims, Dk, Dv, 0, L, p, [1] * B), slots[j]), \
                f"restored decode step {j}"
        del Dk, Dv
        # 5: the microbatch image swapped out of B
        check_layers(dims, Bk, Bv, step.rows_full,
                     host_words(step.host_s[out], L * step.layer_full), step.layer_full,
                     "microbatch swapped out of B")
        del Bk, Bv
        # 6: C holds the microbatch image swapped in
        Ck, Cv = (words(t) for t in step.caches["C"])
        check_layers(dims, Ck, Cv, step.rows_full,
                     host_words(step.host_s[inn], L * step.layer_full), step.layer_full,
                     "microbatch swapped into C")
        del Ck, Cv


@pytest.mark.timeout(600)
@pytest.mark.parametrize("duplex", [True, False])
def test_opt66b_ring_step(bench, duplex):
    """The ragged decode ring of the OPT-66B slice: 64 pushes gathered at
    flush, 4 flushes, restore into a second cache; duplex: two rings taking
    turns, each step restoring the image the other flushed the step before
    while its own flushes go out."""
    import synth
    import torch
    w = synth.WORKLOADS["opt-66b-16l"]
    note(f"bench step {w.name} dims={w.dims} duplex={duplex}")
    step = bench.RingStep(w, 256 << 20, bench.TRANSPORTS[bench.DEFAULT_TRANSPORT[w.name]],
                          duplex=duplex)
    dims = w.dims
    L, B = w.L, w.B
    Ak, Av = (words(t) for t in step.A)
    slots = [oracle.pack(dims, Ak, Av, 0, L, p, [1] * B) for p in step.positions]
    ring = oracle.ring_host(slots)
    del Ak, Av
    for k in range(3):
        note(f"bench step {w.name}: step {k}")
        step.run()
        if k == 0 and duplex:
            continue   # nothing flushed before the first step: no restore yet
        # every ring flushed so far holds the decode positions of A ...
        for i, host in enumerate(step.ring_hosts[:k + 1]):
            assert np.array_equal(host_words(host, ring.nbytes), ring), f"ring {i} host image"
        # ... and D holds them after this step's restore
        Dk, Dv = (words(t) for t in step.D)
        for j, p in enumerate(step.positions):
            assert np.array_equal(oracle.pack(dims, Dk, Dv, 0, L, p, [1] * B), slots[j]), \
                f"step {k}: restored decode step {j}"
        del Dk, Dv
        step.D[0].fill_(0x3A3A)     # the next restore has to write every position again
        step.D[1].fill_(0x3A3A)
        torch.cuda.synchronize()    # the fills run on torch's stream, the restore on another


def ptr_words(ptr, nbytes):
    """uint16 view of nbytes of page-locked host memory at address ptr."""
    import ctypes
    return np.ctypeslib.as_array(ctypes.cast(ptr, ctypes.POINTER(ctypes.c_uint16)),
                                 shape=(nbytes // 2,))


@pytest.mark.timeout(900)
def test_bloom_swap_round(bench):
    """Two round-robin rounds on the BLOOM-176B slice: the image of x-1 is
    rewritten by the swap-out (the host copy is overwritten with a sentinel
    first), and the slot then holds x+1's image."""
    import synth
    w = synth.WORKLOADS["bloom-176b-10l"]
    note(f"bench step {w.name} dims={w.dims}")
    step = bench.SwapStep(w, bench.DEFAULT_SWAP_BANK_MIB.get(w.name, 256) << 20,
                          bench.TRANSPORTS[bench.DEFAULT_TRANSPORT[w.name]])
    dims, L, B = w.dims, w.L, w.B
    for r in range(2):
        x = r % step.N
        out_img = ptr_words(step.img[(x - 1) % step.N], step.image)
        saved = out_img.copy()
        out_img.fill(0xE1E1)
        note(f"bench step {w.name}: round {r}")
        step.run()
        assert np.array_equal(out_img, saved), f"round {r}: image of microbatch {(x - 1) % step.N}"
        del saved
        k, v = (words(t) for t in step.slots[(r + 1) % 2])
        check_layers(dims, k, v, step.rows, ptr_words(step.img[(x + 1) % step.N], step.image),
                     step.per_layer, f"round {r}: slot after the swap-in")
        del k, v


@pytest.mark.timeout(900)
def test_gqa_100k_long_step(bench):
    """The 100K-context step (98 GB of caches): sampled layers of the row
    swap-out and swap-in, the last two streamed prompt layers, and two layers
    of every ring slot."""
    import synth
    w = synth.WORKLOADS["gqa-100k"]
    note(f"bench step {w.name} dims={w.dims}")
    step = bench.LongStep(w, 256 << 20, bench.TRANSPORTS[bench.DEFAULT_TRANSPORT[w.name]])
    L, B, H, D, S = w.dims
    one = (1, B, H, D, S)
    for k in range(2):
        note(f"bench step {w.name}: step {k}")
        step.run()
    out, inn = 1, 0                      # the second step wrote image 1 and read image 0

    def layer(t, l):
        return t.view(L, -1)[l].cpu().numpy().view(np.uint16)

    row_out = ptr_words(step.row_host[out].ptr, step.row_image)
    row_in = ptr_words(step.row_host[inn].ptr, step.row_image)
    per = step.row_layer // 2
    bstar = max(range(B), key=lambda b: step.lens[b])
    n = step.row_count[bstar]
    for l in (0, L // 2, L - 1):
        Kl, Vl = layer(step.A[0], l), layer(step.A[1], l)
        want = oracle.pack(one, Kl, Vl, 0, 1, step.row_start, step.row_count)
        assert np.array_equal(row_out[l * per:(l + 1) * per], want), f"row swapped out, layer {l}"
        # the one-row slot holds the image swapped in
        sk, sv = layer(step.slot1[0], l), layer(step.slot1[1], l)
        got = oracle.pack((1, 1, H, D, S), sk, sv, 0, 1, [0], [n])
        assert np.array_equal(got, row_in[l * per:(l + 1) * per]), f"row swapped in, layer {l}"
    # the last two layers streamed (host regions alternate by layer)
    for l in (L - 2, L - 1):
        Kl, Vl = layer(step.A[0], l), layer(step.A[1], l)
        img = ptr_words(step.prompt_host[l % 2].ptr, step.prompt_layer)
        off = 0
        for c0, nb in step.chunks:
            start, count = oracle.prompt_ranges(B, c0, w.chunk_tokens, step.lens)
            want = oracle.pack(one, Kl, Vl, 0, 1, start, count)
            assert want.nbytes == nb
            assert np.array_equal(img[off // 2:(off + nb) // 2], want), f"prompt layer {l} chunk {c0}"
            off += nb
    # every ring slot, layers 0 and L-1 (a slot is [layer][K, V][row][head][D])
    ring = host_words(step.ring_host, w.decode_steps * step.slot)
    slot_w, lw = step.slot // 2, step.slot // 2 // L
    for l in (0, L - 1):
        Kl, Vl = layer(step.A[0], l), layer(step.A[1], l)
        for j, p in enumerate(step.positions):
            want = oracle.pack(one, Kl, Vl, 0, 1, p, [1] * B)
            got = ring[j * slot_w + l * lw:j * slot_w + (l + 1) * lw]
            assert np.array_equal(got, want), f"ring slot {j}, layer {l}"


@pytest.mark.timeout(300)
def test_buffered_vs_naive_copies(bench):
    """A decode step sent to pinned host memory buffered (one pack, one copy)
    and with one runtime copy per cache region: both host images equal the
    oracle's pack of that step, and the buffered send is the faster."""
    import synth

    import kv_cache_streaming_amd as kv
    w = synth.WORKLOADS["gpt2-small-tiny"]
    note(f"buffered vs naive copies {w.name} dims={w.dims}")
    step = bench.StreamStep(w, bench.DEFAULT_SWAP_BANK_MIB.get(w.name, 256) << 20,
                            bench.TRANSPORTS["auto"])
    r = bench.buffered_vs_naive(step, kv, step.caches["B"], reps=1, keep_image=True)
    L, B, H, D, S = w.dims
    assert r["copies_per_step"] == {"buffered": 1, "per_piece": L * B * H * (D // 8 + 1),
                                    "per_head": 2 * L * B * H}
    Bk, Bv = (words(t) for t in step.caches["B"])
    want = oracle.pack(w.dims, Bk, Bv, 0, L, step.positions[0], [1] * B)
    assert np.array_equal(host_words(r["image"], want.nbytes), want)
    assert r["host_images_equal"]
    assert r["gain_over_per_piece"] > 1 and r["gain_over_per_head"] > 1, r


@pytest.mark.timeout(600)
def test_prompt_and_token_overlap(bench):
    """Layer-by-layer prompt streaming of GPT-2-1.5B against streaming after
    the prompt, and its decode steps streamed through the ring against
    compute that waits for each flush, with busy-waits as the compute: the
    streamed images equal the oracle's, and at compute equal to the transfer
    the overlap saves time."""
    import synth

    import kv_cache_streaming_amd as kv
    w = synth.WORKLOADS["gpt2-1.5b"]
    name = bench.DEFAULT_TRANSPORT[w.name]
    note(f"prompt overlap {w.name} dims={w.dims} transport={name}")
    step = bench.StreamStep(w, 256 << 20, bench.TRANSPORTS[name])
    r = bench.prompt_overlap(step, kv, reps=1)
    L = w.L
    A = [words(t) for t in step.caches["A"]]
    check_layers(w.dims, A[0], A[1], step.rows_prompt,
                 host_words(step.host_p[0], L * step.layer_prompt), step.layer_prompt,
                 "prompt streamed layer by layer")
    equal = r["rows"][1]
    assert equal["overlapped_ms"] < equal["after_ms"] / 1.2, r
    del A
    note(f"token overlap {w.name}")
    t = bench.token_overlap(step, kv, step.caches["B"], reps=1, keep_image=True)
    Bk, Bv = (words(x) for x in step.caches["B"])
    n = t["steps"]
    slots = [oracle.pack(w.dims, Bk, Bv, 0, L, p, [1] * w.B) for p in step.positions[:n]]
    ring = oracle.ring_host(slots)
    assert np.array_equal(host_words(t["image"], ring.nbytes), ring), "ring host image"
    equal = t["rows"][1]
    assert equal["overlapped_ms"] < equal["waiting_ms"] / 1.1, t
