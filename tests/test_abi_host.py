"""Host-side checks of the C-ABI library (no GPU needed, no compute calls).

* the library loads and exports every function ``include/kvstream.h`` declares,
  and the Python binding exposes the same names;
* kv_layout_init validation and the strides of the two cache layouts;
* kv_pack_bytes against the oracle and the closed form 2 x B x S x H x D x P x N
  (lsln.cn decode-only article, "KV Cache capacity");
* argument errors that are decided before any HIP call;
* the swap engine's chunk plan, replayed on the CPU with the oracle: packing
  each chunk's layers and rows and placing its pieces at their host offsets
  must rebuild exactly the oracle's packed image of the whole range.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def kv():
    from libload import kv_module
    return kv_module()


def header_functions():
    text = open(os.path.join(ROOT, "include", "kvstream.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(kv_[a-z_]+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = header_functions()
    for required in ("kv_layout_init", "kv_pack_tokens", "kv_unpack_tokens",
                     "kv_pack_prompt_layer", "kv_swap_out", "kv_swap_in"):
        assert required in names
    assert len(names) >= 20


def test_library_exports_every_declared_symbol(kv):
    lib = ctypes.CDLL(kv.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), f"{name} declared in kvstream.h but not exported"


def test_binding_names_match_header(kv):
    declared = set(header_functions())
    assert set(kv.EXPORTED) == declared
    for name in declared:
        assert callable(getattr(kv, name)), name


def test_version(kv):
    assert kv.kv_version() == 1


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_layout_strides_match_numpy(kv, name):
    w = synth.WORKLOADS[name]
    lay = kv.kv_layout_init(w.L, w.B, w.H, w.D, w.Smax, w.dtype)
    kshape = (w.L, w.B, w.H, w.D // 8, w.Smax, 8)
    vshape = (w.L, w.B, w.H, w.Smax, w.D)
    kstr = [int(np.prod(kshape[i + 1:])) for i in range(6)]
    vstr = [int(np.prod(vshape[i + 1:])) for i in range(5)]
    assert list(lay.k_strides) == kstr and list(lay.v_strides) == vstr
    assert lay.k_bytes == lay.v_bytes == w.L * w.B * w.H * w.D * w.Smax * 2
    assert lay.elem_bytes == 2 and lay.vec_elems == 8


@pytest.mark.parametrize("args", [
    (0, 1, 1, 8, 1), (1, 0, 1, 8, 1), (1, 1, 0, 8, 1), (1, 1, 1, 0, 1), (1, 1, 1, 8, 0),
    (1, 1, 1, 12, 4), (1, 257, 1, 8, 4), (1, 1, 1, 1032, 4), (-1, 1, 1, 8, 4),
    (2**30, 2**8, 2**10, 1024, 2**20),          # bytes overflow int64
    (1, 256, 1, 8, 2**23 + 1),                  # B * Smax >= 2^31
    (1, 1, 1, 1024, 2**24),                     # Smax * D/8 >= 2^31
])
def test_layout_init_rejects(kv, args):
    with pytest.raises(kv.KvError) as e:
        kv.kv_layout_init(*args, kv.KV_F16)
    assert e.value.status == kv.KV_EINVAL


def test_layout_init_rejects_dtype(kv):
    with pytest.raises(kv.KvError):
        kv.kv_layout_init(1, 1, 1, 8, 4, 7)


def test_uninitialised_layout_is_rejected(kv):
    lay = kv.kv_layout()
    with pytest.raises(kv.KvError) as e:
        kv.kv_pack_bytes(lay, 1, None, 1)
    assert e.value.status == kv.KV_EINVAL


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_pack_bytes_closed_form(kv, name):
    w = synth.WORKLOADS[name]
    lay = kv.kv_layout_init(w.L, w.B, w.H, w.D, w.Smax, w.dtype)
    lens = synth.row_lengths(w)
    for nl in (1, w.L):
        for S in (1, w.Smax):
            assert kv.kv_pack_bytes(lay, nl, None, S) == 2 * w.B * S * w.H * w.D * 2 * nl
        got = kv.kv_pack_bytes(lay, nl, lens)
        assert got == 2 * oracle.pack_elems(w.dims, nl, lens)


def test_pack_bytes_page_example(kv):
    lay = kv.kv_layout_init(60, 1, 8, 128, 100000, kv.KV_BF16)
    assert kv.kv_pack_bytes(lay, 60, None, 100000) == 24_576_000_000


def test_errors_before_any_hip_call(kv):
    lay = kv.kv_layout_init(2, 2, 2, 16, 8, kv.KV_F16)
    fake = 1 << 40      # never dereferenced: every call below fails validation first
    with pytest.raises(kv.KvError) as e:        # start + count beyond Smax
        kv.kv_pack_tokens(lay, fake, fake, 0, 1, [7, 0], [2, 1], fake, 1 << 20, stream=0)
    assert e.value.status == kv.KV_ERANGE
    with pytest.raises(kv.KvError) as e:        # layer range
        kv.kv_pack_tokens(lay, fake, fake, 1, 2, [0, 0], [1, 1], fake, 1 << 20, stream=0)
    assert e.value.status == kv.KV_ERANGE
    with pytest.raises(kv.KvError) as e:        # negative count
        kv.kv_unpack_tokens(lay, fake, fake, 0, 1, [0, 0], [-1, 1], fake, 1 << 20, stream=0)
    assert e.value.status == kv.KV_ERANGE
    with pytest.raises(kv.KvError) as e:        # staging too small: 2*1*2*16*2*2 = 256 bytes
        kv.kv_pack_tokens(lay, fake, fake, 0, 1, [0, 0], [1, 1], fake, 255, stream=0)
    assert e.value.status == kv.KV_ESIZE
    with pytest.raises(kv.KvError) as e:        # prompt range beyond Smax
        kv.kv_pack_prompt_layer(lay, fake, fake, 0, 4, 5, None, fake, 1 << 20, stream=0)
    assert e.value.status == kv.KV_ERANGE
    with pytest.raises(kv.KvError) as e:        # row length beyond Smax
        kv.kv_pack_prompt_layer(lay, fake, fake, 0, 0, 4, [9, 1], fake, 1 << 20, stream=0)
    assert e.value.status == kv.KV_ERANGE
    with pytest.raises(kv.KvError) as e:        # missing start
        kv.kv_pack_tokens(lay, fake, fake, 0, 1, None, None, fake, 1 << 20, stream=0)
    assert e.value.status == kv.KV_EINVAL
    assert "start" in kv.kv_last_error()
    for dst, src, nbytes, status in ((fake, fake, 24, kv.KV_EINVAL),   # not whole vectors
                                     (fake, fake, -16, kv.KV_ESIZE),
                                     (0, fake, 64, kv.KV_EINVAL),      # NULL destination
                                     (fake, 0, 64, kv.KV_EINVAL)):
        with pytest.raises(kv.KvError) as e:
            kv.kv_copy_packed(dst, src, nbytes, stream=0)
        assert e.value.status == status
    kv.kv_copy_packed(fake, fake, 0, stream=0)   # nothing to move: nothing enqueued


def replay_plan(kv, dims, l0, nl, start, count, bank_bytes, seed):
    """Run the chunk plan on the CPU with the oracle; return (host image, chunks)."""
    K, V = synth.cache_pair(dims, seed, bits=True)
    L, B, H, D, S = dims
    lay = kv.kv_layout_init(L, B, H, D, S, kv.KV_F16)
    chunks = kv.kv_swap_plan(lay, l0, nl, start, count, bank_bytes)
    total = kv.kv_pack_bytes(lay, nl, count)
    host = np.full(total // 2, 0xA5A5, dtype=np.uint16)
    written = np.zeros(total // 2, dtype=np.int32)
    for c in chunks:
        sub = [count[b] if c["row_begin"] <= b < c["row_end"] else 0 for b in range(B)]
        bank = oracle.pack(dims, K, V, c["layer_begin"], c["layer_count"], start, sub)
        assert bank.nbytes == c["staged_bytes"] <= bank_bytes
        for host_off, bank_off, nbytes in c["pieces"]:
            assert host_off % 2 == 0 and bank_off % 2 == 0 and nbytes % 2 == 0
            host[host_off // 2:(host_off + nbytes) // 2] = bank[bank_off // 2:(bank_off + nbytes) // 2]
            written[host_off // 2:(host_off + nbytes) // 2] += 1
    assert np.all(written == 1), "chunks must cover the host image exactly once"
    assert np.array_equal(host, oracle.pack(dims, K, V, l0, nl, start, count))
    return chunks


def test_swap_plan_whole_layers(kv):
    dims = (6, 3, 2, 16, 10)
    start, count = [0, 2, 5], [10, 7, 3]
    layer = 2 * 2 * 16 * 2 * 20
    chunks = replay_plan(kv, dims, 1, 5, start, count, 2 * layer + 17, seed=3)
    assert [c["layer_count"] for c in chunks] == [2, 2, 1]
    assert all(len(c["pieces"]) == 1 for c in chunks)


def test_swap_plan_row_groups(kv):
    dims = (3, 5, 2, 16, 12)
    start, count = [0, 3, 0, 1, 2], [12, 0, 9, 4, 10]
    per_tok_row = 2 * 2 * 16 * 2
    chunks = replay_plan(kv, dims, 0, 3, start, count, 13 * per_tok_row, seed=4)
    assert all(c["layer_count"] == 1 and len(c["pieces"]) == 2 for c in chunks)
    assert len(chunks) > 3


def test_swap_plan_random(kv):
    rng = np.random.default_rng(12)
    for it in range(20):
        L, B, H, S = (int(rng.integers(1, 5)), int(rng.integers(1, 6)), int(rng.integers(1, 4)),
                      int(rng.integers(1, 20)))
        D = 8 * int(rng.integers(1, 4))
        start = rng.integers(0, S, size=B)
        count = [int(rng.integers(0, S - s + 1)) for s in start]
        l0 = int(rng.integers(0, L))
        nl = int(rng.integers(0, L - l0 + 1))
        per_row = [2 * H * D * 2 * c for c in count]
        bank = max(max(per_row), 1) + int(rng.integers(0, 3 * H * D * 2 * S + 1))
        replay_plan(kv, (L, B, H, D, S), l0, nl, list(start), count, bank, seed=100 + it)


def test_swap_plan_rejects_a_row_larger_than_a_bank(kv):
    lay = kv.kv_layout_init(2, 2, 2, 16, 8, kv.KV_F16)
    with pytest.raises(kv.KvError) as e:
        kv.kv_swap_plan(lay, 0, 2, [0, 0], [8, 1], 2 * 2 * 16 * 2 * 8 - 1)
    assert e.value.status == kv.KV_ESIZE


@pytest.mark.parametrize("var,val,refused", [
    ("AMD_SERIALIZE_KERNEL", "3", True), ("ROCPROF_COUNTER_COLLECTION", "1", True),
    ("ROCPROF_COUNTER_COLLECTION", "True", True), ("AMD_SERIALIZE_KERNEL", "0", False)])
def test_engine_transport_refused_under_serialised_dispatch(kv, monkeypatch, var, val, refused):
    """KV_XFER_ENGINE makes a stream wait on a DMA copy's completion value;
    when dispatches run one at a time (HIP's AMD_SERIALIZE_KERNEL, or the
    environment rocprofv3 sets for counter collection) that wait would never
    end, so both handles refuse the transport at create time, before any
    other check."""
    monkeypatch.delenv("AMD_SERIALIZE_KERNEL", raising=False)
    monkeypatch.delenv("ROCPROF_COUNTER_COLLECTION", raising=False)
    monkeypatch.setenv(var, val)
    lay = kv.kv_layout_init(2, 2, 2, 64, 16)
    h = ctypes.c_void_p()
    st = kv._lib.kv_swap_create(ctypes.byref(h), ctypes.byref(lay), 4096, 8192, 4096, None,
                                kv.KV_XFER_ENGINE)
    assert st == kv.KV_EINVAL and not h.value
    assert ("KV_XFER_ENGINE" in kv.kv_last_error()) == refused
    slot = kv.kv_pack_bytes(lay, 2, None, 1)
    st = kv._lib.kv_ring_create(ctypes.byref(h), ctypes.byref(lay), 2, 4096, 4096 + 2 * slot,
                                2 * slot, 65536, 4 * slot, None, kv.KV_XFER_ENGINE)
    assert st == kv.KV_EINVAL and not h.value
    assert ("KV_XFER_ENGINE" in kv.kv_last_error()) == refused
    # the other transports are not affected by the setting
    st = kv._lib.kv_swap_create(ctypes.byref(h), ctypes.byref(lay), 4096, 8192, 4096, None,
                                kv.KV_XFER_AUTO)
    assert st == kv.KV_EINVAL and "KV_XFER_ENGINE" not in kv.kv_last_error()


def test_set_option_null_handles(kv):
    for fn in (kv._lib.kv_swap_set_option, kv._lib.kv_ring_set_option):
        assert fn(None, kv.KV_OPT_LINK_BLOCKS, 4) == kv.KV_EINVAL
