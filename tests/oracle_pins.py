"""Pins of the oracle against facts that do not come from the oracle itself.

Each check raises AssertionError on a mismatch.  ``run_all(lib)`` runs every
check against one compiled oracle library; the test suite runs it on the real
oracle (must pass) and, in a subprocess, on mutated copies of ``oracle.c``
(each must fail), so that a plausible mistake anywhere in the oracle -- a
dropped term, a wrong index, transposed operands, a wrong loop order, an
off-by-one, a missing clip, a reversed restore order -- trips at least one pin.

The pins:

* brute force with coordinate-encoding values: every 16-bit word of a tiny
  cache encodes its own (l, b, h, s, d), so each packed word can be decoded;
  the packed buffer must list exactly the selected elements, once each, in
  lexicographic (layer, K-before-V, row, head, token, dim) order -- which is the
  packed-order definition -- and its length must equal the closed form
  2 x B x S x H x D x P x N (lsln.cn decode-only article, "KV Cache capacity");
* numpy special cases: the tiny caches are built as numpy arrays of shape
  [L,B,H,D/8,Smax,8] and [L,B,H,Smax,D] (numpy's C order realises the layouts
  independently of the oracle's offset code), so a range pack equals
  ``K[l,b,h,:,s0:s0+n,:].transpose(1,0,2)`` and ``V[l,b,h,s0:s0+n,:]`` blocks;
* round trip: unpack(pack(C)) into a zero cache reproduces C on the selected
  region and leaves 0 elsewhere; a sentinel cache keeps its sentinel outside;
* pack leaves the source caches untouched;
* prompt ranges: hand-worked clip cases;
* ring restore: the final cache holds, at every position, the value of the
  latest step that named it (last writer wins), written out per element;
* stream_out / stream_in between partitions: coordinate-decoded pieces list
  exactly the shared (global layer, K/V, row, head, token, dim) elements in
  order; a partition sent to itself, or split by layers or rows only, equals
  the already-pinned pack; a split into a grid of destinations followed by
  the merge back reproduces the source (numpy slices of the logical
  [l, b, h, s, d] views), and the pieces' sizes add up to the whole;
* paged pool: the offsets equal numpy's index of arrays shaped like the pool
  layouts; a pool with one block of Smax tokens per row and the identity
  table is the contiguous cache (pack/unpack equal the pinned ones); a random
  pool and block tables assembled into contiguous caches with numpy fancy
  indexing pack to the same words; unpack restores exactly the selected slots.
"""
from __future__ import annotations

import itertools

import numpy as np

import oracle

TINY = (2, 3, 2, 16, 8)     # L, B, H, D, Smax: 1536 words per tensor


def coord_caches(dims):
    """K and V whose words encode (l,b,h,s,d); V words are offset by the K count."""
    L, B, H, D, S = dims
    n = L * B * H * S * D
    assert 2 * n <= 65536
    l, b, h, c, s, e = np.indices((L, B, H, D // 8, S, 8))
    d = c * 8 + e
    code = (((l * B + b) * H + h) * S + s) * D + d
    K = code.astype(np.uint16)                       # shape [L,B,H,D/8,S,8]
    l, b, h, s, d = np.indices((L, B, H, S, D))
    V = (n + ((((l * B + b) * H + h) * S + s) * D + d)).astype(np.uint16)  # [L,B,H,S,D]
    return K, V, n


def decode(words, dims, n):
    L, B, H, D, S = dims
    w = words.astype(np.int64)
    kv = (w >= n).astype(np.int64)
    code = w - kv * n
    l, b, h, s, d = np.unravel_index(code, (L, B, H, S, D))
    return np.stack([l, kv, b, h, s, d], axis=1)


def selected(dims, l0, nl, start, count):
    L, B, H, D, S = dims
    rows = []
    for l in range(l0, l0 + nl):
        for kv in (0, 1):
            for b in range(B):
                for h in range(H):
                    for s in range(start[b], start[b] + count[b]):
                        for d in range(D):
                            rows.append((l, kv, b, h, s, d))
    return rows


def check_brute_force(lib, dims=TINY, cases=None):
    L, B, H, D, S = dims
    K, V, n = coord_caches(dims)
    Kf, Vf = K.ravel().copy(), V.ravel().copy()
    rng = np.random.default_rng(7)
    if cases is None:
        cases = []
        # every (start, count) per row for row 0, the others random incl. empty rows
        for s0 in range(S):
            for c0 in range(0, S - s0 + 1):
                st = [s0] + list(rng.integers(0, S, size=B - 1))
                ct = [c0] + [int(rng.integers(0, S - x + 1)) for x in st[1:]]
                l0 = int(rng.integers(0, L))
                nl = int(rng.integers(0, L - l0 + 1))
                cases.append((l0, nl, st, ct))
        cases.append((0, L, [0] * B, [S] * B))
        cases.append((1, 1, [S - 1] * B, [1] * B))
        cases.append((0, L, [0] * B, [0] * B))
    for l0, nl, st, ct in cases:
        out = oracle.pack(dims, Kf, Vf, l0, nl, st, ct, lib=lib)
        # closed form 2 x B x S x H x D x P x N (P = 2 bytes), with B x S
        # generalised to the sum of the rows' token counts for ragged rows
        tokens = int(np.sum(ct))
        assert out.size * 2 == 2 * tokens * H * D * 2 * nl, "size != closed form"
        if len(set(ct)) == 1:
            assert out.size * 2 == 2 * B * ct[0] * H * D * 2 * nl
        got = decode(out, dims, n)
        want = np.array(selected(dims, l0, nl, st, ct), dtype=np.int64).reshape(-1, 6)
        assert got.shape == want.shape, "wrong number of packed words"
        # lexicographic order of the selected set == the packed-order definition
        assert np.array_equal(got, want), f"packed order/selection wrong for {(l0, nl, st, ct)}"
    assert np.array_equal(Kf, K.ravel()) and np.array_equal(Vf, V.ravel()), "pack wrote its input"


def numpy_pack(K6, V5, l0, nl, start, count):
    parts = []
    L, B, H = K6.shape[:3]
    for l in range(l0, l0 + nl):
        for b in range(B):
            for h in range(H):
                s0, c = start[b], count[b]
                parts.append(K6[l, b, h, :, s0:s0 + c, :].transpose(1, 0, 2).ravel())
        for b in range(B):
            for h in range(H):
                s0, c = start[b], count[b]
                parts.append(V5[l, b, h, s0:s0 + c, :].ravel())
    return np.concatenate(parts) if parts else np.zeros(0, np.uint16)


def check_numpy(lib, dims=(3, 2, 3, 24, 11), seeds=range(12)):
    L, B, H, D, S = dims
    rng = np.random.default_rng(11)
    K = rng.integers(0, 1 << 16, size=(L, B, H, D // 8, S, 8), dtype=np.uint32).astype(np.uint16)
    V = rng.integers(0, 1 << 16, size=(L, B, H, S, D), dtype=np.uint32).astype(np.uint16)
    Kf, Vf = K.ravel(), V.ravel()
    for seed in seeds:
        r = np.random.default_rng(seed)
        st = r.integers(0, S, size=B).astype(np.int32)
        ct = np.array([int(r.integers(0, S - x + 1)) for x in st], dtype=np.int32)
        l0 = int(r.integers(0, L))
        nl = int(r.integers(1, L - l0 + 1))
        out = oracle.pack(dims, Kf, Vf, l0, nl, st, ct, lib=lib)
        assert np.array_equal(out, numpy_pack(K, V, l0, nl, st, ct)), "pack != numpy transpose"
    # full range of one layer = the layer's K transposed to token-major, then V
    for l in range(L):
        out = oracle.pack(dims, Kf, Vf, l, 1, [0] * B, [S] * B, lib=lib)
        want = np.concatenate([K[l].transpose(0, 1, 3, 2, 4).ravel(), V[l].ravel()])
        assert np.array_equal(out, want), "full-layer pack != transpose"
    # decode step: one token per row
    pos = [S - 1, 3]
    out = oracle.pack(dims, Kf, Vf, 0, L, pos, [1] * B, lib=lib)
    want = []
    for l in range(L):
        want += [K[l, b, h, :, pos[b], :].ravel() for b in range(B) for h in range(H)]
        want += [V[l, b, h, pos[b], :] for b in range(B) for h in range(H)]
    assert np.array_equal(out, np.concatenate(want)), "decode pack != numpy"


def check_round_trip(lib, dims=(2, 3, 2, 32, 9)):
    L, B, H, D, S = dims
    rng = np.random.default_rng(5)
    K = rng.integers(0, 1 << 16, size=(L, B, H, D // 8, S, 8), dtype=np.uint32).astype(np.uint16)
    V = rng.integers(0, 1 << 16, size=(L, B, H, S, D), dtype=np.uint32).astype(np.uint16)
    for seed in range(10):
        r = np.random.default_rng(100 + seed)
        st = r.integers(0, S, size=B).astype(np.int32)
        ct = np.array([int(r.integers(0, S - x + 1)) for x in st], dtype=np.int32)
        l0 = int(r.integers(0, L))
        nl = int(r.integers(0, L - l0 + 1))
        packed = oracle.pack(dims, K.ravel(), V.ravel(), l0, nl, st, ct, lib=lib)
        mk = np.zeros(K.shape, bool)
        mv = np.zeros(V.shape, bool)
        for b in range(B):
            mk[l0:l0 + nl, b, :, :, st[b]:st[b] + ct[b], :] = True
            mv[l0:l0 + nl, b, :, st[b]:st[b] + ct[b], :] = True
        for fill in (0, 0xBEEF):
            K2 = np.full(K.shape, fill, np.uint16)
            V2 = np.full(V.shape, fill, np.uint16)
            k2, v2 = K2.reshape(-1), V2.reshape(-1)
            oracle.unpack(dims, k2, v2, l0, nl, st, ct, packed, lib=lib)
            assert np.array_equal(K2[mk], K[mk]) and np.array_equal(V2[mv], V[mv]), \
                "round trip lost data"
            assert np.all(K2[~mk] == fill) and np.all(V2[~mv] == fill), \
                "unpack wrote outside the selected region"


def check_prompt_ranges(lib):
    # hand-worked: a 4096-token chunk starting at 4096 over rows of these lengths
    st, ct = oracle.prompt_ranges(4, 4096, 4096, [3000, 5000, 9000, 8192], lib=lib)
    assert list(st) == [4096] * 4 and list(ct) == [0, 904, 4096, 4096], (st, ct)
    st, ct = oracle.prompt_ranges(3, 0, 1000, None, lib=lib)
    assert list(ct) == [1000, 1000, 1000]
    st, ct = oracle.prompt_ranges(3, 10, 5, [0, 12, 15], lib=lib)
    assert list(ct) == [0, 2, 5]


def check_ring(lib, dims=(2, 2, 2, 16, 6)):
    L, B, H, D, S = dims
    rng = np.random.default_rng(9)
    steps = 7
    pos = np.array([[j % S, (2 * j + 1) % S] for j in range(steps)], dtype=np.int32)
    pos[5] = pos[1]                              # a later step names an earlier position
    caches, slots = [], []
    for j in range(steps):                      # the cache changes between steps
        K = rng.integers(0, 1 << 16, size=(L, B, H, D // 8, S, 8), dtype=np.uint32).astype(np.uint16)
        V = rng.integers(0, 1 << 16, size=(L, B, H, S, D), dtype=np.uint32).astype(np.uint16)
        caches.append((K, V))
        slots.append(oracle.pack(dims, K.ravel(), V.ravel(), 0, L, pos[j], [1] * B, lib=lib))
    host = oracle.ring_host(slots)
    K2 = np.zeros((L, B, H, D // 8, S, 8), np.uint16)
    V2 = np.zeros((L, B, H, S, D), np.uint16)
    oracle.ring_restore(dims, K2.reshape(-1), V2.reshape(-1), pos, host, lib=lib)
    for b in range(B):
        for p in range(S):
            named = [j for j in range(steps) if pos[j, b] == p]
            if not named:
                assert not K2[:, b, :, :, p, :].any() and not V2[:, b, :, p, :].any()
                continue
            K, V = caches[max(named)]
            assert np.array_equal(K2[:, b, :, :, p, :], K[:, b, :, :, p, :]), "ring: not last writer"
            assert np.array_equal(V2[:, b, :, p, :], V[:, b, :, p, :]), "ring: not last writer"


def check_offsets(lib, dims=(2, 3, 2, 16, 5)):
    """The exported offset functions agree with numpy's C-order index of the layouts."""
    L, B, H, D, S = dims
    for l, b, h, s, d in itertools.product(range(L), range(B), range(H), range(S), range(D)):
        k = oracle.key_offset(dims, l, b, h, s, d, lib=lib)
        v = oracle.value_offset(dims, l, b, h, s, d, lib=lib)
        assert k == np.ravel_multi_index((l, b, h, d // 8, s, d % 8), (L, B, H, D // 8, S, 8))
        assert v == np.ravel_multi_index((l, b, h, s, d), (L, B, H, S, D))


def check_restart_point(lib):
    # hand-worked: 2 workers, 3 microbatches
    acks = [(0, 0, 5), (1, 0, 4), (0, 1, 5), (1, 1, 5), (0, 2, 4), (1, 2, 4)]
    # replicated: mb0 up to 4, mb1 up to 5, mb2 up to 4 -> first gap in (step, mb)
    # order is step 5 of mb 0
    assert oracle.restart_point(2, 3, acks, lib=lib) == (0, 5)
    acks = [(0, 0, 7), (0, 1, 6), (0, 2, 6)]
    assert oracle.restart_point(1, 3, acks, lib=lib) == (1, 7)
    assert oracle.restart_point(1, 2, [], lib=lib) == (0, 0)
    # a worker that acknowledged nothing for microbatch 1 pins it at step 0
    assert oracle.restart_point(2, 2, [(0, 0, 3), (1, 0, 3), (0, 1, 3)], lib=lib) == (1, 0)
    # out-of-order acks: the later step covers the earlier
    assert oracle.restart_point(1, 1, [(0, 0, 9), (0, 0, 2)], lib=lib) == (0, 10)


def check_swap_pays(lib):
    # closed form 1: a link so fast that every transfer beats the step: N+1 steps of t
    pays, lhs, rhs = oracle.swap_pays(100, 0.03, 500, 8, 1e6, 1e18, lib=lib)
    assert lhs == 2 * 100 * 0.03 and abs(rhs - 101 * 0.03) < 1e-12 and pays
    # closed form 2: t = 0, so every step lasts its transfer: (B C / bw) * sum_{i=p}^{N+p} i
    N, p, B, C, bw = 50, 7, 3, 2.0, 5.0
    pays, lhs, rhs = oracle.swap_pays(N, 0.0, p, B, C, bw, lib=lib)
    assert lhs == 0.0 and abs(rhs - B * C / bw * (N + 1) * (2 * p + N) / 2) < 1e-9 and not pays
    # hand-worked crossover: N=2, p=1, B=1, C=1, bw=1, t=2.5 -> steps hold 1,2,3 tokens:
    # max(2.5,1)+max(2.5,2)+max(2.5,3) = 8.0 > 2*2*2.5 = 10? no: 8.0 <= 10 -> pays
    pays, lhs, rhs = oracle.swap_pays(2, 2.5, 1, 1, 1.0, 1.0, lib=lib)
    assert (pays, lhs, rhs) == (True, 10.0, 8.0)
    pays, lhs, rhs = oracle.swap_pays(2, 1.0, 3, 1, 1.0, 1.0, lib=lib)   # 3+4+5 = 12 > 4
    assert (pays, lhs, rhs) == (False, 4.0, 12.0)


def _logical_k(K6):
    """[L,B,H,D/8,S,8] -> [L,B,H,S,D] view order (a copy)."""
    L, B, H, C, S, _ = K6.shape
    return K6.transpose(0, 1, 2, 4, 3, 5).reshape(L, B, H, S, C * 8)


def _meet(a0, an, b0, bn):
    lo, hi = max(a0, b0), min(a0 + an, b0 + bn)
    return range(lo, max(lo, hi))


def check_stream(lib):
    D, S = 16, 6
    src = (2, 3, 1, 3, 10, 3)                 # layers 2..4, heads 1..3, requests 10..12
    dims = oracle.part_dims(src, D, S)
    K, V, n = coord_caches(dims)
    Kf, Vf = K.ravel().copy(), V.ravel().copy()
    start, count = [1, 0, 3], [4, 6, 2]
    dsts = [src, (0, 10, 0, 10, 0, 20), (3, 1, 0, 2, 11, 5), (0, 3, 2, 5, 0, 11),
            (4, 4, 3, 1, 12, 1), (5, 2, 0, 8, 0, 20), (2, 3, 0, 8, 13, 4), (2, 2, 2, 1, 9, 3)]
    for dst in dsts:
        out = oracle.stream_out(src, dst, D, S, Kf, Vf, start, count, lib=lib)
        got = decode(out, dims, n)
        got[:, 0] += src[0]                  # local -> global
        got[:, 2] += src[4]
        got[:, 3] += src[2]
        want = [(gl, kv, gr, gh, s, d)
                for gl in _meet(src[0], src[1], dst[0], dst[1]) for kv in (0, 1)
                for gr in _meet(src[4], src[5], dst[4], dst[5])
                for gh in _meet(src[2], src[3], dst[2], dst[3])
                for s in range(start[gr - src[4]], start[gr - src[4]] + count[gr - src[4]])
                for d in range(D)]
        want = np.array(want, dtype=np.int64).reshape(-1, 6)
        assert got.shape == want.shape and np.array_equal(got, want), f"stream_out piece for {dst}"
    assert np.array_equal(Kf, K.ravel()) and np.array_equal(Vf, V.ravel()), "stream_out wrote its input"
    # special cases that reduce to the pinned pack
    whole = oracle.stream_out(src, src, D, S, Kf, Vf, start, count, lib=lib)
    assert np.array_equal(whole, oracle.pack(dims, Kf, Vf, 0, 3, start, count, lib=lib))
    lay1 = oracle.stream_out(src, (3, 1, 0, 9, 0, 99), D, S, Kf, Vf, start, count, lib=lib)
    assert np.array_equal(lay1, oracle.pack(dims, Kf, Vf, 1, 1, start, count, lib=lib))
    rows = oracle.stream_out(src, (0, 9, 0, 9, 11, 1), D, S, Kf, Vf, start, count, lib=lib)
    assert np.array_equal(rows, oracle.pack(dims, Kf, Vf, 0, 3, start, [0, 6, 0], lib=lib))

    # split into a 2 x 2 x 2 grid of destinations, then merge back
    D, S = 16, 7
    src = (4, 4, 8, 4, 20, 4)
    dims = oracle.part_dims(src, D, S)
    rng = np.random.default_rng(21)
    K6 = rng.integers(0, 1 << 16, size=(4, 4, 4, D // 8, S, 8), dtype=np.uint32).astype(np.uint16)
    V5 = rng.integers(0, 1 << 16, size=(4, 4, 4, S, D), dtype=np.uint32).astype(np.uint16)
    start = np.array([0, 2, 5, 1], np.int32)
    count = np.array([7, 3, 0, 6], np.int32)
    Kl, Vl = _logical_k(K6), V5
    total = 0
    back_k = np.zeros_like(K6)
    back_v = np.zeros_like(V5)
    for dl, dh, dr in itertools.product((0, 2), (0, 2), (0, 2)):
        dst = (4 + dl, 2, 8 + dh, 2, 20 + dr, 2)
        shift = 1 if dr else 0               # the destination keeps its tokens one slot later
        dst_start = [int(start[dr + b]) + (shift if start[dr + b] + count[dr + b] + shift <= S else 0)
                     for b in range(2)]
        dst_count = [int(count[dr + b]) for b in range(2)]
        piece = oracle.stream_out(src, dst, D, S, K6.ravel(), V5.ravel(), start, count, lib=lib)
        total += piece.size
        dK = np.full((2, 2, 2, D // 8, S, 8), 0xABCD, np.uint16)
        dV = np.full((2, 2, 2, S, D), 0xABCD, np.uint16)
        dk, dv = dK.reshape(-1), dV.reshape(-1)
        oracle.stream_in(dst, src, D, S, dk, dv, dst_start, dst_count, piece, lib=lib)
        dKl = _logical_k(dK)
        for b in range(2):
            a, c, e = int(start[dr + b]), dst_count[b], dst_start[b]
            assert np.array_equal(dKl[:, b, :, e:e + c], Kl[dl:dl + 2, dr + b, dh:dh + 2, a:a + c]), \
                f"merged K of {dst}"
            assert np.array_equal(dV[:, b, :, e:e + c], Vl[dl:dl + 2, dr + b, dh:dh + 2, a:a + c]), \
                f"merged V of {dst}"
            mk = np.ones(dKl.shape, bool)
            mk[:, b, :, e:e + c] = False
            mk[:, 1 - b] = False
            assert np.all(dKl[mk] == 0xABCD) and np.all(dV[mk] == 0xABCD), "stream_in wrote outside"
        # and back to a source-shaped cache
        back = oracle.stream_out(dst, src, D, S, dk, dv, dst_start, dst_count, lib=lib)
        assert np.array_equal(back, piece), "piece changed on the way back"
        oracle.stream_in(src, dst, D, S, back_k.reshape(-1), back_v.reshape(-1), start, count,
                         back, lib=lib)
    assert total == oracle.pack_elems(dims, 4, count, lib=lib), "pieces do not add up to the whole"
    mk = np.zeros(K6.shape, bool)
    mv = np.zeros(V5.shape, bool)
    for b in range(4):
        mk[:, b, :, :, start[b]:start[b] + count[b], :] = True
        mv[:, b, :, start[b]:start[b] + count[b], :] = True
    assert np.array_equal(back_k[mk], K6[mk]) and not back_k[~mk].any(), "split + merge lost K"
    assert np.array_equal(back_v[mv], V5[mv]) and not back_v[~mv].any(), "split + merge lost V"


def check_paged(lib):
    # offsets: numpy's C-order index of the pool layouts
    pd = (2, 3, 2, 16, 4)
    L, NB, H, D, P = pd
    for l, blk, h, o, d in itertools.product(range(L), range(NB), range(H), range(P), range(D)):
        assert oracle.paged_key_offset(pd, l, blk, h, o, d, lib=lib) == \
            np.ravel_multi_index((l, blk, h, d // 8, o, d % 8), (L, NB, H, D // 8, P, 8))
        assert oracle.paged_value_offset(pd, l, blk, h, o, d, lib=lib) == \
            np.ravel_multi_index((l, blk, h, o, d), (L, NB, H, P, D))
    rng = np.random.default_rng(17)
    # identity: one block of Smax tokens per row is the contiguous cache
    dims = (3, 4, 2, 24, 9)
    L, B, H, D, S = dims
    K = rng.integers(0, 1 << 16, size=L * B * H * D * S, dtype=np.uint32).astype(np.uint16)
    V = rng.integers(0, 1 << 16, size=K.size, dtype=np.uint32).astype(np.uint16)
    ident = np.arange(B, dtype=np.int32).reshape(B, 1)
    for seed in range(8):
        r = np.random.default_rng(seed)
        st = r.integers(0, S, size=B).astype(np.int32)
        ct = np.array([int(r.integers(0, S - x + 1)) for x in st], np.int32)
        l0 = int(r.integers(0, L))
        nl = int(r.integers(0, L - l0 + 1))
        got = oracle.pack_paged((L, B, H, D, S), K, V, l0, nl, ident, st, ct, lib=lib)
        assert np.array_equal(got, oracle.pack(dims, K, V, l0, nl, st, ct, lib=lib)), "identity pool"
        k2, v2 = np.zeros_like(K), np.zeros_like(V)
        oracle.unpack_paged((L, B, H, D, S), k2, v2, l0, nl, ident, st, ct, got, lib=lib)
        k3, v3 = np.zeros_like(K), np.zeros_like(V)
        oracle.unpack(dims, k3, v3, l0, nl, st, ct, got, lib=lib)
        assert np.array_equal(k2, k3) and np.array_equal(v2, v3), "identity pool unpack"
    # random pool and tables, assembled into contiguous caches by numpy
    L, NB, H, D, P, B, stride = 2, 17, 3, 16, 4, 3, 5
    Kp = rng.integers(0, 1 << 16, size=(L, NB, H, D // 8, P, 8), dtype=np.uint32).astype(np.uint16)
    Vp = rng.integers(0, 1 << 16, size=(L, NB, H, P, D), dtype=np.uint32).astype(np.uint16)
    S = stride * P
    for seed in range(6):
        r = np.random.default_rng(50 + seed)
        table = r.integers(0, NB, size=(B, stride)).astype(np.int32)   # blocks may be shared
        sidx = np.arange(S)
        blk = table[:, sidx // P]                                       # [B, S]
        Kc = Kp[:, blk, :, :, sidx % P, :]        # [B, S, L, H, C, 8] after advanced indexing
        Kc = np.ascontiguousarray(Kc.transpose(2, 0, 3, 4, 1, 5))       # [L, B, H, C, S, 8]
        Vc = Vp[:, blk, :, sidx % P, :]           # [B, S, L, H, D]
        Vc = np.ascontiguousarray(Vc.transpose(2, 0, 3, 1, 4))          # [L, B, H, S, D]
        st = r.integers(0, S, size=B).astype(np.int32)
        ct = np.array([int(r.integers(0, S - x + 1)) for x in st], np.int32)
        got = oracle.pack_paged((L, NB, H, D, P), Kp.ravel(), Vp.ravel(), 0, L, table, st, ct, lib=lib)
        want = oracle.pack((L, B, H, D, S), Kc.ravel(), Vc.ravel(), 0, L, st, ct, lib=lib)
        assert np.array_equal(got, want), "paged pack != contiguous pack of the assembled cache"
    # round trip with distinct blocks: exactly the selected slots come back
    table = rng.permutation(NB)[:B * stride].reshape(B, stride).astype(np.int32)
    st = np.array([1, 0, 7], np.int32)
    ct = np.array([17, 0, 9], np.int32)
    packed = oracle.pack_paged((L, NB, H, D, P), Kp.ravel(), Vp.ravel(), 0, L, table, st, ct, lib=lib)
    k2 = np.full(Kp.shape, 0xD00D, np.uint16)
    v2 = np.full(Vp.shape, 0xD00D, np.uint16)
    oracle.unpack_paged((L, NB, H, D, P), k2.reshape(-1), v2.reshape(-1), 0, L, table, st, ct,
                        packed, lib=lib)
    mk = np.zeros(Kp.shape, bool)
    mv = np.zeros(Vp.shape, bool)
    for b in range(B):
        for s_ in range(st[b], st[b] + ct[b]):
            mk[:, table[b, s_ // P], :, :, s_ % P, :] = True
            mv[:, table[b, s_ // P], :, s_ % P, :] = True
    assert np.array_equal(k2[mk], Kp[mk]) and np.all(k2[~mk] == 0xD00D), "paged round trip K"
    assert np.array_equal(v2[mv], Vp[mv]) and np.all(v2[~mv] == 0xD00D), "paged round trip V"


def run_all(lib):
    check_offsets(lib)
    check_brute_force(lib)
    check_numpy(lib)
    check_round_trip(lib)
    check_prompt_ranges(lib)
    check_ring(lib)
    check_restart_point(lib)
    check_swap_pays(lib)
    check_stream(lib)
    check_paged(lib)


if __name__ == "__main__":          # used by the mutant test: exit 0 iff every pin holds
    import sys
    run_all(oracle.load(sys.argv[1]))
