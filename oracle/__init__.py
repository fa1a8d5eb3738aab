"""The oracle: a plain, slow CPU implementation of the KV buffered-copy path.

TEST INFRASTRUCTURE ONLY.  The product library never imports, links or runs
anything here; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` do.  The arithmetic lives in
``oracle.c`` (plain C99 loops, one 16-bit element at a time); this module only
marshals numpy arrays into it.

Sources (the pages this project follows):

* "DejaVu: KV-Cache Streaming for Fast, Fault-Tolerant Generative LLM
  Serving", section "Method details": Fig 6 (max-length preallocated cache,
  non-contiguous key updates), Buffered copies (Fig 7a), Layer-by-layer prompt
  cache streaming (Fig 7b), Table 1 (gather/scatter), Microbatch swapping
  workflow (Fig 9).
* lsln.cn decode-only inference article, section "KV Cache capacity": the
  closed form 2 x B x S x H x D x P x N.

Function map: ``pack`` is gather, ``unpack`` is scatter, ``swap_out`` is a pack
over a layer range into host memory, ``swap_in`` the matching unpack,
``ring_host`` / ``ring_restore`` the staging-ring image and its restore,
``prompt_ranges`` the per-row ranges of a prompt-layer pack, ``stream_out`` /
``stream_in`` the piece of one worker's partition that another holds and its
merge (Table 1, Fast prompt KV transfer), ``pack_paged`` / ``unpack_paged`` the
same packed format gathered from a block-table pool, ``restart_point``
the (microbatch, step) a pipeline resumes from after a failure (Failure
detection and recovery, Fig 10).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# KV_ORACLE_LIB names another build of oracle.c (the sanitizer build of the
# host-side tests); the in-tree build otherwise
_LIB = os.environ.get("KV_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_p = ctypes.c_void_p


def build(out: str = _LIB, src: str = _SRC, extra_flags: tuple = ()) -> str:
    """Compile ``oracle.c`` with gcc into a shared library (no OpenMP, -O2)."""
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-Wall", "-Werror",
           *extra_flags, "-o", out, src]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def load(path: str = _LIB):
    """Load (building first if missing) and return the oracle ctypes library."""
    global _lib
    if path == _LIB and _lib is not None:
        return _lib
    if not os.path.exists(path):
        build(path)
    lib = ctypes.CDLL(path)
    lib.oracle_key_offset.restype = _i64
    lib.oracle_key_offset.argtypes = [_i64] * 10
    lib.oracle_value_offset.restype = _i64
    lib.oracle_value_offset.argtypes = [_i64] * 10
    lib.oracle_pack_elems.restype = _i64
    lib.oracle_pack_elems.argtypes = [_i64, _i64, _i64, _i64, _p]
    lib.oracle_pack.restype = None
    lib.oracle_pack.argtypes = [_i64] * 5 + [_p, _p, _i64, _i64, _p, _p, _p]
    lib.oracle_unpack.restype = None
    lib.oracle_unpack.argtypes = [_i64] * 5 + [_p, _p, _i64, _i64, _p, _p, _p]
    lib.oracle_prompt_ranges.restype = None
    lib.oracle_prompt_ranges.argtypes = [_i64, _i32, _i32, _p, _p, _p]
    lib.oracle_restart_point.restype = None
    lib.oracle_restart_point.argtypes = [_i64, _i64, _i64, _p, _p, _p, _i64, _p, _p]
    lib.oracle_swap_pays.restype = ctypes.c_int
    lib.oracle_swap_pays.argtypes = [_i64, ctypes.c_double, _i64, _i64, ctypes.c_double,
                                     ctypes.c_double, _p, _p]
    lib.oracle_paged_key_offset.restype = _i64
    lib.oracle_paged_key_offset.argtypes = [_i64] * 9
    lib.oracle_paged_value_offset.restype = _i64
    lib.oracle_paged_value_offset.argtypes = [_i64] * 9
    lib.oracle_pack_paged.restype = None
    lib.oracle_pack_paged.argtypes = [_i64] * 4 + [_p, _p, _i64, _i64, _i64, _p, _i64, _p, _p, _p]
    lib.oracle_unpack_paged.restype = None
    lib.oracle_unpack_paged.argtypes = [_i64] * 4 + [_p, _p, _i64, _i64, _i64, _p, _i64, _p, _p, _p]
    lib.oracle_stream_elems.restype = _i64
    lib.oracle_stream_elems.argtypes = [_p, _p, _i64, _p]
    lib.oracle_stream_out.restype = None
    lib.oracle_stream_out.argtypes = [_i64, _i64, _p, _p, _p, _p, _p, _p, _p]
    lib.oracle_stream_in.restype = None
    lib.oracle_stream_in.argtypes = [_i64, _i64, _p, _p, _p, _p, _p, _p, _p]
    lib.oracle_ring_restore.restype = None
    lib.oracle_ring_restore.argtypes = [_i64] * 5 + [_p, _p, _i64, _p, _i64, _p]
    if path == _LIB:
        _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _rows(x, B: int) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int32).reshape(-1))
    if a.size != B:
        raise ValueError(f"expected {B} per-row values, got {a.size}")
    return a


def _u16(a: np.ndarray, name: str) -> np.ndarray:
    if a.dtype != np.uint16 or not a.flags["C_CONTIGUOUS"]:
        raise TypeError(f"{name} must be a C-contiguous uint16 array")
    return a


def key_offset(dims, l, b, h, s, d, lib=None) -> int:
    L, B, H, D, S = dims
    return (lib or load()).oracle_key_offset(L, B, H, D, S, l, b, h, s, d)


def value_offset(dims, l, b, h, s, d, lib=None) -> int:
    L, B, H, D, S = dims
    return (lib or load()).oracle_value_offset(L, B, H, D, S, l, b, h, s, d)


def pack_elems(dims, layer_count: int, count, lib=None) -> int:
    """16-bit elements one pack moves: 2 * layer_count * H * D * sum(count)."""
    L, B, H, D, S = dims
    c = _rows(count, B)
    return (lib or load()).oracle_pack_elems(H, D, layer_count, B, _ptr(c))


def pack(dims, key, value, layer_begin, layer_count, start, count, lib=None) -> np.ndarray:
    """Gather the selected region of both caches into a new packed uint16 array."""
    lib = lib or load()
    L, B, H, D, S = dims
    key, value = _u16(key, "key"), _u16(value, "value")
    st, ct = _rows(start, B), _rows(count, B)
    out = np.empty(pack_elems(dims, layer_count, ct, lib), dtype=np.uint16)
    lib.oracle_pack(L, B, H, D, S, _ptr(key), _ptr(value), layer_begin, layer_count,
                    _ptr(st), _ptr(ct), _ptr(out))
    return out


def unpack(dims, key, value, layer_begin, layer_count, start, count, packed, lib=None) -> None:
    """Scatter ``packed`` into the caches in place (inverse of :func:`pack`)."""
    lib = lib or load()
    L, B, H, D, S = dims
    key, value = _u16(key, "key"), _u16(value, "value")
    st, ct = _rows(start, B), _rows(count, B)
    packed = _u16(np.ascontiguousarray(packed), "packed")
    need = pack_elems(dims, layer_count, ct, lib)
    if packed.size < need:
        raise ValueError(f"packed holds {packed.size} elements, {need} needed")
    lib.oracle_unpack(L, B, H, D, S, _ptr(key), _ptr(value), layer_begin, layer_count,
                      _ptr(st), _ptr(ct), _ptr(packed))


def prompt_ranges(B: int, tok_begin: int, tok_count: int, row_len=None, lib=None):
    """Per-row (start, count) of a prompt-layer pack, clipped to each row's length."""
    lib = lib or load()
    st = np.zeros(B, dtype=np.int32)
    ct = np.zeros(B, dtype=np.int32)
    rl = None if row_len is None else _rows(row_len, B)
    lib.oracle_prompt_ranges(B, tok_begin, tok_count, None if rl is None else _ptr(rl),
                             _ptr(st), _ptr(ct))
    return st, ct


def swap_out(dims, key, value, layer_begin, layer_count, start, count, lib=None) -> np.ndarray:
    """Host image of a swap-out: one pack over the whole layer range."""
    return pack(dims, key, value, layer_begin, layer_count, start, count, lib)


def swap_in(dims, key, value, layer_begin, layer_count, start, count, host, lib=None) -> None:
    """Swap-in: unpack a host image back into the caches."""
    unpack(dims, key, value, layer_begin, layer_count, start, count, host, lib)


def ring_host(slots) -> np.ndarray:
    """Host image of a staging ring: the single-token slots in step order."""
    return np.concatenate([np.asarray(s, dtype=np.uint16) for s in slots])


def ring_restore(dims, key, value, positions, host, lib=None) -> None:
    """Unpack every ring slot of ``host`` in ascending step order (in place)."""
    lib = lib or load()
    L, B, H, D, S = dims
    key, value = _u16(key, "key"), _u16(value, "value")
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int32).reshape(-1, B))
    steps = pos.shape[0]
    slot = 2 * L * H * D * B
    host = _u16(np.ascontiguousarray(host), "host")
    if host.size < steps * slot:
        raise ValueError("host image shorter than the ring's steps")
    lib.oracle_ring_restore(L, B, H, D, S, _ptr(key), _ptr(value), steps, _ptr(pos), slot,
                            _ptr(host))


def restart_point(workers: int, microbatches: int, acks, lib=None):
    """(j, t) to resume from, given acknowledgements [(x, j, t), ...]."""
    lib = lib or load()
    a = np.asarray(list(acks), dtype=np.int64).reshape(-1, 3)
    xs, js, ts = (np.ascontiguousarray(a[:, i]) for i in range(3))
    max_step = int(a[:, 2].max()) + 1 if len(a) else 0
    j = np.zeros(1, np.int64)
    t = np.zeros(1, np.int64)
    lib.oracle_restart_point(workers, microbatches, len(a), _ptr(xs), _ptr(js), _ptr(ts),
                             max_step, _ptr(j), _ptr(t))
    return int(j[0]), int(t[0])


def swap_pays(N: int, t: float, p: int, B: int, C: float, bw: float, lib=None):
    """(pays, lhs, rhs) of the Appendix E microbatch-swapping inequality."""
    lib = lib or load()
    lhs = np.zeros(1, np.float64)
    rhs = np.zeros(1, np.float64)
    r = lib.oracle_swap_pays(N, t, p, B, C, bw, _ptr(lhs), _ptr(rhs))
    return bool(r), float(lhs[0]), float(rhs[0])


def _part(p) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(p, dtype=np.int64).reshape(-1))
    if a.size != 6:
        raise ValueError("a partition is (layer0, layers, head0, heads, row0, rows)")
    return a


def part_dims(part, D: int, Smax: int):
    """(L, B, H, D, Smax) of the cache that holds `part`."""
    p = _part(part)
    return (int(p[1]), int(p[5]), int(p[3]), D, Smax)


def stream_elems(src, dst, D: int, count, lib=None) -> int:
    """16-bit elements of the piece `src` sends `dst` (count: per source row)."""
    lib = lib or load()
    s, d = _part(src), _part(dst)
    c = _rows(count, int(s[5]))
    return lib.oracle_stream_elems(_ptr(s), _ptr(d), D, _ptr(c))


def stream_out(src, dst, D: int, Smax: int, key, value, start, count, lib=None) -> np.ndarray:
    """The piece of the source partition's caches that `dst` holds."""
    lib = lib or load()
    s, d = _part(src), _part(dst)
    key, value = _u16(key, "key"), _u16(value, "value")
    st, ct = _rows(start, int(s[5])), _rows(count, int(s[5]))
    out = np.empty(stream_elems(s, d, D, ct, lib), dtype=np.uint16)
    lib.oracle_stream_out(D, Smax, _ptr(s), _ptr(d), _ptr(key), _ptr(value), _ptr(st), _ptr(ct),
                          _ptr(out))
    return out


def stream_in(dst, src, D: int, Smax: int, key, value, start, count, piece, lib=None) -> None:
    """Merge the piece `src` sent into the destination caches (in place)."""
    lib = lib or load()
    s, d = _part(src), _part(dst)
    key, value = _u16(key, "key"), _u16(value, "value")
    st, ct = _rows(start, int(d[5])), _rows(count, int(d[5]))
    piece = _u16(np.ascontiguousarray(piece), "piece")
    need = lib.oracle_stream_elems(_ptr(d), _ptr(s), D, _ptr(ct))   # the meet is symmetric
    if piece.size < need:
        raise ValueError(f"piece holds {piece.size} elements, {need} needed")
    lib.oracle_stream_in(D, Smax, _ptr(d), _ptr(s), _ptr(key), _ptr(value), _ptr(st), _ptr(ct),
                         _ptr(piece))


# ---- paged pool: dims are (L, NB, H, D, P) = layers, physical blocks, heads,
# head dim, tokens per block

def paged_key_offset(pdims, l, blk, h, o, d, lib=None) -> int:
    L, NB, H, D, P = pdims
    return (lib or load()).oracle_paged_key_offset(NB, H, D, P, l, blk, h, o, d)


def paged_value_offset(pdims, l, blk, h, o, d, lib=None) -> int:
    L, NB, H, D, P = pdims
    return (lib or load()).oracle_paged_value_offset(NB, H, D, P, l, blk, h, o, d)


def _table(table, B):
    t = np.ascontiguousarray(np.asarray(table, dtype=np.int32))
    if t.ndim != 2 or t.shape[0] != B:
        raise ValueError(f"block table must be [B={B}, stride]")
    return t


def pack_paged(pdims, key, value, layer_begin, layer_count, table, start, count, lib=None):
    """Gather rows' token ranges from a paged pool into the packed format."""
    lib = lib or load()
    L, NB, H, D, P = pdims
    key, value = _u16(key, "key"), _u16(value, "value")
    st = np.ascontiguousarray(np.asarray(start, dtype=np.int32).reshape(-1))
    B = st.size
    ct = _rows(count, B)
    tb = _table(table, B)
    out = np.empty(2 * layer_count * H * D * int(ct.sum()), dtype=np.uint16)
    lib.oracle_pack_paged(NB, H, D, P, _ptr(key), _ptr(value), layer_begin, layer_count, B,
                          _ptr(tb), tb.shape[1], _ptr(st), _ptr(ct), _ptr(out))
    return out


def unpack_paged(pdims, key, value, layer_begin, layer_count, table, start, count, packed,
                 lib=None) -> None:
    """Scatter ``packed`` into the pool in place (inverse of :func:`pack_paged`)."""
    lib = lib or load()
    L, NB, H, D, P = pdims
    key, value = _u16(key, "key"), _u16(value, "value")
    st = np.ascontiguousarray(np.asarray(start, dtype=np.int32).reshape(-1))
    B = st.size
    ct = _rows(count, B)
    tb = _table(table, B)
    packed = _u16(np.ascontiguousarray(packed), "packed")
    need = 2 * layer_count * H * D * int(ct.sum())
    if packed.size < need:
        raise ValueError(f"packed holds {packed.size} elements, {need} needed")
    lib.oracle_unpack_paged(NB, H, D, P, _ptr(key), _ptr(value), layer_begin, layer_count, B,
                            _ptr(tb), tb.shape[1], _ptr(st), _ptr(ct), _ptr(packed))
