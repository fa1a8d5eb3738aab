"""Python binding of ``libkvstream.so``, the MI355X KV-cache buffered-copy library.

Argument marshalling only: every function here forwards to the C entry point
of the same name (declared in ``include/kvstream.h``); all data movement
runs in the library's HIP kernels and copy streams.  Buffers may be passed as
torch tensors (their ``data_ptr()`` is used), as raw integer addresses, or as
numpy arrays for host-side per-row arguments.  Streams may be passed as
``torch.cuda.Stream`` objects, raw ``hipStream_t`` integers, or ``None`` (the
current torch stream).

The library must be built (``kv_cache_streaming_amd._build.build()``); importing
this package raises ``ImportError`` when it is missing -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVSTREAM_LIB names another build of the same library (the sanitizer build
# of the host-side tests); the in-tree build otherwise
LIB_PATH = os.environ.get("KVSTREAM_LIB") or os.path.join(_HERE, "libkvstream.so")

KV_OK, KV_EINVAL, KV_ERANGE, KV_ESIZE, KV_EHIP, KV_EBUSY = 0, -1, -2, -3, -4, -5
KV_F16, KV_BF16 = 0, 1
KV_XFER_AUTO, KV_XFER_KERNEL, KV_XFER_RUNTIME, KV_XFER_DMA, KV_XFER_DMA_OUT, KV_XFER_ENGINE = 0, 1, 2, 3, 4, 5
KV_RING_GATHER_EACH_STEP, KV_RING_GATHER_AT_FLUSH = 0, 1
KV_OPT_DMA_ENGINE, KV_OPT_LINK_BLOCKS = 1, 2
KV_MAX_ROWS = 256
STATUS_NAMES = {0: "KV_OK", -1: "KV_EINVAL", -2: "KV_ERANGE", -3: "KV_ESIZE",
                -4: "KV_EHIP", -5: "KV_EBUSY"}


class KvError(RuntimeError):
    """A library call returned a negative kv_status."""

    def __init__(self, status: int, func: str, message: str):
        self.status = status
        self.func = func
        super().__init__(f"{func}: {STATUS_NAMES.get(status, status)}: {message}")


class kv_layout(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int32), ("B", ctypes.c_int32), ("H", ctypes.c_int32),
                ("D", ctypes.c_int32), ("Smax", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("elem_bytes", ctypes.c_int32), ("vec_elems", ctypes.c_int32),
                ("k_strides", ctypes.c_int64 * 6), ("v_strides", ctypes.c_int64 * 5),
                ("k_bytes", ctypes.c_int64), ("v_bytes", ctypes.c_int64),
                ("magic", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]

    @property
    def dims(self):
        return (self.L, self.B, self.H, self.D, self.Smax)


class kv_chunk(ctypes.Structure):
    _fields_ = [("layer_begin", ctypes.c_int32), ("layer_count", ctypes.c_int32),
                ("row_begin", ctypes.c_int32), ("row_end", ctypes.c_int32),
                ("staged_bytes", ctypes.c_int64), ("pieces", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("host_off", ctypes.c_int64 * 2),
                ("bank_off", ctypes.c_int64 * 2), ("bytes", ctypes.c_int64 * 2)]


class kv_paged(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int32), ("blocks", ctypes.c_int32), ("H", ctypes.c_int32),
                ("D", ctypes.c_int32), ("block_tokens", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("elem_bytes", ctypes.c_int32), ("vec_elems", ctypes.c_int32),
                ("k_strides", ctypes.c_int64 * 6), ("v_strides", ctypes.c_int64 * 5),
                ("k_bytes", ctypes.c_int64), ("v_bytes", ctypes.c_int64),
                ("magic", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


class kv_part(ctypes.Structure):
    """A worker's partition: global layer, head and request (row) ranges."""
    _fields_ = [("layer0", ctypes.c_int32), ("layers", ctypes.c_int32),
                ("head0", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("row0", ctypes.c_int32), ("rows", ctypes.c_int32)]


class kv_kernel_stat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 40), ("launches", ctypes.c_int64),
                ("ms", ctypes.c_double), ("bytes", ctypes.c_int64)]


class kv_profile_window(ctypes.Structure):
    _fields_ = [("span_ms", ctypes.c_double), ("hbm_busy_ms", ctypes.c_double),
                ("hbm_bytes", ctypes.c_int64), ("hbm_launches", ctypes.c_int64),
                ("link_busy_ms", ctypes.c_double), ("link_bytes", ctypes.c_int64),
                ("link_launches", ctypes.c_int64)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_LAY = ctypes.POINTER(kv_layout)
_PART = ctypes.POINTER(kv_part)
_PG = ctypes.POINTER(kv_paged)

# name -> (restype, argtypes), mirroring include/kvstream.h
_SIGNATURES = {
    "kv_version": (ctypes.c_int, []),
    "kv_last_error": (ctypes.c_char_p, []),
    "kv_layout_init": (ctypes.c_int, [_LAY, _I32, _I32, _I32, _I32, _I32, _I32]),
    "kv_pack_bytes": (_I64, [_LAY, _I32, _P, _I32]),
    "kv_pack_tokens": (ctypes.c_int, [_LAY, _P, _P, _I32, _I32, _P, _P, _P, _I64, _P]),
    "kv_unpack_tokens": (ctypes.c_int, [_LAY, _P, _P, _I32, _I32, _P, _P, _P, _I64, _P]),
    "kv_pack_prompt_layer": (ctypes.c_int, [_LAY, _P, _P, _I32, _I32, _I32, _P, _P, _I64, _P]),
    "kv_unpack_prompt_layer": (ctypes.c_int, [_LAY, _P, _P, _I32, _I32, _I32, _P, _P, _I64, _P]),
    "kv_paged_init": (ctypes.c_int, [_PG, _I32, _I32, _I32, _I32, _I32, _I32]),
    "kv_paged_pack_bytes": (_I64, [_PG, _I32, _I32, _P]),
    "kv_pack_paged": (ctypes.c_int, [_PG, _P, _P, _I32, _I32, _I32, _P, _I32, _P, _P, _P, _I64,
                                     _P]),
    "kv_unpack_paged": (ctypes.c_int, [_PG, _P, _P, _I32, _I32, _I32, _P, _I32, _P, _P, _P, _I64,
                                       _P]),
    "kv_paged_check_table": (ctypes.c_int, [_PG, _I32, _P, _I32, _P, _P]),
    "kv_stream_bytes": (_I64, [_LAY, _PART, _PART, _P]),
    "kv_stream_out": (ctypes.c_int, [_LAY, _PART, _P, _P, _PART, _P, _P, _P, _I64, _P]),
    "kv_stream_in": (ctypes.c_int, [_LAY, _PART, _P, _P, _PART, _P, _P, _P, _I64, _P]),
    "kv_copy_packed": (ctypes.c_int, [_P, _P, _I64, _P]),
    "kv_swap_create": (ctypes.c_int, [ctypes.POINTER(_P), _LAY, _P, _P, _I64, _P, _I32]),
    "kv_swap_destroy": (ctypes.c_int, [_P]),
    "kv_swap_set_option": (ctypes.c_int, [_P, _I32, _I64]),
    "kv_ring_set_option": (ctypes.c_int, [_P, _I32, _I64]),
    "kv_swap_out": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _P, _P, _P, _I64, _P, _P]),
    "kv_swap_in": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _P, _P, _P, _I64, _P, _P]),
    "kv_stream_prompt_layer": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _P, _P, _I64, _P, _P]),
    "kv_swap_out_noalloc": (ctypes.c_int, [_LAY, _P, _P, _I32, _I32, _P, _P, _P, _I64, _P]),
    "kv_swap_plan": (_I64, [_LAY, _I32, _I32, _P, _P, _I64, _P, _I64]),
    "kv_ring_create": (ctypes.c_int, [ctypes.POINTER(_P), _LAY, _I32, _P, _P, _I64, _P, _I64, _P,
                                      _I32]),
    "kv_ring_destroy": (ctypes.c_int, [_P]),
    "kv_ring_push": (ctypes.c_int, [_P, _P, _P, _P, _P]),
    "kv_ring_flush": (ctypes.c_int, [_P, _P, _P]),
    "kv_ring_restore": (ctypes.c_int, [_P, _P, _P, _P, _P]),
    "kv_ring_restore_steps": (ctypes.c_int, [_P, _P, _P, _I64, _P, _P]),
    "kv_ring_set_gather": (ctypes.c_int, [_P, _I32]),
    "kv_ring_steps": (_I64, [_P]),
    "kv_ring_durable_steps": (_I64, [_P]),
    "kv_mbswap_create": (ctypes.c_int, [ctypes.POINTER(_P), _LAY, _I32, _P, _P, _P, _P, _P, _P, _P,
                                        _P, _P, _P]),
    "kv_mbswap_destroy": (ctypes.c_int, [_P]),
    "kv_mbswap_start": (ctypes.c_int, [_P, _P]),
    "kv_mbswap_current": (ctypes.c_int, [_P, ctypes.POINTER(_I32), ctypes.POINTER(_P),
                                         ctypes.POINTER(_P)]),
    "kv_mbswap_round": (ctypes.c_int, [_P, _P, _P]),
    "kv_swap_pays": (ctypes.c_int, [_I64, ctypes.c_double, _I64, _I64, ctypes.c_double,
                                    ctypes.c_double, ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_double)]),
    "kv_acklog_create": (ctypes.c_int, [ctypes.POINTER(_P), _I32, _I32]),
    "kv_acklog_destroy": (ctypes.c_int, [_P]),
    "kv_ack": (ctypes.c_int, [_P, _I32, _I32, _I64]),
    "kv_ack_restart_point": (ctypes.c_int, [_P, ctypes.POINTER(_I32), ctypes.POINTER(_I64)]),
    "kv_ring_reset": (ctypes.c_int, [_P]),
    "kv_profile_begin": (ctypes.c_int, []),
    "kv_profile_end": (ctypes.c_int, [ctypes.POINTER(kv_kernel_stat), _I32]),
    "kv_profile_last_window": (ctypes.c_int, [ctypes.POINTER(kv_profile_window)]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run kv_cache_streaming_amd._build.build() "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()
EXPORTED = tuple(_SIGNATURES)


def _check(status: int, func: str) -> int:
    if status < 0:
        raise KvError(int(status), func, _lib.kv_last_error().decode(errors="replace"))
    return status


def _addr(x) -> int | None:
    """Device/host address of a tensor, array or integer (None stays None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    raise TypeError(f"cannot take the address of {type(x).__name__}")


def _nbytes(x) -> int:
    if hasattr(x, "untyped_storage"):
        return x.numel() * x.element_size()
    if isinstance(x, np.ndarray):
        return x.nbytes
    raise TypeError("pass the byte count explicitly for raw addresses")


def _stream(s) -> int | None:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _event(e) -> int | None:
    if e is None:
        return None
    if isinstance(e, int):
        return e
    # torch.cuda.Event creates its hipEvent lazily, on first record: record it
    # once so that a real handle exists (the library re-records it).
    if not e.cuda_event:
        e.record()
    if not e.cuda_event:
        raise ValueError("could not obtain a hipEvent from the torch event")
    return e.cuda_event


class _Rows:
    """Keeps an int32 array alive for the duration of a call."""

    def __init__(self, x, B: int, name: str):
        if x is None:
            self.arr, self.ptr = None, None
            return
        a = np.ascontiguousarray(np.asarray(x, dtype=np.int32).reshape(-1))
        if a.size != B:
            raise ValueError(f"{name} needs {B} per-row values, got {a.size}")
        self.arr, self.ptr = a, a.ctypes.data


# ---------------------------------------------------------------- layout

def kv_version() -> int:
    return _lib.kv_version()


def kv_last_error() -> str:
    return _lib.kv_last_error().decode(errors="replace")


def kv_layout_init(L: int, B: int, H: int, D: int, Smax: int, dtype: int = KV_F16) -> kv_layout:
    lay = kv_layout()
    _check(_lib.kv_layout_init(ctypes.byref(lay), L, B, H, D, Smax, dtype), "kv_layout_init")
    return lay


def kv_pack_bytes(lay: kv_layout, layer_count: int, count=None, uniform_count: int = 0) -> int:
    c = _Rows(count, lay.B, "count")
    return _check(_lib.kv_pack_bytes(ctypes.byref(lay), layer_count, c.ptr, uniform_count),
                  "kv_pack_bytes")


# ---------------------------------------------------------------- pack / unpack

def kv_pack_tokens(lay, k, v, layer_begin, layer_count, start, count, staging,
                   staging_bytes=None, stream=None) -> None:
    st, ct = _Rows(start, lay.B, "start"), _Rows(count, lay.B, "count")
    nb = _nbytes(staging) if staging_bytes is None else staging_bytes
    _check(_lib.kv_pack_tokens(ctypes.byref(lay), _addr(k), _addr(v), layer_begin, layer_count,
                               st.ptr, ct.ptr, _addr(staging), nb, _stream(stream)),
           "kv_pack_tokens")


def kv_unpack_tokens(lay, k, v, layer_begin, layer_count, start, count, staging,
                     staging_bytes=None, stream=None) -> None:
    st, ct = _Rows(start, lay.B, "start"), _Rows(count, lay.B, "count")
    nb = _nbytes(staging) if staging_bytes is None else staging_bytes
    _check(_lib.kv_unpack_tokens(ctypes.byref(lay), _addr(k), _addr(v), layer_begin, layer_count,
                                 st.ptr, ct.ptr, _addr(staging), nb, _stream(stream)),
           "kv_unpack_tokens")


def kv_pack_prompt_layer(lay, k, v, layer, tok_begin, tok_count, row_len, staging,
                         staging_bytes=None, stream=None) -> None:
    rl = _Rows(row_len, lay.B, "row_len")
    nb = _nbytes(staging) if staging_bytes is None else staging_bytes
    _check(_lib.kv_pack_prompt_layer(ctypes.byref(lay), _addr(k), _addr(v), layer, tok_begin,
                                     tok_count, rl.ptr, _addr(staging), nb, _stream(stream)),
           "kv_pack_prompt_layer")


def kv_unpack_prompt_layer(lay, k, v, layer, tok_begin, tok_count, row_len, staging,
                           staging_bytes=None, stream=None) -> None:
    rl = _Rows(row_len, lay.B, "row_len")
    nb = _nbytes(staging) if staging_bytes is None else staging_bytes
    _check(_lib.kv_unpack_prompt_layer(ctypes.byref(lay), _addr(k), _addr(v), layer, tok_begin,
                                       tok_count, rl.ptr, _addr(staging), nb, _stream(stream)),
           "kv_unpack_prompt_layer")


def kv_swap_plan(lay, layer_begin, layer_count, start, count, bank_bytes):
    """Chunks the swap engine would use, as a list of dicts (host-only)."""
    st, ct = _Rows(start, lay.B, "start"), _Rows(count, lay.B, "count")
    n = _check(_lib.kv_swap_plan(ctypes.byref(lay), layer_begin, layer_count, st.ptr, ct.ptr,
                                 bank_bytes, None, 0), "kv_swap_plan")
    arr = (kv_chunk * max(n, 1))()
    _check(_lib.kv_swap_plan(ctypes.byref(lay), layer_begin, layer_count, st.ptr, ct.ptr,
                             bank_bytes, ctypes.cast(arr, _P), n), "kv_swap_plan")
    out = []
    for c in arr[:n]:
        out.append(dict(layer_begin=c.layer_begin, layer_count=c.layer_count,
                        row_begin=c.row_begin, row_end=c.row_end, staged_bytes=c.staged_bytes,
                        pieces=[(c.host_off[p], c.bank_off[p], c.bytes[p]) for p in range(c.pieces)]))
    return out


# ---------------------------------------------------------------- paged pools

def kv_paged_init(L: int, blocks: int, H: int, D: int, block_tokens: int,
                  dtype: int = KV_F16) -> kv_paged:
    pg = kv_paged()
    _check(_lib.kv_paged_init(ctypes.byref(pg), L, blocks, H, D, block_tokens, dtype),
           "kv_paged_init")
    return pg


def _b_rows(start):
    a = np.ascontiguousarray(np.asarray(start, dtype=np.int32).reshape(-1))
    return a, a.size


def kv_paged_pack_bytes(pg, layer_count: int, B: int, count=None) -> int:
    ct = _Rows(count, B, "count")
    return _check(_lib.kv_paged_pack_bytes(ctypes.byref(pg), layer_count, B, ct.ptr),
                  "kv_paged_pack_bytes")


def _table_stride(table, table_stride):
    if table_stride is not None:
        return table_stride
    if hasattr(table, "shape") and len(table.shape) == 2:
        return int(table.shape[1])
    raise ValueError("pass table_stride for a flat block table")


def kv_pack_paged(pg, k, v, layer_begin, layer_count, table, start, count, staging,
                  staging_bytes=None, stream=None, table_stride=None) -> None:
    st, B = _b_rows(start)
    ct = _Rows(count, B, "count")
    nb = _nbytes(staging) if staging_bytes is None else staging_bytes
    _check(_lib.kv_pack_paged(ctypes.byref(pg), _addr(k), _addr(v), layer_begin, layer_count, B,
                              _addr(table), _table_stride(table, table_stride), st.ctypes.data,
                              ct.ptr, _addr(staging), nb, _stream(stream)), "kv_pack_paged")


def kv_unpack_paged(pg, k, v, layer_begin, layer_count, table, start, count, staging,
                    staging_bytes=None, stream=None, table_stride=None) -> None:
    st, B = _b_rows(start)
    ct = _Rows(count, B, "count")
    nb = _nbytes(staging) if staging_bytes is None else staging_bytes
    _check(_lib.kv_unpack_paged(ctypes.byref(pg), _addr(k), _addr(v), layer_begin, layer_count,
                                B, _addr(table), _table_stride(table, table_stride),
                                st.ctypes.data, ct.ptr, _addr(staging), nb, _stream(stream)),
           "kv_unpack_paged")


def kv_paged_check_table(pg, table, start, count=None) -> None:
    """Host validation of a block table (numpy int32 [B, stride])."""
    t = np.ascontiguousarray(np.asarray(table, dtype=np.int32))
    st, B = _b_rows(start)
    ct = _Rows(count, B, "count")
    _check(_lib.kv_paged_check_table(ctypes.byref(pg), B, t.ctypes.data, t.shape[1],
                                     st.ctypes.data, ct.ptr), "kv_paged_check_table")


# ---------------------------------------------------------------- partitions

def _part(p) -> kv_part:
    if isinstance(p, kv_part):
        return p
    vals = [int(x) for x in p]
    if len(vals) != 6:
        raise ValueError("a partition is (layer0, layers, head0, heads, row0, rows)")
    return kv_part(*vals)


def kv_stream_bytes(lay, self_part, peer_part, count=None) -> int:
    me = _part(self_part)
    ct = _Rows(count, me.rows, "count")
    return _check(_lib.kv_stream_bytes(ctypes.byref(lay), ctypes.byref(me),
                                       ctypes.byref(_part(peer_part)), ct.ptr), "kv_stream_bytes")


def kv_stream_out(lay, src_part, k, v, dst_part, start, count, staging, staging_bytes=None,
                  stream=None) -> None:
    src = _part(src_part)
    st, ct = _Rows(start, src.rows, "start"), _Rows(count, src.rows, "count")
    nb = _nbytes(staging) if staging_bytes is None else staging_bytes
    _check(_lib.kv_stream_out(ctypes.byref(lay), ctypes.byref(src), _addr(k), _addr(v),
                              ctypes.byref(_part(dst_part)), st.ptr, ct.ptr, _addr(staging), nb,
                              _stream(stream)), "kv_stream_out")


def kv_stream_in(lay, dst_part, k, v, src_part, start, count, staging, staging_bytes=None,
                 stream=None) -> None:
    dst = _part(dst_part)
    st, ct = _Rows(start, dst.rows, "start"), _Rows(count, dst.rows, "count")
    nb = _nbytes(staging) if staging_bytes is None else staging_bytes
    _check(_lib.kv_stream_in(ctypes.byref(lay), ctypes.byref(dst), _addr(k), _addr(v),
                             ctypes.byref(_part(src_part)), st.ptr, ct.ptr, _addr(staging), nb,
                             _stream(stream)), "kv_stream_in")


def kv_copy_packed(dst, src, nbytes=None, stream=None) -> None:
    """Device-to-device move of a packed block (``nbytes`` defaults to the
    source's size)."""
    nb = _nbytes(src) if nbytes is None else nbytes
    _check(_lib.kv_copy_packed(_addr(dst), _addr(src), nb, _stream(stream)), "kv_copy_packed")


# ---------------------------------------------------------------- swap engine

class KvSwap:
    """Handle of a swap engine (kv_swap_create / kv_swap_destroy)."""

    def __init__(self, lay, bank0, bank1, bank_bytes=None, copy_stream=None,
                 transport=KV_XFER_AUTO):
        self.lay = lay
        self._keep = (bank0, bank1)
        self._destroy = _lib.kv_swap_destroy
        nb = min(_nbytes(bank0), _nbytes(bank1)) if bank_bytes is None else bank_bytes
        h = _P()
        _check(_lib.kv_swap_create(ctypes.byref(h), ctypes.byref(lay), _addr(bank0), _addr(bank1),
                                   nb, _stream(copy_stream), transport), "kv_swap_create")
        self._h = h

    def close(self):
        """Destroy the handle; KvError when its DMA copies could not be waited for."""
        if getattr(self, "_h", None):
            h, self._h = self._h, None
            _check(self._destroy(h), "kv_swap_destroy")

    def __del__(self):
        try:
            self.close()
        except KvError:
            pass

    def set_option(self, option: int, value: int) -> None:
        _check(_lib.kv_swap_set_option(self._h, option, value), "kv_swap_set_option")

    def swap_out(self, k, v, layer_begin, layer_count, start, count, host, host_bytes=None,
                 compute=None, done=None):
        st, ct = _Rows(start, self.lay.B, "start"), _Rows(count, self.lay.B, "count")
        nb = _nbytes(host) if host_bytes is None else host_bytes
        _check(_lib.kv_swap_out(self._h, _addr(k), _addr(v), layer_begin, layer_count, st.ptr,
                                ct.ptr, _addr(host), nb, _stream(compute), _event(done)),
               "kv_swap_out")

    def swap_in(self, k, v, layer_begin, layer_count, start, count, host, host_bytes=None,
                compute=None, done=None):
        st, ct = _Rows(start, self.lay.B, "start"), _Rows(count, self.lay.B, "count")
        nb = _nbytes(host) if host_bytes is None else host_bytes
        _check(_lib.kv_swap_in(self._h, _addr(k), _addr(v), layer_begin, layer_count, st.ptr,
                               ct.ptr, _addr(host), nb, _stream(compute), _event(done)),
               "kv_swap_in")

    def stream_prompt_layer(self, k, v, layer, tok_begin, tok_count, row_len, host,
                            host_bytes=None, compute=None, done=None):
        rl = _Rows(row_len, self.lay.B, "row_len")
        nb = _nbytes(host) if host_bytes is None else host_bytes
        _check(_lib.kv_stream_prompt_layer(self._h, _addr(k), _addr(v), layer, tok_begin,
                                           tok_count, rl.ptr, _addr(host), nb, _stream(compute),
                                           _event(done)), "kv_stream_prompt_layer")


def kv_swap_out_noalloc(lay, k, v, layer_begin, layer_count, start, count, host,
                        host_bytes=None, stream=None) -> None:
    """Swap-out through the library's static scratch buffer on one stream
    (allocates nothing; see kv_swap_out_noalloc in kvstream.h)."""
    st, ct = _Rows(start, lay.B, "start"), _Rows(count, lay.B, "count")
    nb = _nbytes(host) if host_bytes is None else host_bytes
    _check(_lib.kv_swap_out_noalloc(ctypes.byref(lay), _addr(k), _addr(v), layer_begin,
                                    layer_count, st.ptr, ct.ptr, _addr(host), nb, _stream(stream)),
           "kv_swap_out_noalloc")


def kv_swap_create(lay, bank0, bank1, bank_bytes=None, copy_stream=None,
                   transport=KV_XFER_AUTO) -> KvSwap:
    return KvSwap(lay, bank0, bank1, bank_bytes, copy_stream, transport)


def kv_swap_destroy(e: KvSwap) -> None:
    e.close()


def kv_swap_set_option(e: KvSwap, option: int, value: int) -> None:
    e.set_option(option, value)


def kv_ring_set_option(r: "KvRing", option: int, value: int) -> None:
    r.set_option(option, value)


def kv_swap_out(e: KvSwap, *args, **kw) -> None:
    e.swap_out(*args, **kw)


def kv_swap_in(e: KvSwap, *args, **kw) -> None:
    e.swap_in(*args, **kw)


def kv_stream_prompt_layer(e: KvSwap, *args, **kw) -> None:
    e.stream_prompt_layer(*args, **kw)


# ---------------------------------------------------------------- staging ring

class KvRing:
    """Handle of a decode-step staging ring (kv_ring_create / kv_ring_destroy)."""

    def __init__(self, lay, R, bank0, bank1, host, bank_bytes=None, host_bytes=None,
                 copy_stream=None, transport=KV_XFER_AUTO):
        self.lay = lay
        self.R = R
        self._keep = (bank0, bank1, host)
        self._destroy = _lib.kv_ring_destroy
        nb = min(_nbytes(bank0), _nbytes(bank1)) if bank_bytes is None else bank_bytes
        hb = _nbytes(host) if host_bytes is None else host_bytes
        h = _P()
        _check(_lib.kv_ring_create(ctypes.byref(h), ctypes.byref(lay), R, _addr(bank0),
                                   _addr(bank1), nb, _addr(host), hb, _stream(copy_stream),
                                   transport), "kv_ring_create")
        self._h = h

    def close(self):
        """Destroy the handle; KvError when its DMA copies could not be waited for."""
        if getattr(self, "_h", None):
            h, self._h = self._h, None
            _check(self._destroy(h), "kv_ring_destroy")

    def __del__(self):
        try:
            self.close()
        except KvError:
            pass

    def push(self, k, v, pos, compute=None):
        p = _Rows(pos, self.lay.B, "pos")
        _check(_lib.kv_ring_push(self._h, _addr(k), _addr(v), p.ptr, _stream(compute)),
               "kv_ring_push")

    def flush(self, compute=None, done=None):
        _check(_lib.kv_ring_flush(self._h, _stream(compute), _event(done)), "kv_ring_flush")

    def restore(self, k, v, compute=None, done=None):
        _check(_lib.kv_ring_restore(self._h, _addr(k), _addr(v), _stream(compute), _event(done)),
               "kv_ring_restore")

    def restore_steps(self, k, v, n, compute=None, done=None):
        _check(_lib.kv_ring_restore_steps(self._h, _addr(k), _addr(v), n, _stream(compute),
                                          _event(done)), "kv_ring_restore_steps")

    def set_gather(self, mode: int) -> None:
        _check(_lib.kv_ring_set_gather(self._h, mode), "kv_ring_set_gather")

    def set_option(self, option: int, value: int) -> None:
        _check(_lib.kv_ring_set_option(self._h, option, value), "kv_ring_set_option")

    @property
    def steps(self) -> int:
        return _check(_lib.kv_ring_steps(self._h), "kv_ring_steps")

    @property
    def durable_steps(self) -> int:
        return _check(_lib.kv_ring_durable_steps(self._h), "kv_ring_durable_steps")

    def reset(self):
        _check(_lib.kv_ring_reset(self._h), "kv_ring_reset")


def kv_ring_create(lay, R, bank0, bank1, host, bank_bytes=None, host_bytes=None,
                   copy_stream=None, transport=KV_XFER_AUTO) -> KvRing:
    return KvRing(lay, R, bank0, bank1, host, bank_bytes, host_bytes, copy_stream, transport)


def kv_ring_destroy(r: KvRing) -> None:
    r.close()


def kv_ring_push(r: KvRing, *args, **kw) -> None:
    r.push(*args, **kw)


def kv_ring_flush(r: KvRing, *args, **kw) -> None:
    r.flush(*args, **kw)


def kv_ring_restore(r: KvRing, *args, **kw) -> None:
    r.restore(*args, **kw)


def kv_ring_restore_steps(r: KvRing, *args, **kw) -> None:
    r.restore_steps(*args, **kw)


def kv_ring_set_gather(r: KvRing, mode: int) -> None:
    r.set_gather(mode)


def kv_ring_steps(r: KvRing) -> int:
    return r.steps


def kv_ring_durable_steps(r: KvRing) -> int:
    return r.durable_steps


# ---------------------------------------------------------------- microbatch swapping

class KvMbSwap:
    """Microbatch swapping on two device slots (kv_mbswap_create / _destroy)."""

    def __init__(self, lay, slots, swap_in_engine: KvSwap, rings, prompt_host, prompt_bytes,
                 prompt_len, swap_stream=None):
        n = len(rings)
        self.lay, self.n = lay, n
        self._keep = (slots, swap_in_engine, rings, prompt_host)
        self._destroy = _lib.kv_mbswap_destroy
        ring_ptrs = (_P * n)(*[r._h.value for r in rings])
        host_ptrs = (_P * n)(*[_addr(h) for h in prompt_host])
        self._bytes = np.ascontiguousarray(np.asarray(prompt_bytes, dtype=np.int64))
        self._len = np.ascontiguousarray(np.asarray(prompt_len, dtype=np.int32).reshape(-1))
        if self._len.size != n * lay.B or self._bytes.size != n:
            raise ValueError("prompt_len needs microbatches*B values, prompt_bytes one per microbatch")
        (k0, v0), (k1, v1) = slots
        h = _P()
        _check(_lib.kv_mbswap_create(ctypes.byref(h), ctypes.byref(lay), n, _addr(k0), _addr(v0),
                                     _addr(k1), _addr(v1), swap_in_engine._h, ring_ptrs, host_ptrs,
                                     self._bytes.ctypes.data, self._len.ctypes.data,
                                     _stream(swap_stream)), "kv_mbswap_create")
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            self._destroy(self._h)
            self._h = None

    __del__ = close

    def start(self, compute=None):
        _check(_lib.kv_mbswap_start(self._h, _stream(compute)), "kv_mbswap_start")

    def current(self):
        """(microbatch, k address, v address) of the current round."""
        x, k, v = _I32(), _P(), _P()
        _check(_lib.kv_mbswap_current(self._h, ctypes.byref(x), ctypes.byref(k), ctypes.byref(v)),
               "kv_mbswap_current")
        return x.value, k.value, v.value

    def round(self, pos, compute=None):
        p = _Rows(pos, self.lay.B, "pos")
        _check(_lib.kv_mbswap_round(self._h, p.ptr, _stream(compute)), "kv_mbswap_round")


def kv_mbswap_create(*args, **kw) -> KvMbSwap:
    return KvMbSwap(*args, **kw)


def kv_mbswap_destroy(m: KvMbSwap) -> None:
    m.close()


def kv_mbswap_start(m: KvMbSwap, compute=None) -> None:
    m.start(compute)


def kv_mbswap_current(m: KvMbSwap):
    return m.current()


def kv_mbswap_round(m: KvMbSwap, pos, compute=None) -> None:
    m.round(pos, compute)


def kv_swap_pays(N: int, t: float, p: int, B: int, C: float, bw: float):
    """(pays, lhs, rhs) of the Appendix E break-even test."""
    lhs, rhs = ctypes.c_double(), ctypes.c_double()
    r = _check(_lib.kv_swap_pays(N, t, p, B, C, bw, ctypes.byref(lhs), ctypes.byref(rhs)),
               "kv_swap_pays")
    return bool(r), lhs.value, rhs.value


# ---------------------------------------------------------------- acknowledgement log

class KvAckLog:
    """Handle of an acknowledgement log (kv_acklog_create / kv_acklog_destroy)."""

    def __init__(self, workers: int, microbatches: int):
        self._destroy = _lib.kv_acklog_destroy
        h = _P()
        _check(_lib.kv_acklog_create(ctypes.byref(h), workers, microbatches), "kv_acklog_create")
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            self._destroy(self._h)
            self._h = None

    __del__ = close

    def ack(self, x: int, j: int, t: int) -> None:
        _check(_lib.kv_ack(self._h, x, j, t), "kv_ack")

    def restart_point(self):
        j, t = _I32(), _I64()
        _check(_lib.kv_ack_restart_point(self._h, ctypes.byref(j), ctypes.byref(t)),
               "kv_ack_restart_point")
        return j.value, t.value


def kv_acklog_create(workers: int, microbatches: int) -> KvAckLog:
    return KvAckLog(workers, microbatches)


def kv_acklog_destroy(a: KvAckLog) -> None:
    a.close()


def kv_ack(a: KvAckLog, x: int, j: int, t: int) -> None:
    a.ack(x, j, t)


def kv_ack_restart_point(a: KvAckLog):
    return a.restart_point()


def kv_ring_reset(r: KvRing) -> None:
    r.reset()


# ---------------------------------------------------------------- live timing

def kv_profile_begin() -> None:
    _check(_lib.kv_profile_begin(), "kv_profile_begin")


def kv_profile_end(max_entries: int = 16):
    """Per-kernel {name: (launches, ms, bytes)} since kv_profile_begin."""
    arr = (kv_kernel_stat * max_entries)()
    n = _check(_lib.kv_profile_end(arr, max_entries), "kv_profile_end")
    return {arr[i].name.decode(): (arr[i].launches, arr[i].ms, arr[i].bytes)
            for i in range(min(n, max_entries))}


def kv_profile_last_window() -> dict:
    """Union of the timed kernel intervals of the window kv_profile_end last
    closed: {span_ms, hbm_busy_ms, hbm_bytes, hbm_launches, link_busy_ms,
    link_bytes, link_launches}."""
    w = kv_profile_window()
    _check(_lib.kv_profile_last_window(ctypes.byref(w)), "kv_profile_last_window")
    return {name: getattr(w, name) for name, _ in kv_profile_window._fields_}
