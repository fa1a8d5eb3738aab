"""Benchmark of the KV buffered-copy path on one MI355X.

By default one step is one pass of the whole path over one batch of the
100K-context workload (LongStep below: 60 layers, 4 rows of U{20000..99936}
tokens, 8 KV heads, D=128, bf16, Smax=100000; 98.3 GB of caches):

  1. row swap: the row with the longest context is packed and swapped out
     to pinned host memory while that row's previous image is swapped into a
     free one-row slot (both link directions at once);
  2. prompt streaming: every row's prompt leaves layer by layer in
     4096-token chunks, each chunk packed into a staging bank and copied to
     pinned host memory while the next chunk is packed;
  3. decode: 64 single-token packs at each row's own position into a
     16-slot staging ring gathered at flush, flushed to pinned host memory
     when full, then restored into the cache.

Host images are double-buffered across steps, so each step's inbound
transfers read what an earlier step wrote.  Each workload's step runs with
the transport listed in DEFAULT_TRANSPORT unless --transport names another.
Inputs are resident in HBM before the timed region.  `value` is the KV
payload the step moves across the host link (both directions) per second.
`roofline` describes the pack/unpack kernel with the most GPU time:
algorithmic bytes (payload read + payload written) per launch over its
average duration, both measured live with hipEvents bound to every launch's
dispatch (the kernel's own begin and end timestamps).  `cpu_baseline` is the
oracle on a bounded sample of the same step (single-threaded; its
`all_cores` entry runs the same calls in pieces over the host's cores).
`metric_parts` sets the metric's two figures side by side (host-link rates
per direction against PCIe peak; the dominant kernel's algorithmic, payload
and counted-traffic rates against HBM peak and, with the detail, against
the plain-copy ceiling); `context` puts the pages' own figures beside what
is measured here (the link's rate, and with the detail the gains of
buffered copies and of streaming beside compute); `detail` holds every kernel's launches and rates and the
isolated measurements (link and HBM copy ceilings, large slices, decode
loops, a decode step sent buffered against one copy call per region,
layer-by-layer prompt streaming against streaming after the prompt, decode
steps streamed through the ring beside compute against compute that waits
for each flush, the microbatch schedule, the 2 x 2 repartition).

`--workload` selects the other shapes, each with the step its class below
describes: gpt2-1.5b (StreamStep: prompt streaming of 48 layers beside the
load of an earlier prompt image, 24 ring pushes with 3 flushes and a ring
restore, and a microbatch swap-out beside a swap-in), opt-66b-16l (RingStep:
the decode ring of a 16-layer OPT-66B stage), bloom-176b-10l (SwapStep:
duplex microbatch swapping on a 10-layer BLOOM-176B stage, plus the
steady-state schedule against its Appendix E prediction), gpt2-small-tiny
(the GPT-2-1.5B step at GPT-2-small size).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# A step drives up to eight streams (compute streams, one copy stream per link
# direction, the swap stream of the microbatch schedule) besides the default
# one.  HIP maps streams onto a fixed number of hardware queues per process;
# with fewer queues than streams, streams share a queue and their work
# serialises: the two link directions stop overlapping, and a swap-in waits
# behind the compute it should hide under.  Ask for sixteen (must happen before
# the HIP runtime starts).
if int(os.environ.get("GPU_MAX_HW_QUEUES", "0") or 0) < 16:
    os.environ["GPU_MAX_HW_QUEUES"] = "16"

METRIC = "KV pack/unpack GB/s (% HBM peak) + swap host-link GB/s, 1 MI355X"
# The pages' own figures around this path (other hardware; context, not targets):
# DejaVu's serving throughput over FasterTransformer, the estimate of one
# 2048-token OPT-175B prompt-KV transfer (9 GiB) over eight PCIe 5.0 x16 links,
# the gain of buffered copies over one copy call per small region when
# streaming a request's cache out (prompt 500, 500 new tokens), and the further
# gain of streaming layer by layer and overlapping it with compute.
PAGES_THROUGHPUT_VS_FT = "1.88x (OPT-66B), 2x (BLOOM-176B): system throughput on A100-80GB / V100-16GB clusters"
PAGES_OPT175B_KV_BYTES = 2048 * 4.5 * (1 << 20)   # 2048 tokens x 4.5 MiB
PAGES_OPT175B_ESTIMATE_MS = 17.6                  # over 8 links of 64 GB/s
PAGES_BUFFERED_GAIN = "95x: buffered copies over many small copy calls, streaming to remote CPU memory"
PAGES_OVERLAP_GAIN = "1.4x more: layer-by-layer prompt streaming and token streaming overlapped with compute"
HBM_PEAK_GBPS = 8000.0
PCIE_PEAK_GBPS = 63.0          # PCIe 5.0 x16, per direction

RING_GATHER = 1   # kv_ring_gather of the rings the steps use (set from --ring-gather)
WHOLE_CALLS = True   # swaps of complete images as one call each (set from --swap-calls)


_T0 = time.perf_counter()


def progress(msg):
    """One line on stderr as each phase of the run ends (stdout holds only the
    result line)."""
    print(f"[bench {time.perf_counter() - _T0:7.1f} s] {msg}", file=sys.stderr, flush=True)


def counters_file(workload, kernel_name):
    return os.path.join(ROOT, "profiles", f"traffic_{kernel_name}_{workload}.txt")


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="gqa-100k", choices=sorted(STEPS),
                    help="gqa-100k (the largest workload that fits one GPU) is the headline; "
                         "the others measure the remaining workloads")
    ap.add_argument("--swap-bank-mib", type=int, default=None,
                    help="banks of the swap engines in MiB (default: the workload's entry in "
                         "DEFAULT_SWAP_BANK_MIB, else 256; 0 for the BLOOM step: one layer)")
    ap.add_argument("--transport", choices=("auto", "kernel", "runtime", "dma", "dma_out", "engine"),
                    default=None,
                    help="bank<->host transfers (see kv_transport in include/kvstream.h); "
                         "default: the workload's entry in DEFAULT_TRANSPORT")
    ap.add_argument("--ring-gather", choices=("flush", "each"), default="flush",
                    help="rings pack a bank's decode steps at flush time in one pass (flush) or "
                         "each step as it is pushed (each); see kv_ring_set_gather")
    ap.add_argument("--swap-calls", choices=("whole", "layer"), default="whole",
                    help="gpt2 shapes: a complete host image (prompt load, microbatch swap) moves "
                         "in one call the engine chunks by bank (whole) or in one call per layer")
    ap.add_argument("--row-transport", choices=("auto", "kernel", "runtime", "dma", "dma_out",
                                                "engine"), default=None,
                    help="gqa-100k: transport of the row swap (default: --transport)")
    ap.add_argument("--prompt-engines", default=None,
                    help="gqa-100k with --transport engine: comma-separated DMA engines (0-3, or "
                         "-1 for an idle one at each copy) of the prompt-streaming handles; "
                         "chunks alternate over the handles, each with its own copy stream "
                         "(bloom-176b-10l: the same for its swap-out handles, by layer; "
                         "gpt2 shapes: the engines of the prompt, ring and swap-out handles)")
    ap.add_argument("--row-engines", default=None,
                    help="gqa-100k with --row-transport engine: DMA engines of the row swap-out "
                         "handles (the layers split into contiguous ranges over them)")
    ap.add_argument("--row-bank-mib", type=int, default=None,
                    help="gqa-100k: banks of the row swap (0: the whole row image)")
    ap.add_argument("--row-first", type=int, choices=(0, 1), default=None,
                    help="gqa-100k: the prompt's copies wait for the row swap-out's (1)")
    ap.add_argument("--row-in-transport", choices=("auto", "kernel", "runtime", "dma", "dma_out",
                                                   "engine"), default=None,
                    help="gqa-100k: transport of the row swap-in (default: --row-transport)")
    ap.add_argument("--row-in-after", type=int, choices=(0, 1), default=None,
                    help="gqa-100k: the row swap-in's copies wait for the row swap-out's (1)")
    ap.add_argument("--row-link-blocks", type=int, default=None,
                    help="gqa-100k: link-copy workgroups of the row swap-out (KV_OPT_LINK_BLOCKS)")
    ap.add_argument("--link-blocks", type=int, default=None,
                    help="bloom-176b-10l: link-copy workgroups of the swap-out (KV_OPT_LINK_BLOCKS)")
    ap.add_argument("--ring-duplex", type=int, choices=(0, 1), default=None,
                    help="opt-66b-16l: restore the image the other ring flushed in the previous "
                         "step while this step's flushes go out (1), or flush and then restore "
                         "the same ring's image (0); default: DEFAULT_RING_DUPLEX")
    ap.add_argument("--compute-streams", type=int, choices=(1, 2), default=2,
                    help="gpt2 shapes: packs and unpacks of the two link directions on one "
                         "compute stream (1) or one each (2)")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-detail", action="store_true",
                    help="skip the isolated measurements after the timed steps (ceilings, large "
                         "slices, schedule): a kernel trace then holds the steps' launches only")
    ap.add_argument("--slices-only", action="store_true",
                    help="run only the isolated large-slice calls of the workload (the ones the "
                         "70%%-of-peak bar applies to; for gpt2-1.5b also the paged-pool calls, "
                         "for opt-66b-16l the split/merge calls) and print their rates: a "
                         "profiler run then holds those launches alone")
    ap.add_argument("--no-profile", action="store_true",
                    help="do not time launches with events (for external profilers)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this size (counter calibration)")
    return ap.parse_args()


class StreamStep:
    """Prompt streaming, decode ring and microbatch swap of a uniform-prompt
    workload (the GPT-2 shapes), following the DejaVu workers' dataflow:

      1. prompt streaming (prompt worker): the prompt layers of cache A are
         packed layer by layer and copied to pinned host memory;
      2. prompt load (token worker): the prompt image streamed in the
         previous step -- a different request, already in host memory -- is
         copied back through the banks and unpacked into cache B layer by
         layer, while (1) runs: the two link directions carry independent
         data;
      3. decode: single-token packs of cache B at the positions after the
         prompt into the staging ring, flushed to pinned host memory when
         full (replication);
      4. restore: the ring's host image is unpacked into cache D (recovery
         on a fresh worker);
      5. microbatch swap: cache B (microbatch x-1, every position) is
         swapped out layer by layer while microbatch x+1 is swapped in to
         cache C from its host image, duplex."""

    def __init__(self, w, swap_bank_bytes, transport=0, out_engines=None):
        """out_engines: with the engine transport, the DMA engines of the
        device->host handles (prompt streaming, staging ring, swap-out), or
        None for the workload's default (an idle one at each copy)."""
        import torch

        import kv_cache_streaming_amd as kv
        import synth
        self.kv, self.w, self.torch = kv, w, torch
        L, B, H, D, S = w.dims
        self.lay = kv.kv_layout_init(L, B, H, D, S, w.dtype)
        n = L * B * H * D * S
        dev = torch.device("cuda")
        self.caches = {}
        for i, name in enumerate("ABCD"):
            k = torch.empty(n, dtype=torch.int16, device=dev)
            v = torch.empty(n, dtype=torch.int16, device=dev)
            synth.fill_device_cache(k, w.value_seed + 100 * i, w.dtype)
            synth.fill_device_cache(v, w.value_seed + 100 * i + 1, w.dtype)
            self.caches[name] = (k, v)
        self.prompt = int(w.prompt_len)
        self.rows_start = [0] * B
        self.rows_prompt = [self.prompt] * B
        self.rows_full = [self.prompt + w.decode_steps] * B
        self.layer_prompt = kv.kv_pack_bytes(self.lay, 1, self.rows_prompt)
        self.layer_full = kv.kv_pack_bytes(self.lay, 1, self.rows_full)
        self.slot = kv.kv_pack_bytes(self.lay, L, None, 1)

        def bank(nbytes):
            return torch.empty((nbytes + 1) // 2, dtype=torch.int16, device=dev)

        def pinned(nbytes):
            return torch.empty((nbytes + 1) // 2, dtype=torch.int16, pin_memory=True)

        # four streams: prompt-side compute, token-side compute, and one copy
        # stream per link direction (engines of one direction share it)
        self.s = {name: torch.cuda.Stream() for name in ("p", "t", "d2h", "h2d")}
        pb = max(self.layer_prompt, 1)
        sb = swap_bank_bytes
        x = transport
        self.eng_p = kv.KvSwap(self.lay, bank(pb), bank(pb), pb, self.s["d2h"], x)
        self.eng_t = kv.KvSwap(self.lay, bank(pb), bank(pb), pb, self.s["h2d"], x)
        self.eng_o = kv.KvSwap(self.lay, bank(sb), bank(sb), sb, self.s["d2h"], x)
        self.eng_i = kv.KvSwap(self.lay, bank(sb), bank(sb), sb, self.s["h2d"], x)
        R = w.ring_slots
        self.ring_host = pinned(w.decode_steps * self.slot)
        self.ring = kv.KvRing(self.lay, R, bank(R * self.slot), bank(R * self.slot),
                              self.ring_host, copy_stream=self.s["d2h"], transport=x)
        if out_engines is None:
            out_engines = default_out_engines(w.name)
        if out_engines and x == TRANSPORTS["engine"]:
            for h, e in zip((self.eng_p, self.ring, self.eng_o), out_engines):
                h.set_option(kv.KV_OPT_DMA_ENGINE, e)
        self.ring.set_gather(RING_GATHER)
        # double-buffered host images: one written this step, one read
        self.host_p = [pinned(L * self.layer_prompt) for _ in range(2)]
        self.host_s = [pinned(L * self.layer_full) for _ in range(2)]
        self.k = 0
        self.positions = [[self.prompt + j] * B for j in range(w.decode_steps)]

    def link_bytes(self):
        return self.link_bytes_out() + self.link_bytes_in()

    def link_bytes_out(self):
        """prompt streaming, ring flushes, microbatch swap-out"""
        L = self.w.L
        return L * self.layer_prompt + self.w.decode_steps * self.slot + L * self.layer_full

    def link_bytes_in(self):
        """prompt load, ring restore, microbatch swap-in"""
        return self.link_bytes_out()

    def ceiling_caches(self):
        return self.caches["B"], self.caches["C"]

    def run(self):
        torch, w = self.torch, self.w
        L = w.L
        A, Bc, Cc, Dc = (self.caches[n] for n in "ABCD")
        sp, st = self.s["p"], self.s["t"]
        out, inn = self.k % 2, (self.k + 1) % 2
        self.k += 1
        hp_out, hp_in = self.host_p[out].data_ptr(), self.host_p[inn].data_ptr()
        hs_out, hs_in = self.host_s[out].data_ptr(), self.host_s[inn].data_ptr()
        lp, lf = self.layer_prompt, self.layer_full
        # 1+2: prompt streaming out of A || loading an earlier prompt into B
        if WHOLE_CALLS:
            # the earlier prompt is complete on the host: one call, chunked by
            # the engine into bank-sized pieces
            self.eng_t.swap_in(Bc[0], Bc[1], 0, L, self.rows_start, self.rows_prompt, hp_in,
                               L * lp, st)
        for l in range(L):
            self.eng_p.stream_prompt_layer(A[0], A[1], l, 0, self.prompt, None,
                                           hp_out + l * lp, lp, sp)
            if not WHOLE_CALLS:
                self.eng_t.swap_in(Bc[0], Bc[1], l, 1, self.rows_start, self.rows_prompt,
                                   hp_in + l * lp, lp, st)
        # 3: decode steps of B into the staging ring
        self.ring.reset()
        for pos in self.positions:
            self.ring.push(Bc[0], Bc[1], pos, st)
        self.ring.flush(st)
        # 4: restore the ring into D
        self.ring.restore(Dc[0], Dc[1], st)
        # 5: swap out microbatch x-1 (B) || swap in microbatch x+1 (into C)
        if WHOLE_CALLS:
            self.eng_o.swap_out(Bc[0], Bc[1], 0, L, self.rows_start, self.rows_full, hs_out,
                                L * lf, st)
            self.eng_i.swap_in(Cc[0], Cc[1], 0, L, self.rows_start, self.rows_full, hs_in,
                               L * lf, sp)
        else:
            for l in range(L):
                self.eng_o.swap_out(Bc[0], Bc[1], l, 1, self.rows_start, self.rows_full,
                                    hs_out + l * lf, lf, st)
                self.eng_i.swap_in(Cc[0], Cc[1], l, 1, self.rows_start, self.rows_full,
                                   hs_in + l * lf, lf, sp)
        torch.cuda.synchronize()

    def run_one_stream(self):
        """The same step with every pack and unpack on one compute stream: a
        direction's pack (or unpack) of layer l+1 is enqueued before the other
        direction's unpack of layer l, so each link keeps a bank ready while
        the HBM kernels run one at a time instead of splitting the bandwidth."""
        torch, w = self.torch, self.w
        L = w.L
        A, Bc, Cc, Dc = (self.caches[n] for n in "ABCD")
        c = self.s["p"]
        out, inn = self.k % 2, (self.k + 1) % 2
        self.k += 1
        hp_out, hp_in = self.host_p[out].data_ptr(), self.host_p[inn].data_ptr()
        hs_out, hs_in = self.host_s[out].data_ptr(), self.host_s[inn].data_ptr()
        lp, lf = self.layer_prompt, self.layer_full
        for l in range(L + 1):
            if l < L:
                self.eng_p.stream_prompt_layer(A[0], A[1], l, 0, self.prompt, None,
                                               hp_out + l * lp, lp, c)
            if l >= 1:
                self.eng_t.swap_in(Bc[0], Bc[1], l - 1, 1, self.rows_start, self.rows_prompt,
                                   hp_in + (l - 1) * lp, lp, c)
        self.ring.reset()
        for pos in self.positions:
            self.ring.push(Bc[0], Bc[1], pos, c)
        self.ring.flush(c)
        self.ring.restore(Dc[0], Dc[1], c)
        for l in range(L + 1):
            if l < L:
                self.eng_o.swap_out(Bc[0], Bc[1], l, 1, self.rows_start, self.rows_full,
                                    hs_out + l * lf, lf, c)
            if l >= 1:
                self.eng_i.swap_in(Cc[0], Cc[1], l - 1, 1, self.rows_start, self.rows_full,
                                   hs_in + (l - 1) * lf, lf, c)
        torch.cuda.synchronize()


def _pinned(torch, nbytes):
    return torch.empty((nbytes + 1) // 2, dtype=torch.int16, pin_memory=True)


class HostBuffer:
    """Page-locked host memory of exactly `nbytes` (hipHostMalloc).  torch rounds
    a pinned request up to a power of two, which for host images of tens of GB
    nearly doubles the page-locked footprint."""

    def __init__(self, kv, nbytes):
        lib = kv._lib      # resolves to the HIP runtime the library and torch share
        lib.hipHostMalloc.restype = ctypes.c_int
        lib.hipHostMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t,
                                      ctypes.c_uint]
        lib.hipHostFree.restype = ctypes.c_int
        lib.hipHostFree.argtypes = [ctypes.c_void_p]
        self._free = lib.hipHostFree
        p = ctypes.c_void_p()
        r = lib.hipHostMalloc(ctypes.byref(p), nbytes, 0)
        if r != 0 or not p.value:
            raise MemoryError(f"hipHostMalloc of {nbytes} bytes failed (hipError {r})")
        self.ptr, self.nbytes = p.value, nbytes

    def data_ptr(self):
        return self.ptr

    def close(self):
        if getattr(self, "ptr", None):
            self._free(self.ptr)
            self.ptr = None

    __del__ = close


class TimingEvent:
    """A HIP event for timing only: created with hipEventDisableSystemFence, so
    recording it does not write back and invalidate the caches (a default
    event does, which adds that cost to the interval it closes and slows the
    work after it).  Same use as torch.cuda.Event(enable_timing=True)."""

    _lib = None

    def __init__(self):
        import kv_cache_streaming_amd as kv
        lib = TimingEvent._lib
        if lib is None:
            lib = kv._lib      # resolves to the HIP runtime the library and torch share
            lib.hipEventCreateWithFlags.restype = ctypes.c_int
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.restype = ctypes.c_int
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.restype = ctypes.c_int
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            lib.hipEventDestroy.restype = ctypes.c_int
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            TimingEvent._lib = lib
        e = ctypes.c_void_p()
        r = lib.hipEventCreateWithFlags(ctypes.byref(e), 0x20000000)   # hipEventDisableSystemFence
        if r != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed (hipError {r})")
        self.e = e.value

    def record(self, stream=None):
        import torch
        s = stream if stream is not None else torch.cuda.current_stream()
        r = self._lib.hipEventRecord(self.e, s.cuda_stream)
        if r != 0:
            raise RuntimeError(f"hipEventRecord failed (hipError {r})")

    def elapsed_time(self, end):
        """Milliseconds from this event to `end` (both complete)."""
        ms = ctypes.c_float()
        r = self._lib.hipEventElapsedTime(ctypes.byref(ms), self.e, end.e)
        if r != 0:
            raise RuntimeError(f"hipEventElapsedTime failed (hipError {r})")
        return ms.value

    def __del__(self):
        if getattr(self, "e", None) and self._lib is not None:
            self._lib.hipEventDestroy(self.e)
            self.e = None


def _bank(torch, nbytes):
    return torch.empty((nbytes + 1) // 2, dtype=torch.int16, device="cuda")


def _filled_cache(torch, w, seed):
    import synth
    n = w.L * w.B * w.H * w.D * w.Smax
    k = torch.empty(n, dtype=torch.int16, device="cuda")
    v = torch.empty(n, dtype=torch.int16, device="cuda")
    synth.fill_device_cache(k, seed, w.dtype)
    synth.fill_device_cache(v, seed + 1, w.dtype)
    return k, v


def _duplex_layers(eng_o, eng_i, src, dst, L, start, count, img_out, img_in, per_layer, s_out,
                   s_in, packed):
    """Layer-pipelined swap-out of `src` || swap-in into `dst`, where `dst` may be
    the region `src` is leaving: the unpack of layer l waits for the pack of
    layer l (event `packed[l]`), nothing else couples the two directions.
    `eng_o` may be a list of swap-out handles: layers alternate over them."""
    outs = eng_o if isinstance(eng_o, list) else [eng_o]
    for l in range(L):
        outs[l % len(outs)].swap_out(src[0], src[1], l, 1, start, count, img_out + l * per_layer,
                                     per_layer, s_out)
        packed[l].record(s_out)
        s_in.wait_event(packed[l])
        eng_i.swap_in(dst[0], dst[1], l, 1, start, count, img_in + l * per_layer, per_layer, s_in)


class RingStep:
    """Decode leg of one token-generation stage of a pipeline: the 16-layer
    OPT-66B slice, ragged current lengths U{256..1800}.  One step = 64 decode
    steps of cache A (one token per row at len_b + j) packed into a 16-slot
    staging ring and flushed to pinned host memory every 16 steps, and a
    ring's host image of 64 steps restored into cache D (recovery on a fresh
    worker).  Duplex (the default): two rings take turns, and the restore
    reads the image the other ring flushed in the previous step while this
    step's flushes go out, each ring on a copy stream of its own, so the two
    link directions run at once; otherwise one ring flushes and then restores
    its own image."""

    def __init__(self, w, swap_bank_bytes, transport=0, out_engines=None, duplex=None):
        """out_engines: with the engine transport, [engine] pins the ring's
        flush copies to that DMA engine (None: an idle one at each copy);
        duplex: None for the workload's default (DEFAULT_RING_DUPLEX)."""
        import torch

        import kv_cache_streaming_amd as kv
        import synth
        self.kv, self.w, self.torch = kv, w, torch
        self.duplex = DEFAULT_RING_DUPLEX.get(w.name, False) if duplex is None else duplex
        self.lay = kv.kv_layout_init(*w.dims, w.dtype)
        self.A = _filled_cache(torch, w, w.value_seed)
        self.D = _filled_cache(torch, w, w.value_seed + 300)
        self.positions = [list(map(int, p)) for p in synth.decode_positions(w)]
        self.slot = kv.kv_pack_bytes(self.lay, w.L, None, 1)
        self.s = {name: torch.cuda.Stream() for name in ("t", "r")}
        R = w.ring_slots
        if out_engines is None:
            out_engines = default_out_engines(w.name)
        self.rings, self.ring_hosts = [], []
        for i in range(2 if self.duplex else 1):
            host = _pinned(torch, w.decode_steps * self.slot)
            ring = kv.KvRing(self.lay, R, _bank(torch, R * self.slot), _bank(torch, R * self.slot),
                             host, copy_stream=torch.cuda.Stream(), transport=transport)
            ring.set_gather(RING_GATHER)
            if out_engines and transport == TRANSPORTS["engine"]:
                ring.set_option(kv.KV_OPT_DMA_ENGINE, out_engines[0])
            self.rings.append(ring)
            self.ring_hosts.append(host)
        self.k = 0

    def link_bytes(self):
        return self.link_bytes_out() + self.link_bytes_in()

    def link_bytes_out(self):
        """ring flushes"""
        return self.w.decode_steps * self.slot

    def link_bytes_in(self):
        """ring restore"""
        return self.w.decode_steps * self.slot

    def ceiling_caches(self):
        return self.A, self.D

    def run(self):
        st = self.s["t"]
        out = self.rings[self.k % len(self.rings)]
        if self.duplex:
            # the image flushed in the previous step (none before the first)
            self.rings[(self.k + 1) % 2].restore(self.D[0], self.D[1], self.s["r"])
        self.k += 1
        out.reset()
        for pos in self.positions:
            out.push(self.A[0], self.A[1], pos, st)
        out.flush(st)
        if not self.duplex:
            out.restore(self.D[0], self.D[1], st)
        self.torch.cuda.synchronize()

    def cpu_ops(self):
        """(layer-0 source, per-op (name, start, count)) for the oracle sample."""
        B = self.w.B
        return self.A, [("decode pack", p, [1] * B) for p in self.positions]

    def repartition(self, kv, reps=3):
        """stream_out / stream_in of the slice's prompt region (every row's
        current length) into 2 pipeline stages x 2 tensor-parallel ranks:
        each piece is 8 layers x 36 heads; rates in HBM bytes (read + write of
        the piece) per second, pieces timed one after another with events."""
        import synth
        torch, w, lay = self.torch, self.w, self.lay
        L, B, H = w.L, w.B, w.H
        src = (0, L, 0, H, 0, B)
        lens = [int(x) for x in synth.row_lengths(w)]
        start = [0] * B
        dsts = [(l0, L // 2, h0, H // 2, 0, B) for l0 in (0, L // 2) for h0 in (0, H // 2)]
        nbytes = kv.kv_stream_bytes(lay, src, dsts[0], lens)
        dlay = kv.kv_layout_init(L // 2, B, H // 2, w.D, w.Smax, w.dtype)
        dn = (L // 2) * B * (H // 2) * w.D * w.Smax
        caches = [(torch.empty(dn, dtype=torch.int16, device="cuda"),
                   torch.empty(dn, dtype=torch.int16, device="cuda")) for _ in dsts]
        st = [torch.empty(nbytes // 2, dtype=torch.int16, device="cuda") for _ in dsts]
        s = self.s["t"]
        out = {"pieces": len(dsts), "piece_bytes": nbytes}
        for name in ("stream_out", "stream_in"):
            def run():
                for i, d in enumerate(dsts):
                    if name == "stream_out":
                        kv.kv_stream_out(lay, src, self.A[0], self.A[1], d, start, lens, st[i],
                                         nbytes, s)
                    else:
                        kv.kv_stream_in(dlay, d, caches[i][0], caches[i][1], src, start, lens,
                                        st[i], nbytes, s)
            secs = [x / len(dsts) for x in rep_seconds(torch, run, s)]
            rate_entry(out, name + "_per_piece", secs, 2 * nbytes, HBM_PEAK_GBPS, "_hbm_GBps")
        del caches, st
        return out


class SwapStep:
    """Microbatch swapping on one stage: the 10-layer BLOOM-176B slice, 16 rows
    of 1500 tokens per microbatch, four microbatches with a host image each
    (13.76 GB) and two device slots.  One step = one round of the round-robin:
    while microbatch x computes in one slot, microbatch x-1 is swapped out of
    the other slot layer by layer and microbatch x+1 is swapped into it, each
    layer's unpack waiting only for that layer's pack (both link directions at
    once)."""

    def __init__(self, w, swap_bank_bytes, transport=0, out_engines=None, link_blocks=None):
        """out_engines: with the engine transport, the DMA engines of the
        swap-out handles (layers alternate over them, each handle with its own
        copy stream); None: one handle, an idle engine at each copy.
        link_blocks: workgroups of the swap-out's link-copy kernel
        (KV_OPT_LINK_BLOCKS; None: the library's default)."""
        import torch

        import kv_cache_streaming_amd as kv
        self.kv, self.w, self.torch = kv, w, torch
        L, B = w.L, w.B
        self.lay = kv.kv_layout_init(*w.dims, w.dtype)
        self.rows_start = [0] * B
        self.rows = [w.prompt_len] * B
        self.per_layer = kv.kv_pack_bytes(self.lay, 1, self.rows)
        self.image = L * self.per_layer
        self.N = w.microbatches
        n = L * B * w.H * w.D * w.Smax
        self.slots = [(torch.empty(n, dtype=torch.int16, device="cuda"),
                       torch.empty(n, dtype=torch.int16, device="cuda")) for _ in range(2)]
        self.host = HostBuffer(kv, self.N * self.image)
        self.img = [self.host.data_ptr() + x * self.image for x in range(self.N)]
        self.s = {name: torch.cuda.Stream() for name in ("out", "in", "d2h", "h2d", "swap")}
        # 0: banks of one layer of a microbatch
        sb = swap_bank_bytes or (-(-self.per_layer // (1 << 20)) << 20)
        self.eng_o = kv.KvSwap(self.lay, _bank(torch, sb), _bank(torch, sb), sb, self.s["d2h"],
                               transport)
        self.eng_out = [self.eng_o]
        if out_engines is None:
            out_engines = default_out_engines(w.name)
        if out_engines and transport == TRANSPORTS["engine"]:
            self.eng_o.set_option(kv.KV_OPT_DMA_ENGINE, out_engines[0])
            for e in out_engines[1:]:
                h = kv.KvSwap(self.lay, _bank(torch, sb), _bank(torch, sb), sb,
                              torch.cuda.Stream(), transport)
                h.set_option(kv.KV_OPT_DMA_ENGINE, e)
                self.eng_out.append(h)
        if link_blocks:
            for h in self.eng_out:
                h.set_option(kv.KV_OPT_LINK_BLOCKS, link_blocks)
        self.eng_i = kv.KvSwap(self.lay, _bank(torch, sb), _bank(torch, sb), sb, self.s["h2d"],
                               transport)
        self.packed = [torch.cuda.Event() for _ in range(L)]
        # every microbatch's host image, written through a swap-out of a slot
        # filled with that microbatch's values; the slots end as round 0
        # expects them: microbatch 0 in slot 0 (computing), N-1 in slot 1
        # (to be swapped out while 1 comes in)
        import synth
        for x in list(range(1, self.N)) + [0]:
            k, v = self.slots[0 if x == 0 else 1]
            synth.fill_device_cache(k, w.value_seed + 40 * x, w.dtype)
            synth.fill_device_cache(v, w.value_seed + 40 * x + 1, w.dtype)
            torch.cuda.synchronize()
            self.eng_o.swap_out(k, v, 0, L, self.rows_start, self.rows, self.img[x], self.image,
                                torch.cuda.current_stream())
            torch.cuda.synchronize()
        self.r = 0

    def link_bytes(self):
        return self.link_bytes_out() + self.link_bytes_in()

    def link_bytes_out(self):
        """swap-out of microbatch x-1"""
        return self.image

    def link_bytes_in(self):
        """swap-in of microbatch x+1"""
        return self.image

    def ceiling_caches(self):
        return self.slots[0], self.slots[1]

    def run(self):
        N, r = self.N, self.r
        self.r += 1
        x = r % N
        other = self.slots[(r + 1) % 2]          # holds x-1, receives x+1
        _duplex_layers(self.eng_out, self.eng_i, other, other, self.w.L, self.rows_start, self.rows,
                       self.img[(x - 1) % N], self.img[(x + 1) % N], self.per_layer,
                       self.s["out"], self.s["in"], self.packed)
        self.torch.cuda.synchronize()

    def cpu_ops(self):
        return self.slots[0], [("swap pack", self.rows_start, self.rows)] * self.w.L

    def schedule(self, kv, rounds_per_mb=2, steady_from=2):
        """The steady-state schedule of the pages' microbatch swapping: after
        each decode step of microbatch x, only that step's new tokens go out
        (an incremental swap-out through a staging ring) while microbatch x+2
        comes back into the slot x leaves, during the step of x+1.  A round
        costs max(t, transfer) for a decode step of t seconds; the rows below
        hold the measured round time against that figure for a few t, with t
        played by a timed busy-wait on the compute stream."""
        import numpy as np
        torch, w, lay = self.torch, self.w, self.lay
        L, B, N = w.L, w.B, self.N
        slot = kv.kv_pack_bytes(lay, L, None, 1)
        rounds = N * rounds_per_mb
        rings = [kv.KvRing(lay, 1, _bank(torch, slot), _bank(torch, slot),
                           _pinned(torch, rounds_per_mb * slot), copy_stream=self.s["d2h"])
                 for _ in range(N)]
        rng = np.random.default_rng(7)
        new = torch.from_numpy(rng.integers(-32768, 32768, size=slot // 2, dtype=np.int16)).cuda()
        by_addr = {t.data_ptr(): t for pair in self.slots for t in pair}
        c = torch.cuda.Stream()
        # busy-wait calibration: cycles per millisecond of the sleep kernel
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(c):
            torch.cuda._sleep(1000)
            e0.record(c)
            torch.cuda._sleep(2_000_000)
            e1.record(c)
        torch.cuda.synchronize()
        cycles_per_ms = 2_000_000 / e0.elapsed_time(e1)
        # transfer time of one image alone (swap-in of a whole microbatch)
        t0 = time.perf_counter()
        self.eng_i.swap_in(self.slots[0][0], self.slots[0][1], 0, L, self.rows_start, self.rows,
                           self.img[0], self.image, c)
        torch.cuda.synchronize()
        transf = time.perf_counter() - t0
        bw = self.image / transf
        C = 2 * L * w.H * w.D * 2
        out = {"microbatches": N, "device_slots": 2, "rounds": rounds,
               "image_bytes": self.image, "step_update_bytes": slot,
               "swap_in_alone_ms": round(transf * 1000, 2), "swap_in_alone_GBps": round(bw / 1e9, 2),
               "rows": []}
        for t_ms in (0.0, 0.5 * transf * 1000, 2.0 * transf * 1000):
            for rg in rings:
                rg.reset()
            m = kv.KvMbSwap(lay, self.slots, self.eng_i, rings, self.img, [self.image] * N,
                            [w.prompt_len] * (N * B), self.s["swap"])
            torch.cuda.synchronize()
            m.start(c)
            marks = []
            gen = [0] * N
            for r in range(rounds):
                ev = torch.cuda.Event(enable_timing=True)
                ev.record(c)
                marks.append(ev)
                x, ka, va = m.current()
                if t_ms > 0:
                    with torch.cuda.stream(c):
                        torch.cuda._sleep(int(t_ms * cycles_per_ms))
                pos = [w.prompt_len + gen[x]] * B
                kv.kv_unpack_tokens(lay, by_addr[ka], by_addr[va], 0, L, pos, [1] * B, new, slot, c)
                m.round(pos, c)
                gen[x] += 1
            end = torch.cuda.Event(enable_timing=True)
            end.record(c)
            marks.append(end)
            torch.cuda.synchronize()
            per = [marks[i].elapsed_time(marks[i + 1]) for i in range(steady_from, rounds)]
            pays, lhs, rhs = kv.kv_swap_pays(64, t_ms / 1000, w.prompt_len, B, C, bw)
            out["rows"].append({"t_ms": round(t_ms, 2),
                                "round_ms_median": round(float(np.median(per)), 2),
                                "predicted_round_ms": round(max(t_ms, transf * 1000), 2),
                                "appendix_e_64_tokens": {"pays": pays, "lhs_s": round(lhs, 3),
                                                         "rhs_s": round(rhs, 3)}})
            m.close()
        for rg in rings:
            rg.close()
        return out


class LongStep:
    """The 100K-context workload: 60 layers, 4 rows, 8 KV heads, D=128, bf16,
    current lengths U{20000..99936}.  One step = the row of the longest context
    swapped out to pinned host memory while its previous image is swapped
    into a free one-row slot (a cache of its own, as a swapped-in request
    lands in a free slot; both directions at once), the whole prompt of every
    row streamed out in 4096-token chunks per layer, and 64 decode steps
    through a 16-slot staging ring restored into the cache."""

    def __init__(self, w, swap_bank_bytes, transport=0, row_transport=None, prompt_engines=None,
                 row_link_blocks=None, row_engines=None, row_first=None, row_bank_bytes=None,
                 row_in_transport=None, row_in_after=None):
        """row_transport: the row swap's kv_transport (None: the workload's
        default, else `transport`); prompt_engines: DMA engines of the
        prompt-streaming handles with the engine transport (None: the
        workload's default); row_link_blocks: link-copy workgroups of the
        row swap-out (None: the workload's default); row_engines: with the
        engine transport for the row, the DMA engines of its swap-out handles
        (the layers split into as many contiguous ranges, one call each);
        row_first: the prompt's copies start once the row swap-out's copies
        are done (the two outgoing legs take the link one after the other);
        row_bank_bytes: the row swap's banks (None: the workload's default;
        0: the whole row image, packed in one pass before its copy and
        unpacked in one pass after it); row_in_transport: the row swap-in's
        kv_transport (None: the workload's default, else the row swap's);
        row_in_after: the row swap-in's copies start once the row swap-out's
        copies are done."""
        import torch

        import kv_cache_streaming_amd as kv
        import synth
        self.kv, self.w, self.torch = kv, w, torch
        L, B = w.L, w.B
        if row_transport is None:
            row_transport = TRANSPORTS.get(DEFAULT_ROW_TRANSPORT.get(w.name), transport)
        if prompt_engines is None:
            prompt_engines = [int(x) for x in DEFAULT_PROMPT_ENGINES.get(w.name, "-1").split(",")]
        if row_link_blocks is None:
            row_link_blocks = DEFAULT_ROW_LINK_BLOCKS.get(w.name, 0)
        if row_engines is None:
            row_engines = [int(x) for x in DEFAULT_ROW_ENGINES.get(w.name, "-1").split(",")]
        self.row_first = DEFAULT_ROW_FIRST.get(w.name, False) if row_first is None else row_first
        self.row_in_after = bool(row_in_after)
        if row_in_transport is None:
            row_in_transport = row_transport
        if row_bank_bytes is None:
            row_bank_bytes = DEFAULT_ROW_BANK_MIB.get(w.name, swap_bank_bytes >> 20) << 20
        self.row_done = torch.cuda.Event()
        self.lay = kv.kv_layout_init(*w.dims, w.dtype)
        self.lens = [int(x) for x in synth.row_lengths(w)]
        self.positions = [list(map(int, p)) for p in synth.decode_positions(w)]
        self.A = _filled_cache(torch, w, w.value_seed)
        self.s = {name: torch.cuda.Stream()
                  for name in ("p", "t", "out", "in", "d2h", "d2h_row", "h2d")}
        # prompt chunks of one layer: (first token, bytes); every layer has the same
        ch = w.chunk_tokens
        self.chunks = []
        for c0 in range(0, max(self.lens), ch):
            cnt = [max(0, min(ch, n - c0)) for n in self.lens]
            self.chunks.append((c0, kv.kv_pack_bytes(self.lay, 1, cnt)))
        self.prompt_layer = sum(c[1] for c in self.chunks)
        cb = max(c[1] for c in self.chunks)
        # prompt-streaming handles: chunks alternate over them, each with its
        # own copy stream, so that a handle's next copy is already queued on
        # its DMA engine while the other's runs
        self.eng_p, self.p_copy = [], []
        for i, e in enumerate(prompt_engines if transport == TRANSPORTS["engine"] else [-1]):
            cs = self.s["d2h"] if i == 0 else torch.cuda.Stream()
            self.p_copy.append(cs)
            h = kv.KvSwap(self.lay, _bank(torch, cb), _bank(torch, cb), cb, cs, transport)
            if transport == TRANSPORTS["engine"]:
                h.set_option(kv.KV_OPT_DMA_ENGINE, e)
            self.eng_p.append(h)
        # layer l's chunks land in host region l % 2, one layer each: the host
        # buffer a prompt worker forwards from (the whole prompt, 60 GB at these
        # lengths, need not stay page-locked on this side)
        self.prompt_host = [HostBuffer(kv, self.prompt_layer) for _ in range(2)]
        # the swapped row
        bstar = max(range(B), key=lambda b: self.lens[b])
        self.row_start = [0] * B
        self.row_count = [self.lens[b] if b == bstar else 0 for b in range(B)]
        self.row_layer = kv.kv_pack_bytes(self.lay, 1, self.row_count)
        self.row_image = L * self.row_layer
        # the row swap's banks, 0 meaning the whole image (one chunk each way);
        # a bank holds at least one row of one layer (the engine splits at rows)
        ob = row_bank_bytes or (-(-self.row_image // (1 << 20)) << 20)
        ob = max(ob, -(-self.row_layer // (1 << 20)) << 20)
        rt = row_transport
        self.eng_o = []
        for i, e in enumerate(row_engines if rt == TRANSPORTS["engine"] else [-1]):
            cs = self.s["d2h_row"] if i == 0 else torch.cuda.Stream()
            h = kv.KvSwap(self.lay, _bank(torch, ob), _bank(torch, ob), ob, cs, rt)
            if rt == TRANSPORTS["engine"]:
                h.set_option(kv.KV_OPT_DMA_ENGINE, e)
            if row_link_blocks:
                h.set_option(kv.KV_OPT_LINK_BLOCKS, row_link_blocks)
            self.eng_o.append(h)
        # the one-row slot: the row's packed image is the same bytes in a cache
        # of one row (the other rows move no tokens)
        self.lay1 = kv.kv_layout_init(L, 1, w.H, w.D, w.Smax, w.dtype)
        n1 = L * w.H * w.D * w.Smax
        self.slot1 = (torch.empty(n1, dtype=torch.int16, device="cuda"),
                      torch.empty(n1, dtype=torch.int16, device="cuda"))
        self.eng_i = kv.KvSwap(self.lay1, _bank(torch, ob), _bank(torch, ob), ob, self.s["h2d"],
                               row_in_transport)
        # the first step swaps in whatever the second image holds: its bytes
        # only have to be there, not to be a real row (no kernels at set-up,
        # so a counter run sees the steps' launches only)
        self.row_host = [HostBuffer(kv, self.row_image) for _ in range(2)]
        torch.cuda.synchronize()
        self.slot = kv.kv_pack_bytes(self.lay, L, None, 1)
        R = w.ring_slots
        self.ring_host = _pinned(torch, w.decode_steps * self.slot)
        self.ring = kv.KvRing(self.lay, R, _bank(torch, R * self.slot), _bank(torch, R * self.slot),
                              self.ring_host, copy_stream=self.s["d2h"], transport=transport)
        self.ring.set_gather(RING_GATHER)
        self.k = 0

    def link_bytes(self):
        return self.link_bytes_out() + self.link_bytes_in()

    def link_bytes_out(self):
        """prompt streaming, row swap-out, ring flushes"""
        return self.w.L * self.prompt_layer + self.row_image + self.w.decode_steps * self.slot

    def link_bytes_in(self):
        """row swap-in, ring restore"""
        return self.row_image + self.w.decode_steps * self.slot

    def ceiling_caches(self):
        return self.A, self.A

    def run(self):
        torch, w = self.torch, self.w
        out, inn = self.k % 2, (self.k + 1) % 2
        self.k += 1
        n = len(self.eng_o)
        for i, h in enumerate(self.eng_o):
            l0, l1 = w.L * i // n, w.L * (i + 1) // n
            h.swap_out(self.A[0], self.A[1], l0, l1 - l0, self.row_start, self.row_count,
                       self.row_host[out].data_ptr() + l0 * self.row_layer,
                       (l1 - l0) * self.row_layer, self.s["out"],
                       self.row_done if ((self.row_first or self.row_in_after) and i == n - 1)
                       else None)
        if self.row_first:
            for cs in self.p_copy:
                cs.wait_event(self.row_done)
        if self.row_in_after:
            self.s["h2d"].wait_event(self.row_done)
        self.eng_i.swap_in(self.slot1[0], self.slot1[1], 0, w.L, [0], [max(self.row_count)],
                           self.row_host[inn], self.row_image, self.s["in"])
        k, n = 0, len(self.eng_p)
        for l in range(w.L):
            off = self.prompt_host[l % 2].data_ptr()
            for c0, nb in self.chunks:
                self.eng_p[k % n].stream_prompt_layer(self.A[0], self.A[1], l, c0,
                                                      w.chunk_tokens, self.lens, off, nb,
                                                      self.s["p"])
                off += nb
                k += 1
        st = self.s["t"]
        self.ring.reset()
        for pos in self.positions:
            self.ring.push(self.A[0], self.A[1], pos, st)
        self.ring.flush(st)
        self.ring.restore(self.A[0], self.A[1], st)
        torch.cuda.synchronize()

    def cpu_ops(self):
        B, ch = self.w.B, self.w.chunk_tokens
        ops = []
        for c0, nb in self.chunks:
            cnt = [max(0, min(ch, n - c0)) for n in self.lens]
            ops.append(("prompt chunk pack", [c0 if c else 0 for c in cnt], cnt))
        ops.append(("row swap pack", self.row_start, self.row_count))
        return self.A, ops


STEPS = {"gpt2-small-tiny": StreamStep, "gpt2-1.5b": StreamStep, "opt-66b-16l": RingStep,
         "bloom-176b-10l": SwapStep, "gqa-100k": LongStep}

# The transport each step runs with unless --transport names one: the one
# measured fastest for that step (ties go to the one that leaves the tile
# kernels more of HBM).  GPT-2-1.5B: with the named-engine device->host leg
# the step takes 107-110 ms against 108-115 ms with the link-copy kernel
# (alternating runs on one box), with the tile kernels at 0.63-0.66 of peak
# instead of 0.54-0.56; the BLOOM step runs 2-3% faster with the link-copy
# kernel, and the OPT-66B ring keeps the link-copy kernel too: pinned to one
# engine it matched it on one box (below) and took 15.7 ms on another.  The 100K-context step streams its
# prompt on DMA engine 0 through two handles (the next chunk's copy is
# queued on the engine while the other runs) and swaps its row with the
# link-copy kernel from 16 workgroups, through banks that hold the whole row
# image (packed in one pass before the copy), the prompt's copies after the
# row's: 1469-1471 ms (66.9-67.0 GB/s) with its pack kernels at 0.63 of HBM
# peak, against 1477 ms (66.7 GB/s) and 0.32 with the link-copy kernel for
# every outgoing copy (two runs each, one box).
DEFAULT_TRANSPORT = {"gpt2-small-tiny": "auto", "gpt2-1.5b": "engine", "opt-66b-16l": "auto",
                     "bloom-176b-10l": "auto", "gqa-100k": "engine"}
TRANSPORTS = {"auto": 0, "kernel": 1, "runtime": 2, "dma": 3, "dma_out": 4, "engine": 5}
# the long-context step's row swap transport (absent: the step's transport),
# its prompt handles' DMA engines and its row swap-out's link-copy workgroups
DEFAULT_ROW_TRANSPORT = {"gqa-100k": "auto"}
# swap banks: the BLOOM step's hold one layer of a microbatch (0), so each
# layer is packed in one pass and copied as one piece: 281-282 ms per round
# (97.5-98.0 GB/s) with its unpacks at 0.61 of HBM peak in the step, against
# 297 ms (92.6 GB/s) and 0.44 with 256 MiB banks (6 row groups per layer)
DEFAULT_SWAP_BANK_MIB = {"bloom-176b-10l": 0}
# DMA engines of the device->host handles when a step runs with the engine
# transport (the GPT-2 steps: prompt, ring, swap-out; the OPT-66B ring: its
# flushes; the BLOOM step: its swap-out handles); absent: an idle engine at
# each copy.  The OPT-66B ring pinned to engine 0 took 11.04-11.05 ms with
# its gather kernel at 0.45 of HBM peak on one box (11.0-11.05 ms and
# 0.40-0.43 with the link-copy kernel, 11.85 ms with an idle engine at each
# copy) and 15.7 ms on another, so its default transport stays the kernel.
DEFAULT_OUT_ENGINES = {"opt-66b-16l": "0"}


DEFAULT_PROMPT_ENGINES = {"gqa-100k": "0,0"}
# the OPT-66B ring step restores the previous step's image while it flushes:
# 6.53 ms (92.4 GB/s across the link, both directions at 46.2 GB/s) against
# 11.0 ms (54.9 GB/s) flushing and then restoring one ring (two runs each,
# one box, the link-copy transport; the runtime's DMA copies both ways 6.48
# ms; named engines 10.85 ms: the two directions did not overlap)
DEFAULT_RING_DUPLEX = {"opt-66b-16l": True}
DEFAULT_ROW_LINK_BLOCKS = {"gqa-100k": 16}
DEFAULT_ROW_ENGINES = {}
DEFAULT_ROW_FIRST = {"gqa-100k": True}
DEFAULT_ROW_BANK_MIB = {"gqa-100k": 0}


def default_out_engines(name):
    e = DEFAULT_OUT_ENGINES.get(name)
    return [int(x) for x in e.split(",")] if e else None


def link_ceiling(step, kv, transport, target_bytes=4 << 30, reps=3):
    """GB/s the host link reaches through this library with `transport`, each
    way and both ways at once: a swap-out and a swap-in of whole layers (every
    row, all Smax positions; about 4 GB) through 256 MiB banks on streams of
    their own, timed from the first enqueue to the synchronisation after the
    last.  The swap-in lands in the step's second cache, or in the last layers
    when the step has one cache (contents after the timed steps are not
    used)."""
    torch, lay = step.torch, step.lay
    L, B, S = lay.L, lay.B, lay.Smax
    full = [S] * B
    per_layer = kv.kv_pack_bytes(lay, 1, full)
    nl = max(1, min(L, target_bytes // per_layer))
    nbytes = nl * per_layer
    src, dst = step.ceiling_caches()
    l_in = L - nl if src is dst else 0
    # 256 MiB banks, or one row of one layer when that is larger
    bank = max(256 << 20, -(-kv.kv_pack_bytes(lay, 1, [S] + [0] * (B - 1)) // (1 << 20)) << 20)
    s = {n: torch.cuda.Stream() for n in ("po", "pi", "co", "ci")}
    eo = kv.KvSwap(lay, _bank(torch, bank), _bank(torch, bank), bank, s["co"], transport)
    ei = kv.KvSwap(lay, _bank(torch, bank), _bank(torch, bank), bank, s["ci"], transport)
    ho, hi = HostBuffer(kv, nbytes), HostBuffer(kv, nbytes)
    zero = [0] * B

    def out():
        eo.swap_out(src[0], src[1], 0, nl, zero, full, ho.data_ptr(), nbytes, s["po"])

    def inn():
        ei.swap_in(dst[0], dst[1], l_in, nl, zero, full, hi.data_ptr(), nbytes, s["pi"])

    def both():
        out()
        inn()

    res = {"transport": {v: k for k, v in TRANSPORTS.items()}[transport], "bytes_per_leg": nbytes}
    for name, fn, legs in (("d2h", out, 1), ("h2d", inn, 1), ("duplex_total", both, 2)):
        secs = rep_seconds(torch, fn, None, warm=1, reps=reps)
        res[name] = round(legs * nbytes / float(np.median(secs)) / 1e9, 2)
    eo.close()
    ei.close()
    ho.close()
    hi.close()
    return res


def hbm_copy_ceiling(torch, kv, nbytes=2 << 30, warm=5, reps=20):
    """What HBM gives a plain copy on this GPU, read + write: the library's
    kv_copy_packed (one 16-byte vector per thread, non-temporal loads and
    stores) on 2 GiB, timed from its dispatches, median of `reps` after `warm`
    (2 GiB each way is well past the 256 MB Infinity Cache); and torch's own
    device-to-device copy of the same buffers, timed with events."""
    a = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda").fill_(1)
    b = torch.empty_like(a)
    s = torch.cuda.Stream()
    secs = []
    for i in range(warm + reps):
        kv.kv_profile_begin()
        kv.kv_copy_packed(b, a, nbytes, stream=s)
        torch.cuda.synchronize()
        stats = kv.kv_profile_end()
        if i >= warm:
            secs.append(stats["copy_packed"][1] / 1000)
    out = {"bytes_each_way": nbytes}
    rate_entry(out, "kv_copy_packed", secs, 2 * nbytes, HBM_PEAK_GBPS, "_GBps")
    torch_secs = rep_seconds(torch, lambda: b.copy_(a), torch.cuda.current_stream(), warm=2,
                             reps=5)
    rate_entry(out, "torch_copy", torch_secs, 2 * nbytes, HBM_PEAK_GBPS, "_GBps")
    del a, b
    return out


def rep_seconds(torch, fn, s=None, warm=5, reps=20):
    """Seconds of each of `reps` back-to-back calls of `fn` after `warm` untimed
    ones: events on stream `s` between calls, or (s None: work that spans
    streams) the host clock around each call and a synchronisation."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    if s is None:
        out = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            out.append(time.perf_counter() - t0)
        return out
    ev = [TimingEvent() for _ in range(reps + 1)]
    ev[0].record(s)
    for i in range(reps):
        fn()
        ev[i + 1].record(s)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) / 1000 for i in range(reps)]


def spread(secs):
    """median, p10, p90 of a list of seconds, in microseconds."""
    import numpy as np
    a = np.asarray(secs) * 1e6
    return float(np.median(a)), float(np.percentile(a, 10)), float(np.percentile(a, 90))


def rate_entry(out, name, secs, nbytes, peak, unit_key):
    med, p10, p90 = spread(secs)
    out[name + "_us"] = {"median": round(med, 1), "p10": round(p10, 1), "p90": round(p90, 1),
                         "reps": len(secs)}
    rate = nbytes / (med / 1e6) / 1e9
    out[name + unit_key] = round(rate, 2)
    out[name + "_frac_of_peak"] = round(rate / peak, 4)


def large_slices(step, kv):
    """Isolated rates on the workload's largest slices (median of 20 timed calls
    after 5 warm-up ones, with p10/p90): one pack and one unpack of every layer
    and position of a cache (2.5 GB of payload in one call, past the 256 MB
    Infinity Cache), and one whole-cache swap per link direction alone, in
    one call each as the step issues them."""
    torch, w = step.torch, step.w
    L, B = w.L, w.B
    full = [w.Smax] * B
    payload = kv.kv_pack_bytes(step.lay, L, full)
    st = torch.empty(payload // 2, dtype=torch.int16, device="cuda")
    Bc, Cc = step.caches["B"], step.caches["C"]
    s = step.s["t"]
    out = {"payload_bytes": payload}
    for name, fn in (("pack", lambda: kv.kv_pack_tokens(step.lay, Bc[0], Bc[1], 0, L, [0] * B, full,
                                                       st, payload, s)),
                     ("unpack", lambda: kv.kv_unpack_tokens(step.lay, Cc[0], Cc[1], 0, L, [0] * B,
                                                           full, st, payload, s))):
        rate_entry(out, name, rep_seconds(torch, fn, s), 2 * payload, HBM_PEAK_GBPS, "_hbm_GBps")
    del st
    hs = step.host_s[0].data_ptr()
    total = L * step.layer_full
    for name, fn in (("swap_out", lambda: step.eng_o.swap_out(Bc[0], Bc[1], 0, L, step.rows_start,
                                                              step.rows_full, hs, total, s)),
                     ("swap_in", lambda: step.eng_i.swap_in(Cc[0], Cc[1], 0, L, step.rows_start,
                                                            step.rows_full, hs, total, s))):
        rate_entry(out, name, rep_seconds(torch, fn, None, warm=2, reps=10), total,
                   PCIE_PEAK_GBPS, "_link_GBps")
    return out


def layer_slices(step, kv, cache, start, count, warm=5, reps=20):
    """Isolated one-layer pack and unpack on the workload's own slice shape
    (a BLOOM-176B layer of every row, one 100K-context row): layers 0 and 1
    alternate so every call reads data the last one did not (each layer's
    slice is larger than the 256 MB Infinity Cache or close to it).  Seconds
    are the library's kernel durations timed from their dispatches; each
    unpack writes back what that layer's pack produced, so the cache ends as
    it began.  HBM bytes = read + write of the payload."""
    torch, lay = step.torch, step.lay
    k, v = cache
    B = lay.B
    pb = kv.kv_pack_bytes(lay, 1, count)
    stg = [torch.empty(pb // 2, dtype=torch.int16, device="cuda") for _ in range(2)]
    s = torch.cuda.Stream()
    out = {"payload_bytes": pb}
    for name, fn in (("pack", kv.kv_pack_tokens), ("unpack", kv.kv_unpack_tokens)):
        secs = []
        for i in range(warm + reps):
            l = i % 2
            kv.kv_profile_begin()
            fn(lay, k, v, l, 1, start, count, stg[l], pb, s)
            torch.cuda.synchronize()
            stats = kv.kv_profile_end()
            if i >= warm:
                secs.append(sum(x[1] for x in stats.values()) / 1000)
        rate_entry(out, name, secs, 2 * pb, HBM_PEAK_GBPS, "_hbm_GBps")
    del stg
    return out


def slices_only(step, kv):
    """The isolated large-slice calls of a workload (each moves 256 MiB of
    payload or more): 48 GPT-2-1.5B layers in one call (and the same prompt
    from paged pools of 16- and 256-token blocks), a BLOOM-176B layer of
    every row, one layer of the longest 100K-context row, and the OPT-66B
    slice's split into 2 stages x 2 ranks and its merge."""
    if isinstance(step, StreamStep):
        out = {"gpt2_48_layers": large_slices(step, kv)}
        if step.w.B * step.w.Smax >= 4096:
            out["paged"] = paged_slices(step, kv)
        return out
    if isinstance(step, SwapStep):
        return {"bloom_layer": layer_slices(step, kv, step.slots[0], step.rows_start, step.rows)}
    if isinstance(step, LongStep):
        return {"long_row_layer": layer_slices(step, kv, step.A, step.row_start, step.row_count)}
    if isinstance(step, RingStep):
        return {"repartition_2x2": step.repartition(kv)}
    return {}


def paged_slices(step, kv):
    """Isolated rates of the paged pool kernels on the workload's prompt: every
    layer's 1000 prompt tokens of 8 rows packed from (and unpacked into) a pool
    of 16-token pages and one of 256-token chunks, the rows' blocks scattered
    at random over the pool; HBM bytes = read + write of the payload; median
    of 20 timed calls after 5 warm-up ones."""
    import numpy as np
    torch, w = step.torch, step.w
    L, B, H, D = w.L, w.B, w.H, w.D
    count = [w.prompt_len] * B
    start = [0] * B
    s = step.s["t"]
    out = {}
    for P in (16, 256):
        stride = -(-w.Smax // P)
        NB = B * stride
        pg = kv.kv_paged_init(L, NB, H, D, P, w.dtype)
        n = L * NB * H * D * P
        k = torch.empty(n, dtype=torch.int16, device="cuda").fill_(1)
        v = torch.empty(n, dtype=torch.int16, device="cuda").fill_(2)
        rng = np.random.default_rng(P)
        table = torch.from_numpy(rng.permutation(NB).reshape(B, stride).astype(np.int32)).cuda()
        payload = kv.kv_paged_pack_bytes(pg, L, B, count)
        st = torch.empty(payload // 2, dtype=torch.int16, device="cuda")
        row = {"block_tokens": P, "payload_bytes": payload}
        for name, fn in (("pack", kv.kv_pack_paged), ("unpack", kv.kv_unpack_paged)):
            secs = rep_seconds(torch, lambda: fn(pg, k, v, 0, L, table, start, count, st, payload, s),
                               s)
            rate_entry(row, name, secs, 2 * payload, HBM_PEAK_GBPS, "_hbm_GBps")
        out[f"pages_{P}"] = row
        del k, v, st, table
        torch.cuda.empty_cache()
    return out


def decode_loop(step, kv, cache, reps=5):
    """A decode loop that packs each step as it comes: one kv_pack_tokens call
    per step (one token per row at the workload's decode positions, every
    layer) into that step's slot of a staging buffer.  Wall time per step of
    the whole loop, events on its stream around it (best of `reps` after two
    warm-up loops): issued from Python call by call, and captured once into a
    HIP graph and replayed.  The replay's bytes are compared with the eager
    loop's; the kernels' own time per step comes from their dispatches."""
    torch, lay = step.torch, step.lay
    positions = step.positions
    n = len(positions)
    slot = kv.kv_pack_bytes(lay, lay.L, None, 1)
    st = torch.zeros(n * slot // 2, dtype=torch.int16, device="cuda")
    base = st.data_ptr()
    k, v = cache
    s = torch.cuda.Stream()

    def loop():
        for j, pos in enumerate(positions):
            kv.kv_pack_tokens(lay, k, v, 0, lay.L, pos, None, base + j * slot, slot, s)

    eager = min(rep_seconds(torch, loop, s, warm=2, reps=reps))
    kv.kv_profile_begin()
    loop()
    torch.cuda.synchronize()
    kernel_ms = sum(x[1] for x in kv.kv_profile_end().values())
    want = st.clone()
    st.zero_()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s, capture_error_mode="relaxed"):
        loop()
    torch.cuda.synchronize()

    def replay():
        with torch.cuda.stream(s):
            g.replay()

    graph = min(rep_seconds(torch, replay, s, warm=2, reps=reps))
    torch.cuda.synchronize()
    same = bool(torch.equal(st, want))
    del g, st, want
    return {"steps": n, "bytes_per_step": slot,
            "eager_us_per_step": round(eager / n * 1e6, 2),
            "graph_us_per_step": round(graph / n * 1e6, 2),
            "kernel_us_per_step": round(kernel_ms * 1000 / n, 2),
            "graph_matches_eager": same}


def buffered_vs_naive(step, kv, cache, reps=3, max_copies=200_000, keep_image=False):
    """One decode step's new keys and values (one token per row at the
    workload's first decode positions, every layer) sent to pinned host
    memory in two ways.  Buffered, as the library does it: one kv_pack_tokens
    call into a staging slot, then one device-to-host copy of the slot.
    Naive: one runtime copy per contiguous piece of the cache, straight to
    that piece's place in the same host image.  "per_piece" issues one copy
    per 16-byte key vector and one per value row.  "per_head" issues, per
    head, one strided 2-D copy of its key vectors and one copy of its value
    row.  The naive copies are issued from Python through ctypes.
    `ctypes_us_per_call` is what that loop costs per call around a runtime
    call that does no work.  Times are wall time from the first call to the
    end of the stream, best of `reps`.  The three host images must be
    byte-identical; `keep_image` returns the buffered one as `image`."""
    torch, lay = step.torch, step.lay
    L, B, H, D, S = lay.L, lay.B, lay.H, lay.D, lay.Smax
    C, P = D // 8, 2
    pos = [int(p) for p in step.positions[0]]
    assert all(0 <= p < S for p in pos)
    slot = kv.kv_pack_bytes(lay, L, None, 1)
    k, v = cache
    kb, vb = k.data_ptr(), v.data_ptr()
    lib = kv._lib      # the HIP runtime the library and torch share
    copy1 = lib.hipMemcpyAsync
    copy1.restype = ctypes.c_int
    copy1.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                      ctypes.c_void_p]
    copy2 = lib.hipMemcpy2DAsync
    copy2.restype = ctypes.c_int
    copy2.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                      ctypes.c_size_t, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    noop = lib.hipPeekAtLastError
    noop.restype, noop.argtypes = ctypes.c_int, []
    d2h = 2                                   # hipMemcpyDeviceToHost
    s = torch.cuda.Stream()
    sh = s.cuda_stream
    st = torch.empty(slot // 2, dtype=torch.int16, device="cuda")
    hosts = {name: _pinned(torch, slot) for name in ("buffered", "per_piece", "per_head")}
    for h_ in hosts.values():
        h_.zero_()
    # (host offset, cache address) of every head's key and value run; the
    # packed place of (layer l, K|V, row b, head h) for one token per row
    runs = []
    for l in range(L):
        for b in range(B):
            for h in range(H):
                unit = (l * B + b) * H + h
                ko = ((2 * l) * H * B + H * b + h) * D * P
                vo = ((2 * l + 1) * H * B + H * b + h) * D * P
                runs.append((ko, kb + (unit * C * S + pos[b]) * 16,
                             vo, vb + (unit * S + pos[b]) * D * P))
    # every copy stays inside its buffers
    assert max(r[2] for r in runs) + D * P <= slot and max(r[0] for r in runs) + D * P <= slot
    assert max(r[1] for r in runs) + ((C - 1) * S + 1) * 16 <= kb + lay.k_bytes
    assert min(r[1] for r in runs) >= kb and min(r[3] for r in runs) >= vb
    assert max(r[3] for r in runs) + D * P <= vb + lay.v_bytes
    n_piece, n_head = len(runs) * (C + 1), len(runs) * 2
    torch.cuda.synchronize()

    def buffered():
        kv.kv_pack_tokens(lay, k, v, 0, L, pos, None, st, slot, s)
        return copy1(hosts["buffered"].data_ptr(), st.data_ptr(), slot, d2h, sh)

    def per_piece():
        hb, bad = hosts["per_piece"].data_ptr(), 0
        for ko, ks, vo, vs in runs:
            for c in range(C):
                bad |= copy1(hb + ko + c * 16, ks + c * S * 16, 16, d2h, sh)
            bad |= copy1(hb + vo, vs, D * P, d2h, sh)
        return bad

    def per_head():
        hb, bad = hosts["per_head"].data_ptr(), 0
        for ko, ks, vo, vs in runs:
            bad |= copy2(hb + ko, 16, ks, S * 16, 16, C, d2h, sh)
            bad |= copy1(hb + vo, vs, D * P, d2h, sh)
        return bad

    out = {"bytes_per_step": slot, "copies_per_step": {"buffered": 1, "per_piece": n_piece,
                                                       "per_head": n_head}}
    for name, fn in (("buffered", buffered), ("per_piece", per_piece), ("per_head", per_head)):
        if out["copies_per_step"][name] > max_copies:
            continue
        best = None
        for _ in range(reps + 1):                  # the first pass warms up
            t0 = time.perf_counter()
            rc = fn()
            t1 = time.perf_counter()
            s.synchronize()
            t2 = time.perf_counter()
            if rc:
                raise RuntimeError(f"buffered_vs_naive: a {name} copy failed (hipError {rc})")
            if best is None or t2 - t0 < best[0]:
                best = (t2 - t0, t1 - t0)
        out[f"{name}_us"] = round(best[0] * 1e6, 1)
        out[f"{name}_issue_us"] = round(best[1] * 1e6, 1)
    t0 = time.perf_counter()
    for _ in range(n_head):
        noop()
    out["ctypes_us_per_call"] = round((time.perf_counter() - t0) / n_head * 1e6, 3)
    for name in ("per_piece", "per_head"):
        if f"{name}_us" in out:
            out[f"gain_over_{name}"] = round(out[f"{name}_us"] / out["buffered_us"], 1)
            if not torch.equal(hosts[name], hosts["buffered"]):
                raise RuntimeError(f"buffered_vs_naive: the {name} host image differs")
    out["host_images_equal"] = True
    if keep_image:
        out["image"] = hosts["buffered"]
    del st, hosts
    return out


def prompt_overlap(step, kv, reps=2):
    """Layer-by-layer prompt streaming against streaming once the prompt is
    done.  The pages give no per-layer compute time, so a timed busy-wait of
    t on a compute stream plays each layer's compute, with t set to fractions
    of x, the per-layer transfer time measured alone.  Overlapped: layer l's
    busy-wait, then kv_stream_prompt_layer(l) on the same stream; its pack
    follows the layer's compute, and its copy runs on the copy stream while
    layer l+1 computes.  After: all L busy-waits, then the L layers streamed.
    Times are wall time from the first call until the last copy has landed,
    best of `reps`.  `ideal_ms` is L*max(t, x) + min(t, x), a pipeline of L
    stages."""
    torch, w = step.torch, step.w
    L, A, lp, eng = w.L, step.caches["A"], step.layer_prompt, step.eng_p
    host = step.host_p[0].data_ptr()
    c = torch.cuda.Stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(c):
        torch.cuda._sleep(1000)
        e0.record(c)
        torch.cuda._sleep(2_000_000)
        e1.record(c)
    torch.cuda.synchronize()
    cycles_per_ms = 2_000_000 / e0.elapsed_time(e1)

    def stream(l):
        eng.stream_prompt_layer(A[0], A[1], l, 0, step.prompt, None, host + l * lp, lp, c)

    def run(t_ms, overlap):
        cyc = int(t_ms * cycles_per_ms)
        best = None
        for _ in range(reps + 1):                  # the first pass warms up
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            with torch.cuda.stream(c):
                for l in range(L):
                    if cyc:
                        torch.cuda._sleep(cyc)
                    if overlap:
                        stream(l)
                if not overlap:
                    for l in range(L):
                        stream(l)
            torch.cuda.synchronize()
            dt = (time.perf_counter() - t0) * 1000
            best = dt if best is None else min(best, dt)
        return best

    x = run(0.0, True) / L
    out = {"layers": L, "layer_bytes": lp, "transfer_ms_per_layer": round(x, 3), "rows": []}
    for f in (0.5, 1.0, 2.0):
        t = f * x
        after, over = run(t, False), run(t, True)
        out["rows"].append({"compute_ms_per_layer": round(t, 3), "after_ms": round(after, 2),
                            "overlapped_ms": round(over, 2),
                            "ideal_ms": round(L * max(t, x) + min(t, x), 2),
                            "gain": round(after / over, 2)})
    return out


def token_overlap(step, kv, cache, reps=2, keep_image=False):
    """Decode steps streamed through the staging ring while the next steps
    compute, against compute that waits for each bank's flush.  A timed
    busy-wait of t on the compute stream plays each decode step's compute.
    The pages give no step time, so t is set so that a bank's R steps take
    ½, 1 and 2 times x, the flush of one bank measured alone.  Overlapped:
    each step's busy-wait, then kv_ring_push; a full bank is packed and
    copied out on the copy stream while the next bank's steps compute.
    Waiting: the same calls, but after each full bank the compute stream
    waits for that bank's copy to land.  Times are wall time until the host
    image is complete, best of `reps`.  `ideal_ms` is n·max(R·t, x) + min(R·t, x)
    over the n banks.  `keep_image` returns the host image as `image`."""
    torch, w, lay = step.torch, step.w, step.lay
    R, positions = w.ring_slots, step.positions
    nsteps = len(positions)
    banks = nsteps // R
    slot = kv.kv_pack_bytes(lay, lay.L, None, 1)
    k, v = cache
    c, cs = torch.cuda.Stream(), torch.cuda.Stream()
    hostbuf = _pinned(torch, nsteps * slot)
    ring = kv.KvRing(lay, R, _bank(torch, R * slot), _bank(torch, R * slot), hostbuf,
                     copy_stream=cs)
    ring.set_gather(kv.KV_RING_GATHER_AT_FLUSH)
    landed = torch.cuda.Event()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(c):
        torch.cuda._sleep(1000)
        e0.record(c)
        torch.cuda._sleep(2_000_000)
        e1.record(c)
    torch.cuda.synchronize()
    cycles_per_ms = 2_000_000 / e0.elapsed_time(e1)

    def run(t_ms, wait):
        cyc = int(t_ms * cycles_per_ms)
        best = None
        for _ in range(reps + 1):                  # the first pass warms up
            ring.reset()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            with torch.cuda.stream(c):
                for j, pos in enumerate(positions[:banks * R]):
                    if cyc:
                        torch.cuda._sleep(cyc)
                    ring.push(k, v, pos, c)
                    if wait and (j + 1) % R == 0:
                        ring.flush(c, landed)      # nothing left to copy: marks the bank's copy
                        c.wait_event(landed)
                ring.flush(c)
            torch.cuda.synchronize()
            dt = (time.perf_counter() - t0) * 1000
            best = dt if best is None else min(best, dt)
        return best

    x = run(0.0, True) / banks
    out = {"steps": banks * R, "ring_slots": R, "bank_bytes": R * slot,
           "flush_ms_per_bank": round(x, 3), "rows": []}
    for f in (0.5, 1.0, 2.0):
        t = f * x / R
        waiting, over = run(t, True), run(t, False)
        out["rows"].append({"compute_ms_per_step": round(t, 4), "waiting_ms": round(waiting, 2),
                            "overlapped_ms": round(over, 2),
                            "ideal_ms": round(banks * max(R * t, x) + min(R * t, x), 2),
                            "gain": round(waiting / over, 2)})
    ring.close()
    if keep_image:
        out["image"] = hostbuf
    return out


def decode_step_us(step, kv, reps=3):
    """GPU time per decode step of the workload's decode steps, with a ring of
    one bank holding them all (no bank reuse, so no wait for a flush copy):
    each step packed as it is pushed (`each_step`), or all packed in one pass
    at the flush (`at_flush`).  The time is the library's pack kernels' own
    duration (timed from their dispatches), summed and divided by the steps;
    the flush's device-to-host copy is not in it.  `at_flush_GBps` is the
    one-pass gather's HBM rate (payload read + written).  Best of `reps`."""
    torch, w = step.torch, step.w
    st = step.s["t"]
    Bc = step.caches["B"]
    n = len(step.positions)
    bank = [torch.empty(n * step.slot // 2, dtype=torch.int16, device="cuda") for _ in range(2)]
    hostbuf = _pinned(torch, n * step.slot)
    ring = kv.KvRing(step.lay, n, bank[0], bank[1], hostbuf, copy_stream=step.s["d2h"])
    out = {}
    for name, mode in (("each_step", kv.KV_RING_GATHER_EACH_STEP),
                       ("at_flush", kv.KV_RING_GATHER_AT_FLUSH)):
        ring.set_gather(mode)
        best = None
        for _ in range(reps):
            ring.reset()
            torch.cuda.synchronize()
            kv.kv_profile_begin()
            for pos in step.positions:
                ring.push(Bc[0], Bc[1], pos, st)
            ring.flush(st)
            torch.cuda.synchronize()
            stats = kv.kv_profile_end()
            ms = sum(v[1] for k, v in stats.items() if not k.startswith("link_copy"))
            best = ms if best is None else min(best, ms)
        out[name] = round(best * 1000 / n, 2)
        if name == "at_flush":
            out["at_flush_GBps"] = round(2 * n * step.slot / (best / 1000) / 1e9, 1)
    ring.close()
    return out


def read_counters(workload, kernel_name, algorithmic):
    """Per-launch HBM traffic of `kernel_name` from the committed counter summary
    of the workload, or None when absent, taken on a different kernel source or
    on a different mix of launches (another algorithmic size per launch)."""
    path = counters_file(workload, kernel_name)
    if not os.path.exists(path):
        return None
    import hashlib
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    src = os.path.join(ROOT, "kv_cache_streaming_amd", "csrc", "kernels.hip")
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    if fields.get("kernels_sha256_16") != digest or fields.get("kernel") != kernel_name:
        return None
    if fields.get("algorithmic_bytes_per_launch") != str(algorithmic):
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


CPU_THREADS_MAX = 16   # the host cores one GPU's share of the machine may use
MAX_PASSES = 1000      # cap on repeated passes over a per-layer CPU sample


def oracle_pieces(B, start, count, threads):
    """Disjoint parts of one call's selection: each row's token range cut into
    runs of at most ceil(total / (4 * threads)) tokens, as (start, count) rows
    with every other row's count at 0."""
    total = int(sum(int(c) for c in count))
    size = max(1, -(-total // (4 * threads)))
    out = []
    for b in range(B):
        c = int(count[b])
        for t0 in range(0, c, size):
            st, ct = [0] * B, [0] * B
            st[b], ct[b] = int(start[b]) + t0, min(size, c - t0)
            out.append((st, ct))
    return out


def _meets(a, b):
    """Two (array, layer range, row, token range) regions share an element."""
    return (a[0] == b[0] and a[3] == b[3] and a[1] < b[2] and b[1] < a[2]
            and a[4] < b[5] and b[4] < a[5])


def cpu_all_cores(oracle, dims, pairs, budget_s, max_passes):
    """The same oracle calls on every host core the run may use.  Each
    (pack, unpack) pair of the sample is cut into disjoint pieces of its
    selection (`oracle_pieces`), and consecutive pairs whose pieces touch
    disjoint elements are grouped, up to 64 pieces per thread in a group; a
    pool of threads runs the oracle's own C pack and unpack on a group's
    pieces (the C calls release the interpreter lock), one group after
    another.  The pieces' unpacks write disjoint elements and together move
    exactly the bytes of the whole calls; the oracle itself is unchanged and
    single-threaded."""
    import threading

    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    threads = max(1, min(CPU_THREADS_MAX, len(os.sched_getaffinity(0))))
    L, B, H, D, S = dims
    lib = oracle.load()

    rows = []   # keeps every piece's row arrays alive while their addresses are in use

    def piece_jobs(src, dst, l0, nl, start, count):
        jobs = []
        for st, ct in oracle_pieces(B, start, count, threads):
            b = next(r for r in range(B) if ct[r] > 0)
            st_a, ct_a = np.asarray(st, np.int32), np.asarray(ct, np.int32)
            rows.append((st_a, ct_a))
            jobs.append({"src": (src[0].ctypes.data, src[1].ctypes.data),
                         "dst": (dst[0].ctypes.data, dst[1].ctypes.data),
                         "l0": l0, "nl": nl, "st": st_a.ctypes.data, "ct": ct_a.ctypes.data,
                         "n": oracle.pack_elems(dims, nl, ct),
                         "read": (id(src[0]), l0, l0 + nl, b, st[b], st[b] + ct[b]),
                         "write": (id(dst[0]), l0, l0 + nl, b, st[b], st[b] + ct[b])})
        return jobs

    local = threading.local()   # one packed buffer per thread, reused by its pieces

    def run(job):
        n = job["n"]
        if getattr(local, "n", 0) < n:
            local.buf = np.empty(n, np.uint16)
            local.n, local.ptr = n, local.buf.ctypes.data
        args = (job["l0"], job["nl"], job["st"], job["ct"], local.ptr)
        lib.oracle_pack(L, B, H, D, S, *job["src"], *args)
        lib.oracle_unpack(L, B, H, D, S, *job["dst"], *args)
        return 4 * n

    for name, src, dst, *_ in pairs:
        for a in (*src, *dst):
            assert a.dtype == np.uint16 and a.flags["C_CONTIGUOUS"], name
    # the pieces and their groups, marshalled once before the clock starts;
    # a group's regions are indexed by (array, row)
    plan, group, names, reads, writes = [], [], [], {}, {}

    def clash(jobs):
        def hit(r, index):
            return any(_meets(r, x) for x in index.get((r[0], r[3]), ()))
        return any(hit(j["write"], writes) or hit(j["write"], reads) or hit(j["read"], writes)
                   for j in jobs)

    for pair in pairs + [None]:
        jobs = [] if pair is None else piece_jobs(*pair[1:])
        if group and (pair is None or len(group) + len(jobs) > 64 * threads or clash(jobs)):
            plan.append((group, names))
            group, names, reads, writes = [], [], {}, {}
        group += jobs
        for j in jobs:
            reads.setdefault((j["read"][0], j["read"][3]), []).append(j["read"])
            writes.setdefault((j["write"][0], j["write"][3]), []).append(j["write"])
        if pair is not None:
            names.append(pair[0])
    done, ran, passes, groups = 0, {}, 0, 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as pool:
        while time.perf_counter() - t0 < budget_s and passes < max_passes:
            passes += 1
            for group, names in plan:
                if time.perf_counter() - t0 > budget_s:
                    break
                done += sum(pool.map(run, group))
                groups += 1
                for n in names:
                    ran[n] = ran.get(n, 0) + 1
    elapsed = time.perf_counter() - t0
    sample = ", ".join(f"{v} x {k}" for k, v in ran.items())
    return {"value": round(done / elapsed / 1e9, 4), "unit": "GB/s", "cores": threads,
            "sample": f"{sample} ({passes} pass(es), {groups} groups): {done / 1e9:.3f} GB of "
                      f"KV payload in {elapsed:.1f} s, the calls cut into row/token pieces over "
                      f"{threads} threads of the single-threaded C oracle"}


def cpu_baseline(step, budget_s):
    """The oracle, as it stands, on a bounded sample of the same step; then the
    same calls spread over the host's cores (`all_cores`)."""
    import numpy as np

    import oracle
    w = step.w
    L, B, H, D, S = w.dims
    A = [t.cpu().numpy().view(np.uint16) for t in step.caches["A"]]
    Bh = [t.cpu().numpy().view(np.uint16).copy() for t in step.caches["B"]]
    start, prompt, full = step.rows_start, step.rows_prompt, step.rows_full
    ops = []
    for l in range(L):
        ops.append(("prompt pack", l, lambda l=l: oracle.pack(w.dims, A[0], A[1], l, 1, start, prompt)))
        ops.append(("prompt unpack", l, None))
        ops.append(("swap pack", l, lambda l=l: oracle.pack(w.dims, Bh[0], Bh[1], l, 1, start, full)))
        ops.append(("swap unpack", l, None))
        if l < w.decode_steps:
            j = l
            ops.append(("decode pack", j, lambda j=j: oracle.pack(w.dims, Bh[0], Bh[1], 0, L,
                                                                  step.positions[j], [1] * B)))
            ops.append(("restore unpack", j, None))
    done_bytes, ran, last = 0, {}, None
    t0 = time.perf_counter()
    passes = 0
    # whole passes over the step's calls, repeated while the budget lasts
    while time.perf_counter() - t0 < budget_s and passes < 4:
        passes += 1
        done_bytes, last = run_ops(ops, w, oracle, Bh, start, prompt, full, step, L, B,
                                   done_bytes, ran, t0, budget_s)
    elapsed = time.perf_counter() - t0
    sample = ", ".join(f"{v} x {k}" for k, v in ran.items())
    pairs = []
    for l in range(L):
        pairs.append(("prompt pack + unpack", A, Bh, l, 1, start, prompt))
        pairs.append(("swap pack + unpack", Bh, Bh, l, 1, start, full))
        if l < w.decode_steps:
            pairs.append(("decode pack + restore unpack", Bh, Bh, 0, L, step.positions[l], [1] * B))
    return {"value": round(done_bytes / elapsed / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{sample} ({passes} pass(es) over the step's calls): "
                      f"{done_bytes / 1e9:.3f} GB of KV payload in {elapsed:.1f} s "
                      f"(single-threaded C oracle)",
            "all_cores": cpu_all_cores(oracle, w.dims, pairs, budget_s, 4)}


def run_ops(ops, w, oracle, Bh, start, prompt, full, step, L, B, done_bytes, ran, t0, budget_s):
    last = None
    for name, idx, fn in ops:
        if time.perf_counter() - t0 > budget_s:
            break
        if fn is not None:
            last = fn()
        elif name == "prompt unpack":   # each unpack consumes the pack just made
            oracle.unpack(w.dims, Bh[0], Bh[1], idx, 1, start, prompt, last)
        elif name == "swap unpack":
            oracle.unpack(w.dims, Bh[0], Bh[1], idx, 1, start, full, last)
        else:
            oracle.unpack(w.dims, Bh[0], Bh[1], 0, L, step.positions[idx], [1] * B, last)
        done_bytes += last.nbytes
        ran[name] = ran.get(name, 0) + 1
    return done_bytes, last



def cpu_baseline_layer(step, budget_s):
    """The oracle, as it stands, on the workload's per-layer calls, run on a
    host copy of layer 0 (the caches of these workloads are tens of GB)."""
    import numpy as np

    import oracle
    w = step.w
    L, B, H, D, S = w.dims
    dims1 = (1, B, H, D, S)
    n1 = B * H * D * S
    src, ops = step.cpu_ops()
    K = src[0][:n1].cpu().numpy().view(np.uint16)
    V = src[1][:n1].cpu().numpy().view(np.uint16)
    K2, V2 = np.zeros_like(K), np.zeros_like(V)
    done_bytes, ran, passes = 0, {}, 0
    t0 = time.perf_counter()
    # whole passes over the calls while the budget lasts (a decode-only
    # sample is a few milliseconds per pass)
    while time.perf_counter() - t0 < budget_s and passes < MAX_PASSES:
        passes += 1
        for name, start, count in ops:
            if time.perf_counter() - t0 > budget_s:
                break
            packed = oracle.pack(dims1, K, V, 0, 1, start, count)
            oracle.unpack(dims1, K2, V2, 0, 1, start, count, packed)
            done_bytes += 2 * packed.nbytes
            ran[name] = ran.get(name, 0) + 1
    elapsed = time.perf_counter() - t0
    sample = ", ".join(f"{v} x {k} + unpack" for k, v in ran.items())
    pairs = [(name, (K, V), (K2, V2), 0, 1, start, count) for name, start, count in ops]
    return {"value": round(done_bytes / elapsed / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"layer 0 only: {sample} ({passes} pass(es) over the calls): "
                      f"{done_bytes / 1e9:.3f} GB of KV payload packed and unpacked in "
                      f"{elapsed:.1f} s (single-threaded C oracle)",
            "all_cores": cpu_all_cores(oracle, dims1, pairs, budget_s, MAX_PASSES)}

def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the KV pack/unpack and swap path is measured on a single MI355X", flush=True)
        sys.exit(2)
    import torch

    import kv_cache_streaming_amd as kv
    import synth
    w = synth.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    global RING_GATHER, WHOLE_CALLS
    WHOLE_CALLS = args.swap_calls == "whole"
    RING_GATHER = {"flush": kv.KV_RING_GATHER_AT_FLUSH, "each": kv.KV_RING_GATHER_EACH_STEP}[
        args.ring_gather]
    if args.transport is None:
        args.transport = DEFAULT_TRANSPORT[w.name]
    if args.swap_bank_mib is None:
        args.swap_bank_mib = DEFAULT_SWAP_BANK_MIB.get(w.name, 256)
    if STEPS[w.name] is LongStep:
        if args.row_transport is None:
            args.row_transport = DEFAULT_ROW_TRANSPORT.get(w.name, args.transport)
        if args.prompt_engines is None:
            args.prompt_engines = DEFAULT_PROMPT_ENGINES.get(w.name, "-1")
        if args.row_link_blocks is None:
            args.row_link_blocks = DEFAULT_ROW_LINK_BLOCKS.get(w.name, 0)
        if args.row_engines is None:
            args.row_engines = DEFAULT_ROW_ENGINES.get(w.name, "-1")
        if args.row_first is None:
            args.row_first = int(DEFAULT_ROW_FIRST.get(w.name, False))
        if args.row_bank_mib is None:
            args.row_bank_mib = DEFAULT_ROW_BANK_MIB.get(w.name, args.swap_bank_mib)
        if args.row_in_transport is None:
            args.row_in_transport = args.row_transport
        if args.row_in_after is None:
            args.row_in_after = 0
        step = LongStep(w, args.swap_bank_mib << 20, TRANSPORTS[args.transport],
                        TRANSPORTS[args.row_transport],
                        [int(x) for x in args.prompt_engines.split(",")], args.row_link_blocks,
                        [int(x) for x in args.row_engines.split(",")], bool(args.row_first),
                        args.row_bank_mib << 20, TRANSPORTS[args.row_in_transport],
                        bool(args.row_in_after))
    elif STEPS[w.name] is RingStep:
        step = RingStep(w, args.swap_bank_mib << 20, TRANSPORTS[args.transport],
                        [int(x) for x in args.prompt_engines.split(",")]
                        if args.prompt_engines else None,
                        None if args.ring_duplex is None else bool(args.ring_duplex))
    elif STEPS[w.name] is StreamStep:
        step = StreamStep(w, args.swap_bank_mib << 20, TRANSPORTS[args.transport],
                          [int(x) for x in args.prompt_engines.split(",")]
                          if args.prompt_engines else None)
    elif STEPS[w.name] is SwapStep:
        step = SwapStep(w, args.swap_bank_mib << 20, TRANSPORTS[args.transport],
                        [int(x) for x in args.prompt_engines.split(",")]
                        if args.prompt_engines else None, args.link_blocks)
    else:
        step = STEPS[w.name](w, args.swap_bank_mib << 20, TRANSPORTS[args.transport])
    torch.cuda.synchronize()
    progress(f"{w.name}: caches, banks and host images ready")

    if args.calibrate_copy_mib:
        # a plain elementwise kernel that reads and writes exactly this many
        # bytes: the scale for the hardware byte counters
        n = (args.calibrate_copy_mib << 20) // 2
        src = torch.empty(n, dtype=torch.int16, device="cuda").fill_(3)
        dst = torch.empty_like(src)
        torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    if args.slices_only:
        print(json.dumps({"workload": w.name, "large_slices": slices_only(step, kv)}), flush=True)
        return

    if isinstance(step, StreamStep) and args.compute_streams == 1:
        step.run = step.run_one_stream
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    progress(f"{args.warmup} warm-up steps done")
    if not args.no_profile:
        kv.kv_profile_begin()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step.run()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    progress(f"{args.steps} timed steps done: {elapsed / args.steps * 1000:.1f} ms per step")
    stats = {} if args.no_profile else kv.kv_profile_end()
    window = None if args.no_profile else kv.kv_profile_last_window()
    ms = elapsed / args.steps * 1000
    link = step.link_bytes()
    value = link / (ms / 1000) / 1e9

    kernels = {}
    for name, (launches, kms, kbytes) in stats.items():
        if name.startswith("link_copy"):
            # transfers: bytes are host-link bytes, not HBM traffic
            kernels[name] = {"launches_per_step": launches / args.steps,
                             "avg_us": round(kms / launches * 1000, 2),
                             "link_bytes_per_launch": kbytes // launches,
                             "link_GBps": round(kbytes / (kms / 1000) / 1e9, 1),
                             "gpu_ms_per_step": round(kms / args.steps, 3)}
            continue
        avg_ms = kms / launches
        kernels[name] = {"launches_per_step": launches / args.steps,
                         "avg_us": round(avg_ms * 1000, 2),
                         "algorithmic_bytes_per_launch": kbytes // launches,
                         "GBps": round(kbytes / launches / (avg_ms / 1000) / 1e9, 1),
                         "gpu_ms_per_step": round(kms / args.steps, 3)}
    roofline = None
    if any(not k.startswith("link_copy") for k in kernels):
        hbm = [k for k in kernels if not k.startswith("link_copy")]
        dom = max(hbm, key=lambda k: kernels[k]["gpu_ms_per_step"])
        d = kernels[dom]
        traffic = read_counters(w.name, dom, d["algorithmic_bytes_per_launch"])
        roofline = {"bound": "hbm", "kernel": dom, "achieved": d["GBps"], "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": round(d["GBps"] / HBM_PEAK_GBPS, 4),
                    "traffic": traffic,
                    "algorithmic_bytes_per_launch": d["algorithmic_bytes_per_launch"],
                    "avg_us": d["avg_us"]}

    detail = {"kernels": kernels, "link_bytes_per_step": link,
              "link_peak_per_direction_GBps": PCIE_PEAK_GBPS}
    together = None
    if window and window["hbm_busy_ms"] > 0:
        # kernels of different streams overlap: the union of their intervals is
        # the time the pack/unpack kernels kept HBM busy, and their bytes over
        # that time the rate they reached together
        gbps = window["hbm_bytes"] / (window["hbm_busy_ms"] / 1000) / 1e9
        together = {"busy_ms_per_step": round(window["hbm_busy_ms"] / args.steps, 3),
                    "busy_share_of_step": round(window["hbm_busy_ms"] / (elapsed * 1000), 4),
                    "algorithmic_bytes_per_step": window["hbm_bytes"] // args.steps,
                    "GBps": round(gbps, 1), "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
                    "link_busy_share_of_step": round(window["link_busy_ms"] / (elapsed * 1000), 4)}
        detail["hbm_kernels_together"] = together
    # each link direction on its own: bytes per step over the step time, as a
    # share of the PCIe 5.0 x16 peak (and, with the detail, of the ceiling the
    # same transport reaches alone)
    out_b, in_b = step.link_bytes_out(), step.link_bytes_in()
    directions = {}
    for name, nb in (("d2h", out_b), ("h2d", in_b)):
        gbps = nb / (ms / 1000) / 1e9
        directions[name] = {"bytes_per_step": nb, "GBps": round(gbps, 2),
                            "frac_of_pcie_peak": round(gbps / PCIE_PEAK_GBPS, 4)}
    detail["link_directions"] = directions
    if not args.no_profile and not args.no_detail:
        ceil = link_ceiling(step, kv, TRANSPORTS[args.transport])
        progress("link ceiling measured")
        detail["link_ceiling_GBps"] = ceil
        for name in ("d2h", "h2d"):
            directions[name]["frac_of_ceiling"] = round(directions[name]["GBps"] / ceil[name], 4)
        if args.row_transport not in (None, args.transport):
            detail["link_ceiling_row_transport_GBps"] = link_ceiling(
                step, kv, TRANSPORTS[args.row_transport])
        if isinstance(step, StreamStep):
            detail["decode_step_us"] = decode_step_us(step, kv)
            detail["decode_loop"] = decode_loop(step, kv, step.caches["B"])
            detail["buffered_vs_naive"] = buffered_vs_naive(step, kv, step.caches["B"])
            detail["prompt_overlap"] = prompt_overlap(step, kv)
            detail["token_overlap"] = token_overlap(step, kv, step.caches["B"])
            detail["large_slices"] = large_slices(step, kv)
            if step.w.B * step.w.Smax >= 4096:
                detail["paged_slices"] = paged_slices(step, kv)
        if isinstance(step, SwapStep):
            detail["layer_slices"] = layer_slices(step, kv, step.slots[0], step.rows_start,
                                                  step.rows)
            detail["microbatch_schedule"] = step.schedule(kv)
        if isinstance(step, LongStep):
            detail["layer_slices"] = layer_slices(step, kv, step.A, step.row_start,
                                                  step.row_count)
            detail["decode_loop"] = decode_loop(step, kv, step.A)
            detail["buffered_vs_naive"] = buffered_vs_naive(step, kv, step.A)
            detail["token_overlap"] = token_overlap(step, kv, step.A)
        if isinstance(step, RingStep):
            detail["repartition_2x2"] = step.repartition(kv)
            detail["decode_loop"] = decode_loop(step, kv, step.A)
            detail["buffered_vs_naive"] = buffered_vs_naive(step, kv, step.A)
            detail["token_overlap"] = token_overlap(step, kv, step.A)
        detail["hbm_copy_ceiling"] = hbm_copy_ceiling(torch, kv)
        progress("detail measured")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = (cpu_baseline(step, args.cpu_baseline_seconds) if isinstance(step, StreamStep)
               else cpu_baseline_layer(step, args.cpu_baseline_seconds))
        progress("oracle baseline timed")

    line = {"metric": METRIC, "value": round(value, 3), "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u16",
            "data": "synthetic",
            "config": {"workload": w.name, "L": w.L, "B": w.B, "H": w.H, "D": w.D,
                       "Smax": w.Smax, "kv_dtype": "fp16" if w.dtype == 0 else "bf16",
                       "prompt_len": w.prompt_len or f"U{{{w.len_lo}..{w.len_hi}}}",
                       "decode_steps": w.decode_steps, "ring_slots": w.ring_slots,
                       "chunk_tokens": w.chunk_tokens, "microbatches": w.microbatches,
                       "swap_bank_mib": args.swap_bank_mib,
                       "transport": args.transport, "ring_gather": args.ring_gather,
                       "compute_streams": args.compute_streams, "swap_calls": args.swap_calls,
                       **({"row_transport": args.row_transport,
                           "prompt_engines": args.prompt_engines,
                           "row_engines": args.row_engines,
                           "row_first": args.row_first,
                           "row_in_transport": args.row_in_transport,
                           "row_in_after": args.row_in_after,
                           "row_bank_mib": args.row_bank_mib,
                           "row_link_blocks": args.row_link_blocks}
                          if isinstance(step, LongStep) else {}),
                       "hw_queues": int(os.environ["GPU_MAX_HW_QUEUES"])},
            "roofline": roofline, "cpu_baseline": cpu, "detail": detail}
    # the metric names two figures: the in-step pack/unpack rate (of the
    # busiest HBM kernel, and of all of them together, with their shares of
    # the HBM peak) and the host-link rate (value)
    line["metric_parts"] = {
        "swap_host_link_GBps": line["value"],
        "host_link_d2h_GBps": directions["d2h"]["GBps"],
        "host_link_d2h_frac_of_pcie": directions["d2h"]["frac_of_pcie_peak"],
        "host_link_h2d_GBps": directions["h2d"]["GBps"],
        "host_link_h2d_frac_of_pcie": directions["h2d"]["frac_of_pcie_peak"],
        "pack_unpack_GBps": roofline["achieved"] if roofline else None,
        "pack_unpack_hbm_frac": roofline["frac"] if roofline else None,
        "pack_unpack_kernel": roofline["kernel"] if roofline else None,
        "pack_unpack_together_GBps": together["GBps"] if together else None,
        "pack_unpack_together_hbm_frac": together["frac_of_peak"] if together else None}
    if roofline:
        line["metric_parts"]["pack_unpack_payload_GBps"] = round(roofline["achieved"] / 2, 1)
        if roofline["traffic"]:
            line["metric_parts"]["pack_unpack_counter_traffic_GBps"] = round(
                roofline["traffic"] / (roofline["avg_us"] * 1e3), 1)
    # the pages' transfer estimate redone with this link's measured rate
    d2h = detail.get("link_ceiling_GBps", {}).get("d2h") or directions["d2h"]["GBps"]
    if d2h:
        one = PAGES_OPT175B_KV_BYTES / (d2h * 1e9) * 1000
        line["context"] = {"pages_throughput_vs_fastertransformer": PAGES_THROUGHPUT_VS_FT,
                           "pages_opt175b_2048_token_kv_ms_estimate_8_links": PAGES_OPT175B_ESTIMATE_MS,
                           "same_9_GiB_at_this_link_GBps": d2h,
                           "same_9_GiB_ms_one_link": round(one, 1),
                           "same_9_GiB_ms_8_links": round(one / 8, 1)}
        lap = detail.get("prompt_overlap")
        if lap:
            line["context"]["pages_layer_streaming_and_overlap_gain"] = PAGES_OVERLAP_GAIN
            line["context"]["this_gpu_prompt_overlap_gain_at_equal_compute"] = lap["rows"][1]["gain"]
        tok = detail.get("token_overlap")
        if tok:
            line["context"]["pages_layer_streaming_and_overlap_gain"] = PAGES_OVERLAP_GAIN
            line["context"]["this_gpu_token_overlap_gain_at_equal_compute"] = tok["rows"][1]["gain"]
        naive = detail.get("buffered_vs_naive")
        if naive:
            line["context"]["pages_buffered_copy_gain_over_naive_copies"] = PAGES_BUFFERED_GAIN
            for name in ("per_piece", "per_head"):
                if f"gain_over_{name}" in naive:
                    line["context"][f"this_gpu_decode_step_gain_over_{name}_copies"] = \
                        naive[f"gain_over_{name}"]
    ceiling = detail.get("hbm_copy_ceiling")
    if ceiling and roofline:
        # the dominant kernel against what HBM gives a plain copy on this GPU
        line["metric_parts"]["pack_unpack_frac_of_copy_ceiling"] = round(
            roofline["achieved"] / ceiling["kv_copy_packed_GBps"], 4)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
