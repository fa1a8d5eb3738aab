"""Seeded synthetic inputs for the KV buffered-copy path.

This module holds only input generation -- cache contents, row lengths,
decode positions and the workload shapes -- and none of the method's
arithmetic (no offsets, no packing).  It is the one module that both the
HIP-path tests and the oracle-side tests draw their inputs from.

Workloads stand in for the pages' served models.  The shapes follow the
models the DejaVu summary evaluates ("Experimental setup": GPT2-1.5B, OPT-66B,
BLOOM-176B, fp16) and the long-context example of the lsln.cn decode-only
article ("KV Cache capacity": 100K context, 60 layers, 8 heads, 128 dims,
BF16).  Generated lengths on the pages are sampled from LMSys; that dataset is
not used here -- seeded uniform integer lengths stand in for it.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

F16 = 0
BF16 = 1


@dataclass(frozen=True)
class Workload:
    """One KV-cache shape and the call sequence run on it."""
    name: str
    L: int
    B: int
    H: int
    D: int
    Smax: int
    dtype: int
    value_seed: int
    length_seed: int
    prompt_len: int = 0          # uniform prompt length (0: per-row lengths)
    len_lo: int = 0              # per-row current lengths ~ U{len_lo..len_hi}
    len_hi: int = 0
    decode_steps: int = 0
    ring_slots: int = 0          # R: steps per staging bank
    chunk_tokens: int = 0        # prompt chunk size (0: whole prompt per layer)
    microbatches: int = 0        # swap round-robin microbatches
    extra: dict = field(default_factory=dict)

    @property
    def dims(self):
        return (self.L, self.B, self.H, self.D, self.Smax)


# The five workloads.  Seeds: values 1000+id, lengths 2000+id.
WORKLOADS = {
    "gpt2-small-tiny": Workload("gpt2-small-tiny", L=12, B=2, H=12, D=64, Smax=128,
                                dtype=F16, value_seed=1001, length_seed=2001,
                                prompt_len=32, decode_steps=16, ring_slots=8),
    "gpt2-1.5b": Workload("gpt2-1.5b", L=48, B=8, H=25, D=64, Smax=1024, dtype=F16,
                          value_seed=1002, length_seed=2002, prompt_len=1000,
                          decode_steps=24, ring_slots=8),
    "opt-66b-16l": Workload("opt-66b-16l", L=16, B=8, H=72, D=128, Smax=2048, dtype=F16,
                            value_seed=1003, length_seed=2003, len_lo=256, len_hi=1800,
                            decode_steps=64, ring_slots=16),
    "bloom-176b-10l": Workload("bloom-176b-10l", L=10, B=16, H=112, D=128, Smax=2048,
                               dtype=F16, value_seed=1004, length_seed=2004,
                               prompt_len=1500, microbatches=4),
    "gqa-100k": Workload("gqa-100k", L=60, B=4, H=8, D=128, Smax=100000, dtype=BF16,
                         value_seed=1005, length_seed=2005, len_lo=20000,
                         len_hi=100000 - 64, decode_steps=64, ring_slots=16,
                         chunk_tokens=4096),
}


def row_lengths(w: Workload) -> np.ndarray:
    """Per-row current lengths: the uniform prompt length, or seeded U{lo..hi}."""
    if w.prompt_len:
        return np.full(w.B, w.prompt_len, dtype=np.int32)
    rng = np.random.default_rng(w.length_seed)
    return rng.integers(w.len_lo, w.len_hi + 1, size=w.B, dtype=np.int64).astype(np.int32)


def decode_positions(w: Workload) -> np.ndarray:
    """[steps, B] positions: row b's step-j token sits at len_b + j."""
    lens = row_lengths(w).astype(np.int64)
    steps = np.arange(w.decode_steps, dtype=np.int64)[:, None]
    return (lens[None, :] + steps).astype(np.int32)


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((u >> 16) & 1)
    return ((u + bias) >> 16).astype(np.uint16)


def cache_values(n: int, seed: int, dtype: int = F16) -> np.ndarray:
    """n 16-bit words: seeded uniform values in [-4, 4], rounded to fp16/bf16."""
    rng = np.random.default_rng(seed)
    x = rng.uniform(-4.0, 4.0, size=n).astype(np.float32)
    if dtype == F16:
        return x.astype(np.float16).view(np.uint16)
    return _to_bf16_bits(x)


def random_bits(n: int, seed: int) -> np.ndarray:
    """n arbitrary 16-bit patterns (NaN payloads, Inf, +-0, subnormals included)."""
    rng = np.random.default_rng(seed)
    a = rng.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)
    # make sure the special classes are present even in short draws
    specials = np.array([0x0000, 0x8000, 0x7C00, 0xFC00, 0x7E01, 0xFD55, 0x0001, 0x83FF,
                         0x7F80, 0xFF80, 0x7FC1, 0x0080], dtype=np.uint16)
    k = min(n, specials.size)
    a[:k] = specials[:k]
    return a


def cache_pair(dims, seed: int, dtype: int = F16, bits: bool = False):
    """(K, V) flat uint16 caches of the given dims, seeded."""
    L, B, H, D, S = dims
    n = L * B * H * D * S
    gen = random_bits if bits else (lambda m, s: cache_values(m, s, dtype))
    return gen(n, seed), gen(n, seed + 7919)


def fill_device_cache(t, seed: int, dtype: int = F16, chunk_elems: int = 1 << 28) -> None:
    """Fill a flat int16/uint16-sized torch device tensor with seeded values in [-4, 4].

    Chunked so the float32 temporary stays small; uses a device generator, so the
    stream of values depends on (seed, chunk_elems) only.
    """
    import torch
    g = torch.Generator(device=t.device)
    g.manual_seed(seed)
    flat = t.view(-1)
    n = flat.numel()
    tgt = torch.float16 if dtype == F16 else torch.bfloat16
    for i in range(0, n, chunk_elems):
        m = min(chunk_elems, n - i)
        tmp = torch.empty(m, dtype=torch.float32, device=t.device)
        tmp.uniform_(-4.0, 4.0, generator=g)
        flat[i:i + m].copy_(tmp.to(tgt).view(flat.dtype))
        del tmp
