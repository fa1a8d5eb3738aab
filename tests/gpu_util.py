"""Helpers shared by the GPU tests: host<->device copies of raw 16-bit words."""
from __future__ import annotations

import sys

import numpy as np


def note(msg: str) -> None:
    """Name the case about to run on the GPU (flushed before the GPU step)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev(words: np.ndarray, extra: int = 0, fill: int = 0):
    """Device int16 tensor holding `words` (uint16), plus `extra` trailing words."""
    import torch
    t = torch.full((words.size + extra,), fill - 65536 if fill >= 32768 else fill,
                   dtype=torch.int16, device="cuda")
    if words.size:
        t[:words.size].copy_(torch.from_numpy(words.view(np.int16)))
    return t


def host(t) -> np.ndarray:
    """uint16 numpy copy of a device int16 tensor."""
    return t.detach().cpu().numpy().view(np.uint16).copy()


def empty(words: int, extra: int = 0, fill: int = 0x7A7A):
    """Device int16 tensor of words+extra, filled with a canary pattern."""
    import torch
    return torch.full((words + extra,), fill - 65536 if fill >= 32768 else fill,
                      dtype=torch.int16, device="cuda")


def pinned(words: int, fill: int = 0x5C5C):
    import torch
    t = torch.empty(words, dtype=torch.int16, pin_memory=True)
    t.fill_(fill - 65536 if fill >= 32768 else fill)
    return t


def pinned_host_view(t) -> np.ndarray:
    return t.numpy().view(np.uint16)
