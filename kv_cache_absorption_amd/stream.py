"""Host-side layout of a chunked stream: key groups and KV accounting.

A layer's keys and values live in one caller-owned cache of token rows
[max_tokens, H, d]; chunk c occupies rows [c*T, (c+1)*T).  Chunk 0 holds the
sink.  At chunk step c >= 1 the local group is {sink, chunk c} and the
history group is chunks 1 .. c-1 (EN review, Key Design 1: local = initial
sink frame(s) + current frame(s), history = the frames in between); at c = 0
the local group is chunk 0 alone.  After the switch an L-Layer keeps only its
sink and current rows, an F-Layer keeps everything (EN review, Key Design 3).
"""
from __future__ import annotations

import torch


def chunk_segments(k_cache: torch.Tensor, v_cache: torch.Tensor, c: int, T: int):
    """(local, history) lists of (k, v) row views of one layer's cache at chunk c."""
    def rows(a, b):
        return (k_cache[a:b], v_cache[a:b])
    if c == 0:
        return [rows(0, T)], []
    local = [rows(0, T), rows(c * T, (c + 1) * T)]
    hist = [rows(T, c * T)] if c >= 2 else []
    return local, hist


def kv_bytes(n_keys_per_layer, D: int, elem_bytes: int = 2) -> int:
    """Bytes of K and V held for the given per-layer key counts."""
    total = 0
    for n in n_keys_per_layer:
        total += 2 * int(n) * int(D) * elem_bytes
    return total


def keys_retained(c: int, T: int, is_local) -> list:
    """Per-layer key counts held at chunk c after the switch."""
    full = (c + 1) * T
    local = T if c == 0 else 2 * T
    return [local if flag else full for flag in is_local]


class Workspace:
    """A grow-only device byte buffer reused across calls on one stream."""

    def __init__(self, device):
        self.device = device
        self.buf = None

    def get(self, nbytes: int):
        if nbytes == 0:
            return None
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return self.buf
