"""Seeded synthetic inputs for the ISPA hot path.

This module only draws random tensors.  It contains none of the method's
arithmetic, and both the HIP path and the CPU oracle receive the same
tensors from it (the oracle gets a host copy), so the two sides never need
bit-identical random number generators of their own.

Distributions follow the workload descriptions: Q, K, V ~ N(0, 1);
W ~ N(0, 1/D); history keys carry a per-head offset 0.5 * u_h with u_h a
seeded unit vector, added in fp32 before one round-to-nearest-even cast.
Every tensor is drawn from its own stream, keyed by
(base seed, workload, layer, chunk, tensor id).
"""
from __future__ import annotations

import torch

# tensor ids inside a (workload, layer, chunk) key
T_Q, T_K, T_V, T_W, T_U = 0, 1, 2, 3, 4
_MASK64 = (1 << 64) - 1


def _splitmix64(x: int) -> int:
    x = (x + 0x9E3779B97F4A7C15) & _MASK64
    x = ((x ^ (x >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    x = ((x ^ (x >> 27)) * 0x94D049BB133111EB) & _MASK64
    return x ^ (x >> 31)


def stream_seed(base: int, workload: int, layer: int, chunk: int, tensor: int) -> int:
    """A 63-bit seed for one tensor, mixed from its key."""
    s = base & _MASK64
    for part in (workload, layer, chunk, tensor):
        s = _splitmix64(s ^ (part & _MASK64))
    return s & ((1 << 63) - 1)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, seed: int, device="cpu", std: float = 1.0,
           dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """N(0, std^2) drawn in fp32 and rounded once (RNE) to ``dtype``."""
    x = torch.randn(tuple(shape), generator=_gen(seed, device), device=device,
                    dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def unit_vectors(H: int, d: int, seed: int, device="cpu") -> torch.Tensor:
    """One seeded unit vector per head, fp32 [H, d]."""
    u = torch.randn((H, d), generator=_gen(seed, device), device=device,
                    dtype=torch.float32)
    return u / u.norm(dim=1, keepdim=True)


def keys_with_offset(n: int, H: int, d: int, seed: int, u: torch.Tensor | None,
                     shift: float = 0.5, device="cpu",
                     dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """Keys ~ N(0, 1) plus ``shift * u_h`` per head (fp32), one cast."""
    x = torch.randn((n, H, d), generator=_gen(seed, device), device=device,
                    dtype=torch.float32)
    if u is not None and shift != 0.0:
        x.add_(shift * u.to(device=device, dtype=torch.float32).unsqueeze(0))
    return x.to(dtype)


class GroupInputs:
    """Fixed-history warmup inputs (the single-layer workloads): a sink and a
    history drawn once, then per step a fresh current chunk of queries, keys
    and values.  ``n_q`` queries per step equal the current chunk's keys.

    Sizes are free so tests can use small ragged shapes; the named workloads
    are built by :func:`tiny_fp32` and :func:`wan13b_single_layer`."""

    def __init__(self, n_q, H, d, n_sink, n_hist, dtype, seed, device="cpu",
                 hist_shift=0.5, workload=0, layer=0):
        self.n_q, self.H, self.d = n_q, H, d
        self.D = H * d
        self.dtype, self.seed, self.device = dtype, seed, device
        self.workload, self.layer = workload, layer
        key = lambda chunk, t: stream_seed(seed, workload, layer, chunk, t)  # noqa: E731
        u = unit_vectors(H, d, key(0, T_U), device) if hist_shift else None
        # chunk index 0 = sink, 1 = history block, 2 + i = step i
        self.sink_k = normal((n_sink, H, d), key(0, T_K), device, dtype=dtype)
        self.sink_v = normal((n_sink, H, d), key(0, T_V), device, dtype=dtype)
        self.hist_k = keys_with_offset(n_hist, H, d, key(1, T_K), u, hist_shift,
                                       device, dtype)
        self.hist_v = normal((n_hist, H, d), key(1, T_V), device, dtype=dtype)
        self.w = normal((self.D, self.D), key(0, T_W), device,
                        std=self.D ** -0.5, dtype=dtype)

    def step(self, i: int):
        """(q, k_cur, v_cur) of warmup step i, each [n_q, H, d]."""
        key = lambda t: stream_seed(self.seed, self.workload, self.layer, 2 + i, t)  # noqa: E731
        shp = (self.n_q, self.H, self.d)
        return (normal(shp, key(T_Q), self.device, dtype=self.dtype),
                normal(shp, key(T_K), self.device, dtype=self.dtype),
                normal(shp, key(T_V), self.device, dtype=self.dtype))


def tiny_fp32(seed=1, device="cpu") -> GroupInputs:
    """1 layer, 2 heads x 64 (D = 128), 64 tokens per frame: sink 1 frame,
    current 1 frame, history 6 frames (384 keys), fp32."""
    return GroupInputs(64, 2, 64, 64, 384, torch.float32, seed, device,
                       hist_shift=0.0, workload=1)


def wan13b_single_layer(seed=1, device="cpu") -> GroupInputs:
    """Wan-1.3B-shaped layer: 12 heads x 128 (D = 1536), chunk of 4680
    queries, sink 4680 keys, history 28080 keys shifted by 0.5 u_h, bf16."""
    return GroupInputs(4680, 12, 128, 4680, 28080, torch.bfloat16, seed, device,
                       hist_shift=0.5, workload=2)


class StreamInputs:
    """Chunked-stream inputs (multi-layer workloads): for every (layer, chunk)
    a fresh chunk of Q, K, V [chunk_tokens, H, d]; keys of chunks >= 1 carry
    the layer's per-head offset 0.5 u_{layer,h} (the sink, chunk 0, does not);
    one W per layer ~ N(0, 1/D)."""

    def __init__(self, n_layers, H, d, chunk_tokens, dtype, seed, device="cpu",
                 hist_shift=0.5, workload=3):
        self.n_layers, self.H, self.d = n_layers, H, d
        self.D = H * d
        self.T = chunk_tokens
        self.dtype, self.seed, self.device = dtype, seed, device
        self.workload, self.hist_shift = workload, hist_shift

    def _key(self, layer, chunk, t):
        return stream_seed(self.seed, self.workload, layer, chunk, t)

    def q(self, layer, chunk):
        return normal((self.T, self.H, self.d), self._key(layer, chunk, T_Q),
                      self.device, dtype=self.dtype)

    def kv(self, layer, chunk):
        u = None
        if chunk >= 1 and self.hist_shift:
            u = unit_vectors(self.H, self.d, self._key(layer, 0, T_U), self.device)
        k = keys_with_offset(self.T, self.H, self.d, self._key(layer, chunk, T_K),
                             u, self.hist_shift, self.device, self.dtype)
        v = normal((self.T, self.H, self.d), self._key(layer, chunk, T_V),
                   self.device, dtype=self.dtype)
        return k, v

    def w(self, layer):
        return normal((self.D, self.D), self._key(layer, 0, T_W), self.device,
                      std=self.D ** -0.5, dtype=self.dtype)
