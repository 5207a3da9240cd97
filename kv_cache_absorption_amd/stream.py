"""Host-side layout and driver of a chunked stream: key groups, KV caches,
the warmup -> switch -> post-switch sequence, and KV accounting.

A layer's keys and values live in one device cache of token rows
[capacity, H, d]; while the layer keeps its full history, chunk c occupies
rows [c*T, (c+1)*T).  Chunk 0 holds the sink.  At chunk step c >= 1 the local
group is {sink, chunk c} and the history group is chunks 1 .. c-1 (EN review,
Key Design 1: local = initial sink frame(s) + current frame(s), history = the
frames in between); at c = 0 the local group is chunk 0 alone.  After the
switch an L-Layer keeps only its sink and current rows, an F-Layer keeps
everything (EN review, Key Design 3).

Every arithmetic step runs in libispa; this module only decides which call
gets which rows, allocates caches and buffers with torch, and counts bytes.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib as B


def chunk_segments(k_cache: torch.Tensor, v_cache: torch.Tensor, c: int, T: int, slot: int | None = None):
    """(local, history) lists of (k, v) row views of one layer's cache at chunk
    c, whose rows sit in cache slot ``slot`` (default c: the layer holds every
    chunk in order).  History is every slot between the sink and the current
    chunk."""
    def rows(a, b):
        return (k_cache[a:b], v_cache[a:b])
    sc = c if slot is None else slot
    if c == 0:
        return [rows(0, T)], []
    local = [rows(0, T), rows(sc * T, (sc + 1) * T)]
    hist = [rows(T, sc * T)] if sc >= 2 else []
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
            self.buf = None
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return self.buf

    def release(self):
        self.buf = None


class LayerKV:
    """K and V rows of one layer.

    While the layer is full, slot 0 holds the sink and chunk c >= first lives
    in slot c - first + 1 (first = 1 from the start, so chunk c is in slot c,
    rows [cT, (c+1)T)).  After :meth:`evict_history` (an L-Layer) the cache
    shrinks to two slots: the sink stays in slot 0 and every later chunk is
    written to slot 1, replacing the previous current chunk.
    :meth:`keep_from` makes such a layer full again from its last chunk on
    (re-entering warmup)."""

    def __init__(self, capacity_chunks: int, T: int, H: int, d: int, dtype, device):
        self.T, self.H, self.d = T, H, d
        self.dtype, self.device = dtype, device
        self.local_only = False
        self.first = 1     # first history chunk held while full
        self.last = -1     # last chunk written
        self._alloc(capacity_chunks)

    def _alloc(self, chunks: int):
        self.capacity = chunks
        self.k = torch.empty((chunks * self.T, self.H, self.d), dtype=self.dtype, device=self.device)
        self.v = torch.empty_like(self.k)

    def slot(self, c: int) -> int:
        if self.local_only:
            return min(c, 1)
        if c == 0:
            return 0
        if c < self.first:
            raise ValueError(f"chunk {c} precedes the first history chunk held ({self.first})")
        return c - self.first + 1

    def _rows(self, a: int, b: int):
        return (self.k[a * self.T:b * self.T], self.v[a * self.T:b * self.T])

    def write(self, c: int, k: torch.Tensor, v: torch.Tensor):
        """Store chunk c's keys and values (the output of the model's K/V projection)."""
        s = self.slot(c)
        if s >= self.capacity:
            self.grow(max(s + 1, 2 * self.capacity))
        kk, vv = self._rows(s, s + 1)
        kk.copy_(k)
        vv.copy_(v)
        self.last = c

    def grow(self, chunks: int):
        """Reallocate with room for ``chunks`` slots, keeping the rows held."""
        old_k, old_v, n = self.k, self.v, self.capacity
        self._alloc(chunks)
        self.k[:n * self.T].copy_(old_k)
        self.v[:n * self.T].copy_(old_v)

    def evict_history(self):
        """Keep the sink (slot 0) only, in a two-slot cache; frees the history rows."""
        sink_k, sink_v = self._rows(0, 1)
        sink_k, sink_v = sink_k.clone(), sink_v.clone()
        self.k = self.v = None
        self._alloc(2)
        self.k[:self.T].copy_(sink_k)
        self.v[:self.T].copy_(sink_v)
        self.local_only = True
        self.last = 0  # nothing but the sink is held until the next chunk

    def keep_from(self, c: int):
        """Re-enter warmup at chunk c: a full layer keeps everything; an
        L-Layer becomes full again, holding its sink and its last chunk (if it
        wrote one since the eviction), and keeps every chunk from then on."""
        if not self.local_only:
            return
        if self.last >= 1 and self.last < c:
            self.first = self.last          # already in slot 1
        else:
            self.first = c                  # only the sink is held
        self.local_only = False

    def warmup_groups(self, c: int):
        """(local, history) segment lists at warmup chunk c (the layer is full)."""
        assert not self.local_only
        return chunk_segments(self.k, self.v, c, self.T, self.slot(c))

    def attend_all(self, c: int):
        """Segments of every key the layer holds at chunk c: for a full layer
        rows [0, (c+1)T); for an L-Layer the sink and the current chunk (which
        sit next to each other in slots 0 and 1)."""
        hi = self.slot(c) + 1
        return [self._rows(0, hi)]

    def keys_held(self, c: int) -> int:
        return (self.slot(c) + 1) * self.T

    def bytes_allocated(self) -> int:
        return 2 * self.k.numel() * self.k.element_size()


class IspaStream:
    """One stream of ``n_layers`` attention layers through the ISPA cycle.

    ``with_stats=False`` skips the statistics (a stream that starts after a
    switch made elsewhere, see :meth:`adopt_switch`).

    ``capacity`` is the number of chunk slots each layer's cache starts with
    (an int, or one per layer); a full layer's cache grows when a chunk lands
    past it.

    Usage: for warmup chunks call :meth:`write_kv` then :meth:`warmup` for
    each layer; call :meth:`switch` once; afterwards :meth:`write_kv` and
    :meth:`post` per layer and chunk.  Results of a call live in buffers that
    the next call on the stream overwrites (views are returned).

    Device state per layer: the KV cache, W (bf16 [D, D], y = a W) and the
    warmup statistics.  ``stats="gram"`` (the default) accumulates them in the
    grouping of the printed closed form: one rank-k update of [A_loc | dA]
    into a per-layer state (ispa_accum_gram) for every ``stats_chunks`` (4)
    chunks of a layer (their rows wait in a per-layer buffer; the sums do not
    depend on the grouping, and one update over more rows pays the state's
    read-modify-write once), and G, C = M W and r2 formed once at the switch
    (ispa_gram_finalize), after the rows still waiting are added.  ``stats="direct"``
    accumulates G, C = A_loc^T (dA W) and r2 every chunk (ispa_accum_stats).
    For the switch, G, C (fp32 [N, D, D], so that one call solves every
    layer) and r2 (fp64 [N]); after it dW (fp32), eps (fp64), W + dW (bf16),
    the selection and the L/F mask.
    """

    def __init__(self, n_layers: int, H: int, d: int, T: int, capacity,
                 device, dtype=torch.bfloat16, stats_dtype=torch.float16,
                 lambda_abs: float = 0.0, lambda_rel: float = 1e-3, scale: float | None = None,
                 with_stats: bool = True, stats: str = "gram", stats_chunks: int = 4):
        if dtype != torch.bfloat16:
            raise ValueError("streams run on bf16 Q/K/V")
        if stats not in ("gram", "direct"):
            raise ValueError("stats is 'gram' or 'direct'")
        if stats_chunks < 1:
            raise ValueError("stats_chunks must be >= 1")
        self.N, self.H, self.d, self.T = n_layers, H, d, T
        self.D = H * d
        self.device, self.dtype, self.stats_dtype = device, dtype, stats_dtype
        self.lambda_abs, self.lambda_rel = lambda_abs, lambda_rel
        self.scale = d ** -0.5 if scale is None else scale
        self.L = B.lib()
        D, dev = self.D, device
        f32 = dict(dtype=torch.float32, device=dev)
        caps = [capacity] * n_layers if isinstance(capacity, int) else list(capacity)
        if len(caps) != n_layers:
            raise ValueError("one capacity per layer")
        self.kv = [LayerKV(cap, T, H, d, dtype, dev) for cap in caps]
        self.W = torch.empty((n_layers, D, D), dtype=dtype, device=dev)
        self.stats = stats
        self.stats_chunks = stats_chunks if stats == "gram" else 1
        self._pend = [None] * n_layers  # per layer: (A_loc, dA) rows of stats_chunks chunks
        self._npend = [0] * n_layers    # chunks waiting in them
        self.has_stats = with_stats
        self.G = self.C = self.r2 = self.state = None
        if with_stats and stats == "gram":
            self.state = B.gram_state(D, n_layers, dev)
        elif with_stats:
            self.G = torch.zeros((n_layers, D, D), **f32)
            self.C = torch.zeros((n_layers, D, D), **f32)
            self.r2 = torch.zeros(n_layers, dtype=torch.float64, device=dev)
        self.lse_full = torch.empty((T, H), **f32)
        self.a_loc = torch.empty((T, D), dtype=stats_dtype, device=dev)
        self.delta = torch.empty_like(self.a_loc)
        self.y = torch.empty((T, D), dtype=dtype, device=dev)
        self.ws = Workspace(dev)
        self.switched = False
        self.dW = self.eps = self.info = self.w_eff = None
        self.wq = self.wq_scale = None  # W8A8 projection codes and scales, when quantised
        self.sink8 = None  # fp8 caches of the L-Layers' sinks, when their attention is quantised
        self.cur8 = None   # fp8 cache buffers of the current chunk (reused for every layer)
        self.f8 = None     # per F-Layer, the fp8 caches of its chunks (slot order), when quantised
        self.selected = self.is_local = self.status = None
        self.is_local_host = None
        self.warmups = 1  # warmup phases entered (re-calibration adds one)

    # ------------------------------------------------------------------ helpers
    def _ck(self, st):
        if st != B.ISPA_OK:
            raise B.IspaError(st, self.L.ispa_last_error().decode())

    def _stream(self) -> int:
        return torch.cuda.current_stream(self.device).cuda_stream

    def _segs(self, pairs):
        return B._segs(pairs, self.H, self.d)

    def set_w(self, layer: int, w: torch.Tensor):
        self.W[layer].copy_(w)

    def write_kv(self, layer: int, c: int, k: torch.Tensor, v: torch.Tensor):
        self.kv[layer].write(c, k, v)

    # ------------------------------------------------------------------ warmup
    def warmup(self, layer: int, c: int, q: torch.Tensor):
        """Chunk c of one layer during warmup: dual-stream attention over the
        local and history groups merged by their LSE into A_loc and
        A_full - A_loc (one fused call), and the statistics update.  Returns
        (a_loc, delta, lse_full) views."""
        if self.switched or not self.has_stats:
            raise RuntimeError("warmup needs the statistics and must come before the switch")
        if q.shape != (self.T, self.H, self.d) or q.dtype != self.dtype:
            raise ValueError("q must be [T, H, d] bf16")
        L, s = self.L, self._stream()
        loc, hist = self.kv[layer].warmup_groups(c)
        ls, nl = self._segs(loc)
        hs, nh = self._segs(hist)
        n, sdt = self.T, B._DT[self.stats_dtype]
        need = L.ispa_dual_attn_merge_workspace_bytes(B.ISPA_BF16, n, self.H, self.d, ls, nl, hs, nh)
        if self.stats == "direct":
            need = max(need, L.ispa_accum_stats_workspace_bytes(sdt, n, self.D))
        ws = self.ws.get(need)
        wsp = ws.data_ptr() if ws is not None else None
        a_loc, delta = self.a_loc, self.delta
        if self.stats == "gram" and self.stats_chunks > 1:
            if self._pend[layer] is None:
                rows = self.stats_chunks * n
                self._pend[layer] = (torch.empty((rows, self.D), dtype=self.stats_dtype, device=self.device),
                                     torch.empty((rows, self.D), dtype=self.stats_dtype, device=self.device))
            off = self._npend[layer] * n
            a_loc, delta = self._pend[layer][0][off:off + n], self._pend[layer][1][off:off + n]
        self._ck(L.ispa_dual_attn_merge(B.ISPA_BF16, n, self.H, self.d, self.scale, q.data_ptr(), q.stride(0),
                                        ls, nl, hs, nh, a_loc.data_ptr(), delta.data_ptr(),
                                        sdt, self.lse_full.data_ptr(), wsp, need, s))
        if self.stats == "gram" and self.stats_chunks > 1:
            self._npend[layer] += 1
            if self._npend[layer] == self.stats_chunks:
                self._flush_layer(layer)
        elif self.stats == "gram":
            self._ck(L.ispa_accum_gram(sdt, n, self.D, a_loc.data_ptr(), delta.data_ptr(),
                                       self.state[layer].data_ptr(), s))
        else:
            self._ck(L.ispa_accum_stats(sdt, B.ISPA_BF16, n, self.D,
                                        self.a_loc.data_ptr(), self.delta.data_ptr(),
                                        self.W[layer].data_ptr(), self.G[layer].data_ptr(),
                                        self.C[layer].data_ptr(), self.r2[layer:layer + 1].data_ptr(),
                                        wsp, need, s))
        return a_loc, delta, self.lse_full

    def _flush_layer(self, layer: int):
        # the rows waiting for this layer's statistics, in one rank-k update
        k = self._npend[layer]
        if k:
            a, dl = self._pend[layer]
            self._ck(self.L.ispa_accum_gram(B._DT[self.stats_dtype], k * self.T, self.D, a.data_ptr(),
                                            dl.data_ptr(), self.state[layer].data_ptr(), self._stream()))
            self._npend[layer] = 0

    def flush_statistics(self):
        """Add every layer's waiting chunks to its statistics state now."""
        if self.stats == "gram" and self.state is not None:
            for layer in range(self.N):
                self._flush_layer(layer)

    def statistics(self):
        """G (upper triangle), C and r2 of every layer from the warmup so far
        (with the grouped statistics: formed from the states now, which stay
        as they are).  Returns the (G, C, r2) buffers the solve reads."""
        if not self.has_stats:
            raise RuntimeError("this stream keeps no statistics")
        if self.stats == "gram":
            self.flush_statistics()
            self._reserve_stats_out()
            L, N, D = self.L, self.N, self.D
            need = L.ispa_gram_finalize_workspace_bytes(D)
            if getattr(self, "_fin_ws", None) is None or self._fin_ws.numel() < need:
                self._fin_ws = torch.empty(need, dtype=torch.uint8, device=self.device)
            self._ck(L.ispa_gram_finalize(N, D, self.state.data_ptr(), self.state.shape[1], self.W.data_ptr(),
                                          B.ISPA_BF16, D * D, self.G.data_ptr(), self.C.data_ptr(),
                                          self.r2.data_ptr(), D * D, self._fin_ws.data_ptr(), need,
                                          self._stream()))
        return self.G, self.C, self.r2

    def _reserve_stats_out(self):
        if self.G is None:
            N, D, dev = self.N, self.D, self.device
            self.G = torch.zeros((N, D, D), dtype=torch.float32, device=dev)
            self.C = torch.empty((N, D, D), dtype=torch.float32, device=dev)
            self.r2 = torch.empty(N, dtype=torch.float64, device=dev)

    # ------------------------------------------------------------------ switch
    def reserve_switch(self):
        """Allocate the switch's outputs (dW, eps, info, W + dW) and the solve's
        workspace now, so that :meth:`switch` allocates nothing; they are reused
        by every later switch (re-calibration)."""
        N, D, dev = self.N, self.D, self.device
        if self.stats == "gram" and self.has_stats:
            self._reserve_stats_out()
            need = self.L.ispa_gram_finalize_workspace_bytes(D)
            if getattr(self, "_fin_ws", None) is None or self._fin_ws.numel() < need:
                self._fin_ws = torch.empty(need, dtype=torch.uint8, device=dev)
        if self.dW is None:
            self.dW = torch.empty((N, D, D), dtype=torch.float32, device=dev)
            self.eps = torch.empty(N, dtype=torch.float64, device=dev)
            self.info = torch.empty(N, dtype=torch.int32, device=dev)
            self.w_eff = torch.empty_like(self.W)
        need = self.L.ispa_solve_dw_workspace_bytes(N, D)
        if getattr(self, "_solve_ws", None) is None or self._solve_ws.numel() < need:
            self._solve_ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def switch(self, K: int, evict: bool = True):
        """Ridge solve of every layer in one batched call (dW, eps, W + dW),
        selection of the K lowest-eps layers, then (optionally) eviction of the
        L-Layers' history.  Synchronises once to read the L/F mask on the host,
        which decides the later calls."""
        L, s, N, D = self.L, self._stream(), self.N, self.D
        dev = self.device
        self.reserve_switch()
        self.statistics()
        ws = self._solve_ws
        need = ws.numel()
        self._ck(L.ispa_solve_dw(N, D, self.G.data_ptr(), self.C.data_ptr(), self.r2.data_ptr(), D * D,
                                 self.lambda_abs, self.lambda_rel, self.dW.data_ptr(), self.eps.data_ptr(),
                                 self.info.data_ptr(), self.W.data_ptr(), B.ISPA_BF16,
                                 self.w_eff.data_ptr(), ws.data_ptr(), need, s))
        self.selected = torch.empty(max(K, 1), dtype=torch.int32, device=dev)
        self.is_local = torch.empty(N, dtype=torch.uint8, device=dev)
        self.status = torch.empty(1, dtype=torch.int32, device=dev)
        self._ck(L.ispa_select_layers(N, K, self.eps.data_ptr(), self.selected.data_ptr(),
                                      self.is_local.data_ptr(), self.status.data_ptr(), s))
        self.K = K
        self.is_local_host = [int(x) for x in self.is_local.cpu()]  # synchronises
        if int(self.status.cpu()[0]) != 0 or any(int(x) != 0 for x in self.info.cpu()):
            raise RuntimeError("switch failed: eps is NaN or a Gram matrix is not positive definite")
        self.switched = True
        if evict:
            self.evict()
        return self.selected[:K], self.is_local, self.eps

    def evaluate(self, Ks):
        """Solve every layer on the statistics gathered so far and select the
        K lowest-eps layers for each K in ``Ks``, without ending the warmup
        (a budget / warmup-length sweep: the pages' ablation axes x = K / N and
        the warmup length; EN review, Ablation Study).  The statistics are not
        modified (chunks still waiting are added to the state first, which
        leaves the sums as they are); warmup may continue afterwards.  Returns (eps [N] fp64,
        {K: selected int32 [K]}, {K: is_local uint8 [N]}, info [N] int32,
        dW [N, D, D] fp32), all on the device."""
        if self.switched or not self.has_stats:
            raise RuntimeError("evaluate runs during warmup")
        L, s, N, D, dev = self.L, self._stream(), self.N, self.D, self.device
        self.statistics()
        dW = torch.empty((N, D, D), dtype=torch.float32, device=dev)
        eps = torch.empty(N, dtype=torch.float64, device=dev)
        info = torch.empty(N, dtype=torch.int32, device=dev)
        need = L.ispa_solve_dw_workspace_bytes(N, D)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        self._ck(L.ispa_solve_dw(N, D, self.G.data_ptr(), self.C.data_ptr(), self.r2.data_ptr(), D * D,
                                 self.lambda_abs, self.lambda_rel, dW.data_ptr(), eps.data_ptr(),
                                 info.data_ptr(), None, B.ISPA_BF16, None, ws.data_ptr(), need, s))
        sels, masks = {}, {}
        status = torch.empty(1, dtype=torch.int32, device=dev)
        for K in Ks:
            if not 0 <= K <= N:
                raise ValueError("K must lie in 0 .. n_layers")
            sel = torch.empty(max(K, 1), dtype=torch.int32, device=dev)
            mask = torch.empty(N, dtype=torch.uint8, device=dev)
            self._ck(L.ispa_select_layers(N, K, eps.data_ptr(), sel.data_ptr(), mask.data_ptr(),
                                          status.data_ptr(), s))
            sels[K], masks[K] = sel[:K], mask
        return eps, sels, masks, info, dW

    def evict(self):
        """Free the history rows of every L-Layer; drop the statistics."""
        for layer, flag in enumerate(self.is_local_host):
            if flag:
                self.kv[layer].evict_history()
        self.G = self.C = self.state = None
        self._pend = [None] * self.N
        self._npend = [0] * self.N
        self._solve_ws = self._fin_ws = None
        self.ws.release()

    def adopt_switch(self, is_local, w_eff, dW=None, eps=None):
        """Start a stream directly in the post-switch phase with a selection
        and W + dW computed elsewhere (e.g. an earlier stream of the same
        layers)."""
        self.is_local_host = [int(x) for x in is_local]
        self.w_eff = w_eff
        self.dW, self.eps = dW, eps
        self.switched = True
        for layer, flag in enumerate(self.is_local_host):
            if flag:
                self.kv[layer].evict_history()
        self.G = self.C = self.state = None
        self._pend = [None] * self.N
        self._npend = [0] * self.N
        self.has_stats = False

    def quantize_projections(self):
        """W8A8 post-switch projections (the pages report ISPA combined with
        W8A8 quantisation; EN review, Key Findings): quantise each layer's
        projection once, W + dW for an L-Layer and W for an F-Layer, to FP8
        E4M3 codes with one scale per output column.  Later :meth:`post` calls
        then quantise the attention output per token and project on the fp8
        matrix core.  Call after the switch; a re-calibration drops the codes."""
        if not self.switched:
            raise RuntimeError("projections are quantised after the switch")
        L, s, N, D, dev = self.L, self._stream(), self.N, self.D, self.device
        self.wq = torch.empty((N, D, D), dtype=torch.uint8, device=dev)
        self.wq_scale = torch.empty((N, D), dtype=torch.float32, device=dev)
        need = L.ispa_quantize_w_fp8_workspace_bytes(D, D)
        ws = self.ws.get(need)
        for layer in range(N):
            w = self.w_eff[layer] if self.is_local_host[layer] else self.W[layer]
            self._ck(L.ispa_quantize_w_fp8(B.ISPA_BF16, D, D, w.data_ptr(), self.wq[layer].data_ptr(),
                                           self.wq_scale[layer].data_ptr(), ws.data_ptr(), need, s))

    def quantize_attention(self, f_layers: bool = True):
        """Quantised post-switch attention (fp8 cache, E4M3 codes with a
        power-of-two scale per chunk and head; the attention on the fp8
        matrix core, then the W8A8 projection, ispa_local_attn_fp8_proj).

        L-Layers: each sink is quantised once here, each later current chunk
        in :meth:`post`.  F-Layers (when ``f_layers``): every chunk the layer
        holds is quantised once, the chunks held now at their first
        :meth:`post`, each later chunk at the post() of its own step, and the
        layer attends over all of them (at most ISPA_MAX_SEGS_FP8 chunks).
        Needs :meth:`quantize_projections` first and the L-Layers' sinks
        written (chunk 0); a re-calibration drops the caches."""
        if self.wq is None:
            raise RuntimeError("quantize the projections first")
        s = self._stream()
        need = self.L.ispa_quantize_kv_fp8_workspace_bytes(self.T, self.H, self.d)
        self.sink8 = {}
        for layer, flag in enumerate(self.is_local_host):
            if flag:
                k, v = self.kv[layer]._rows(0, 1)
                self.sink8[layer] = self._chunk_bufs()
                self._quantize_chunk(k, v, self.sink8[layer], need, s)
        self.cur8 = self._chunk_bufs()
        self.f8 = {layer: [] for layer, flag in enumerate(self.is_local_host) if not flag} if f_layers else None

    def quantize_local_attention(self):
        """:meth:`quantize_attention` for the L-Layers only (F-Layers keep
        bf16 attention with the W8A8 projection)."""
        self.quantize_attention(f_layers=False)

    def _chunk_bufs(self):
        L, T, H, d, dev = self.L, self.T, self.H, self.d, self.device
        nb = L.ispa_kv_fp8_bytes(T, H, d)
        return B.Fp8Chunk(torch.empty(nb, dtype=torch.uint8, device=dev),
                          torch.empty(nb, dtype=torch.uint8, device=dev),
                          torch.empty(H, dtype=torch.float32, device=dev),
                          torch.empty(H, dtype=torch.float32, device=dev), T, H)

    def _quantize_chunk(self, k, v, c8, need, s):
        ws = self.ws.get(need)
        self._ck(self.L.ispa_quantize_kv_fp8(B.ISPA_BF16, self.T, self.H, self.d, k.data_ptr(), k.stride(0),
                                             v.data_ptr(), v.stride(0), c8.k_codes.data_ptr(),
                                             c8.v_codes.data_ptr(), c8.k_scales.data_ptr(),
                                             c8.v_scales.data_ptr(), ws.data_ptr(), need, s))

    def recalibrate(self, c: int):
        """Re-enter warmup at chunk c (after a scene change, which the caller
        detects; EN review, Limitations: warmup is re-entered to refresh the
        layer selection and the weight corrections).  The statistics restart
        from zero, every layer goes back to dual-stream attention with its
        original W over the keys it still holds plus the chunks that arrive
        (an L-Layer holds its sink and last chunk), and the next
        :meth:`switch` solves, selects and evicts again."""
        if not self.switched:
            raise RuntimeError("re-calibration starts from a switched stream")
        D, dev = self.D, self.device
        self.has_stats = True
        if self.stats == "gram":
            if self.state is None:
                self.state = B.gram_state(D, self.N, dev)
            else:
                self.state.zero_()
            self._npend = [0] * self.N
        else:
            if self.G is None:
                self.G = torch.empty((self.N, D, D), dtype=torch.float32, device=dev)
                self.C = torch.empty_like(self.G)
            if self.r2 is None:
                self.r2 = torch.empty(self.N, dtype=torch.float64, device=dev)
            self.G.zero_()
            self.C.zero_()
            self.r2.zero_()
        for kv in self.kv:
            kv.keep_from(c)
        self.switched = False
        self.selected = self.is_local = self.status = None
        self.wq = self.wq_scale = None
        self.sink8 = self.cur8 = self.f8 = None
        self.warmups += 1

    # ------------------------------------------------------------------ post-switch
    def post(self, layer: int, c: int, q: torch.Tensor):
        """Chunk c of one layer after the switch: an L-Layer attends to its
        sink and current chunk and projects with W + dW; an F-Layer attends to
        all its keys and projects with W.  Returns the y [T, D] bf16 view."""
        if not self.switched:
            raise RuntimeError("post-switch call before the switch")
        L, s = self.L, self._stream()
        local = bool(self.is_local_host[layer])
        if local and self.sink8 is not None:  # fp8 attention over sink + current, W8A8 projection
            chunks8 = [self.sink8[layer]]
            if self.kv[layer].slot(c) == 1:  # a current chunk besides the sink
                k, v = self.kv[layer]._rows(1, 2)
                self._quantize_chunk(k, v, self.cur8, L.ispa_quantize_kv_fp8_workspace_bytes(self.T, self.H, self.d),
                                     s)
                chunks8.append(self.cur8)
            segs8, ns8 = B._segs_fp8(chunks8)
            need = L.ispa_local_attn_fp8_proj_workspace_bytes(self.T, self.H, self.d)
            ws = self.ws.get(need)
            self._ck(L.ispa_local_attn_fp8_proj(self.T, self.H, self.d, self.scale, B.ISPA_BF16, q.data_ptr(),
                                                q.stride(0), segs8, ns8, self.wq[layer].data_ptr(),
                                                self.wq_scale[layer].data_ptr(), self.y.data_ptr(), B.ISPA_BF16,
                                                ws.data_ptr(), need, s))
            return self.y
        if not local and self.f8 is not None:  # fp8 attention over all the F-Layer's chunks, W8A8 projection
            kvl, chunks8 = self.kv[layer], self.f8[layer]
            n_slots = kvl.slot(c) + 1
            if n_slots > B.ISPA_MAX_SEGS_FP8:
                raise RuntimeError(f"an F-Layer's quantised attention takes at most {B.ISPA_MAX_SEGS_FP8} chunks")
            need_q = L.ispa_quantize_kv_fp8_workspace_bytes(self.T, self.H, self.d)
            while len(chunks8) < n_slots:  # chunks not yet in the fp8 cache (written since the last call)
                k, v = kvl._rows(len(chunks8), len(chunks8) + 1)
                c8 = self._chunk_bufs()
                self._quantize_chunk(k, v, c8, need_q, s)
                chunks8.append(c8)
            segs8, ns8 = B._segs_fp8(chunks8[:n_slots])
            need = L.ispa_local_attn_fp8_proj_workspace_bytes(self.T, self.H, self.d)
            ws = self.ws.get(need)
            self._ck(L.ispa_local_attn_fp8_proj(self.T, self.H, self.d, self.scale, B.ISPA_BF16, q.data_ptr(),
                                                q.stride(0), segs8, ns8, self.wq[layer].data_ptr(),
                                                self.wq_scale[layer].data_ptr(), self.y.data_ptr(), B.ISPA_BF16,
                                                ws.data_ptr(), need, s))
            return self.y
        segs, ns = self._segs(self.kv[layer].attend_all(c))
        if self.wq is not None:  # W8A8 projection
            need = L.ispa_local_attn_proj_fp8_workspace_bytes(self.T, self.H, self.d, segs, ns)
            ws = self.ws.get(need)
            self._ck(L.ispa_local_attn_proj_fp8(self.T, self.H, self.d, self.scale, q.data_ptr(), q.stride(0),
                                                segs, ns, self.wq[layer].data_ptr(),
                                                self.wq_scale[layer].data_ptr(), self.y.data_ptr(),
                                                B.ISPA_BF16, ws.data_ptr() if ws is not None else None,
                                                need, s))
            return self.y
        w = self.w_eff[layer] if local else self.W[layer]
        need = L.ispa_local_attn_proj_workspace_bytes(B.ISPA_BF16, self.T, self.H, self.d, segs, ns)
        ws = self.ws.get(need)
        self._ck(L.ispa_local_attn_proj(B.ISPA_BF16, self.T, self.H, self.d, self.scale, q.data_ptr(),
                                        q.stride(0), segs, ns, w.data_ptr(), B.ISPA_BF16,
                                        self.y.data_ptr(), B.ISPA_BF16,
                                        ws.data_ptr() if ws is not None else None, need, s))
        return self.y

    # ------------------------------------------------------------------ accounting
    def keys_held(self, c: int) -> list:
        return [kv.keys_held(c) for kv in self.kv]

    def kv_bytes_held(self, c: int) -> int:
        """Bytes of the K and V rows the layers hold at chunk c."""
        return kv_bytes(self.keys_held(c), self.D, torch.finfo(self.dtype).bits // 8)

    def kv_bytes_allocated(self) -> int:
        return sum(kv.bytes_allocated() for kv in self.kv)
