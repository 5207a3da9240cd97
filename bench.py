#!/usr/bin/env python3
"""Throughput of the ISPA hot path on one MI355X.

One step is one full cycle of the Wan-1.3B-shaped single-layer workload
(12 heads x 128 = 1536 wide, 4680 queries per chunk, a 4680-key sink, a
28080-key history, fresh current chunk each step):

  8 warmup chunk steps, each ispa_dual_attn_merge (dual-stream attention and
    the LSE merge into A_loc, A_full - A_loc), and after every fourth chunk
    ispa_accum_gram (one rank-k update of [A_loc | A_full - A_loc] over the
    four chunks' rows into the layer's statistics state)
  the switch: ispa_gram_finalize (G, C = M W, r2) -> ispa_solve_dw (dW, eps,
    W + dW) -> ispa_select_layers (K = 1 of 1)
  one post-switch chunk of the (local) layer: ispa_local_attn_proj with W + dW

All inputs are generated on the GPU before the timed region.  Prints one JSON
line; the headline value is dual-stream attention + LSE merge TFLOP/s (QK^T
and PV flops, 4 n_q n_k D per chunk, over the time of the fused call), with
Gram-statistics TFLOP/s and ms per warmup chunk beside it.  The same chunks
through the two separate calls (ispa_dual_attn, then ispa_lse_merge), and
through ispa_accum_stats (G, C and r2 every chunk), are timed after the timed
steps and reported beside it.  The roofline entry is the fused call's single
kernel (attention of both groups and the merge in one pass per query tile and
head), priced against the bf16 MFMA peak, with its HBM bytes from the counter
summary in profiles/ when that was taken on the current attention source.

Other workloads (``--workload``), each one pass of a chunked stream through
IspaStream, timed per chunk with HIP events around the ISPA calls of all
layers (the chunk's Q, K, V are generated on the GPU before its events):

  wan13b_stream  30 layers x 12 heads x 128, 20 chunks of 4680 tokens:
                 warmup chunks 0-5, switch (K = 15), post-switch chunks 6-19
  wan14b_warmup  40 layers x 40 heads x 128, warmup chunks 0-18 (history up
                 to 79560 keys), switch with 40 ridge solves at D = 5120, K = 20
  wan14b_post    40 post-switch chunks of the same 40 layers (20 L-Layers on
                 sink + current, 20 F-Layers on up to 187200 keys), with the
                 selection and W + dW of an untimed wan14b_warmup pass
  wan14b_post_fp8  wan14b_post_w8a8 with the attention quantised too: the
                 L-Layers' sinks to the fp8 cache once at the switch, every
                 later chunk quantised in the post-switch call that first
                 reads it, attention on the fp8 matrix core for all layers
  wan14b_post_w8a8  wan14b_post with the W8A8 projections: W and W + dW
                 quantised once (untimed, at the switch) to FP8 E4M3, the
                 attention output per token, the products on the fp8 matrix core
  wan13b_recal   the wan13b_stream layers with warmup re-entered: warmup 0-5,
                 switch, post-switch 6-11, warmup again at 12-17 (statistics
                 from zero, every layer over the keys it still holds), switch,
                 post-switch 18-23
  wan13b_video   a 30-second video of the wan13b_stream layers: 40 chunks
                 (120 latent frames), warmup chunks 0-3 (12 latent frames),
                 switch (K = 15), post-switch chunks 4-39
  wan13b_video_vanilla  the same 40 chunks without ISPA: every layer attends
                 to its whole history and projects with W
  wan13b_video_fp8  wan13b_video with the quantised post-switch path: at the
                 switch the projections (W + dW, W) and the L-Layers' sinks are
                 quantised once (timed apart from the switch), then every layer
                 attends on the fp8 matrix core and projects with W8A8

The default run also times wan13b_video, wan13b_video_fp8 and
wan13b_video_vanilla on the same inputs and reports ISPA's speed-up over
vanilla (``--no-video`` skips them).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))

STATS_CHUNKS = 4  # warmup chunks per statistics update (their rows in one rank-k update)
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBS = 8000.0
PEAK_FP64_TFLOPS = 78.6


def _fail_multi(n):
    print(json.dumps({"error": f"--gpus {n}: libispa runs on one GPU; "
                      "sharding across GPUs is not implemented"}))
    sys.exit(2)


def _src_hash(name):
    with open(os.path.join(ROOT, "kv_cache_absorption_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic(kernel_file, src):
    """HBM bytes per launch measured with rocprofv3 counters for the current
    source of the kernel, or None if no measurement matches this source."""
    path = os.path.join(ROOT, "profiles", kernel_file)
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if line.startswith("traffic_bytes_per_launch:"):
                rec["bytes"] = float(line.split(":", 1)[1])
            if line.startswith("source_sha256_16:"):
                rec["sha"] = line.split(":", 1)[1].split()[0]
    if rec.get("sha") != _src_hash(src) or "bytes" not in rec:
        return None
    return rec["bytes"]


def _host_info():
    import platform
    import subprocess
    model = platform.processor() or ""
    try:
        for line in subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
    except Exception:  # lscpu missing
        pass
    return {"nproc": os.cpu_count(), "cpu": model, "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}


def cpu_baseline(g, q, kc, vc, budget_s=8.0):
    """The oracle timed on the host cores on bounded samples of the same
    workload, all threads and one thread: dual-stream attention + merge for a
    subset of query rows of one warmup chunk (the headline's unit), the
    grouped statistics for a subset of rows, and one ridge solve at D = 1536."""
    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    import oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits
    cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    k_loc = torch.cat([g.sink_k, kc]).cpu()
    v_loc = torch.cat([g.sink_v, vc]).cpu()
    k_h, v_h = g.hist_k.cpu(), g.hist_v.cpu()
    qh = q.cpu()
    n_k = k_loc.shape[0] + k_h.shape[0]
    D = g.D

    def attention(limit_s):
        rows, t, chunk = 0, 0.0, 64
        while t < limit_s and rows + chunk <= qh.shape[0]:
            t0 = time.perf_counter()
            O.dual_stream_attention(qh[rows:rows + chunk], k_loc, v_loc, k_h, v_h, g.d ** -0.5)
            t += time.perf_counter() - t0
            rows += chunk
        return rows, t

    rng = np.random.default_rng(0)
    a = (0.3 * rng.standard_normal((1024, D))).astype(np.float16)
    dl = (0.1 * rng.standard_normal((1024, D))).astype(np.float16)
    w = (rng.standard_normal((D, D)) / np.sqrt(D)).astype(np.float32)

    def legs():
        rows, ta = attention(budget_s)
        t0 = time.perf_counter()
        G, M, H = O.accumulate_gram(a, dl)
        O.stats_from_gram(G, M, H, w)
        ts = time.perf_counter() - t0
        Gs = G + 1e-3 * np.trace(G) / D * np.eye(D)
        t0 = time.perf_counter()
        O.solve_dw(Gs, M @ w, 0.0)
        tv = time.perf_counter() - t0
        return {"attention": {"TFLOP/s": 4.0 * rows * n_k * D / ta / 1e12, "rows": rows, "s": round(ta, 2)},
                "statistics": {"TFLOP/s": (4.0 * 1024 * D * D) / ts / 1e12, "rows": 1024, "s": round(ts, 2)},
                "solve": {"TFLOP/s": (7.0 / 3.0) * D ** 3 / tv / 1e12, "D": D, "s": round(tv, 2)}}

    all_t = legs()
    with threadpool_limits(limits=1):
        one_t = legs()
    return {"value": all_t["attention"]["TFLOP/s"], "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"fp64 numpy oracle on host cores: dual-stream attention + LSE merge of "
                      f"{all_t['attention']['rows']} of 4680 query rows (12 heads, {n_k} keys) of one warmup chunk "
                      f"(value, all threads); legs below: the grouped statistics of 1024 rows at D = {D} and one "
                      f"ridge solve at D = {D} (hand-written Cholesky), all threads and one thread",
            "legs_all_threads": all_t, "legs_one_thread": one_t, "host": _host_info()}


STREAMS = {
    # name: layers, heads, head_dim, chunks in the pass, warmup chunks, K, workload id
    "wan13b_stream": dict(N=30, H=12, d=128, chunks=20, warm=6, K=15, wid=3),
    "wan14b_warmup": dict(N=40, H=40, d=128, chunks=19, warm=19, K=20, wid=4),
    "wan14b_post": dict(N=40, H=40, d=128, chunks=40, warm=0, K=20, wid=5),
    "wan14b_post_w8a8": dict(N=40, H=40, d=128, chunks=40, warm=0, K=20, wid=5, w8a8=True),
    "wan14b_post_fp8": dict(N=40, H=40, d=128, chunks=40, warm=0, K=20, wid=5, w8a8=True, fp8attn=True),
    # re-calibration: warmup 0-5, switch, post 6-11, warmup re-entered at 12
    # (12-17), switch again, post 18-23
    "wan13b_recal": dict(N=30, H=12, d=128, chunks=24, warm=6, K=15, wid=3, recal=12, warm2=6),
    # budget / warmup sweep: one 8-chunk (24-frame) warmup, evaluated after
    # 2, 4, 6 and 8 chunks (6-24 frames) for x = 0.3, 0.4, 0.5, 0.7
    "wan13b_sweep": dict(N=30, H=12, d=128, chunks=8, warm=8, K=15, wid=3,
                         evaluate_at=(2, 4, 6, 8), xs=(0.3, 0.4, 0.5, 0.7)),
    # a 30-second video (40 chunks of 3 latent frames) with the default warmup
    # of 12 latent frames and ISPA-0.5, and the same chunks without ISPA
    "wan13b_video": dict(N=30, H=12, d=128, chunks=40, warm=4, K=15, wid=3),
    "wan13b_video_vanilla": dict(N=30, H=12, d=128, chunks=40, warm=0, K=0, wid=3, vanilla=True),
    "wan13b_video_fp8": dict(N=30, H=12, d=128, chunks=40, warm=4, K=15, wid=3, w8a8=True, fp8attn=True),
}
TOKENS_PER_CHUNK = 4680  # 3 latent frames of 1560 tokens


def _stream_pass(spec, dev, seed, adopt=None, timed=True):
    """One pass of a chunked stream.  Returns per-chunk records and the stream.

    ``adopt`` = (is_local, W, W + dW) starts the stream after a switch made by
    another pass (post-switch-only workload)."""
    import torch
    import synth
    from kv_cache_absorption_amd.stream import IspaStream

    N, H, d, T = spec["N"], spec["H"], spec["d"], TOKENS_PER_CHUNK
    D = H * d
    si = synth.StreamInputs(N, H, d, T, torch.bfloat16, seed, dev, workload=spec["wid"])
    if adopt is None:
        st = IspaStream(N, H, d, T, spec["chunks"], dev)
        for layer in range(N):
            st.set_w(layer, si.w(layer))
        st.reserve_switch()  # switch buffers allocated before any timed region
    else:
        is_local, W, w_eff = adopt
        caps = [2 if f else spec["chunks"] for f in is_local]
        st = IspaStream(N, H, d, T, caps, dev, with_stats=False)
        st.W = W
        st.adopt_switch(is_local, w_eff)
        if spec.get("w8a8"):
            st.quantize_projections()  # once per switch, before the timed chunks
        if spec.get("fp8attn"):
            # the L-Layers' sinks to the fp8 cache (once per switch); each later
            # chunk (an L-Layer's current chunk, every chunk of an F-Layer) is
            # quantised inside the timed post() call that first reads it
            for layer, flag in enumerate(is_local):
                if flag:
                    k, v = si.kv(layer, 0)
                    st.write_kv(layer, 0, k, v)
            st.quantize_attention()
    stream = torch.cuda.current_stream(dev)
    qbuf = torch.empty((N, T, H, d), dtype=torch.bfloat16, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    recs = []
    switch_ev = []
    quant_ev = []
    selections = []
    evaluations = []
    recal, warm2 = spec.get("recal"), spec.get("warm2", 0)

    def switch_now(evict=True):
        # solve + select only; the L-Layers' eviction (host bookkeeping, frees
        # and copies of the sink rows) runs after the second event
        s0, s1 = ev(), ev()
        s0.record(stream)
        st.switch(spec["K"], evict=False)
        s1.record(stream)
        switch_ev.append((s0, s1))
        if evict:
            st.evict()
        selections.append([i for i, f in enumerate(st.is_local_host) if f])
        if spec.get("w8a8"):
            # the quantised post-switch path: the projections (and with fp8
            # attention the L-Layers' sinks) quantised once per switch, timed
            # apart from the solve and selection
            q0, q1 = ev(), ev()
            q0.record(stream)
            st.quantize_projections()
            if spec.get("fp8attn"):
                st.quantize_attention()
            q1.record(stream)
            quant_ev.append((q0, q1))

    for c in range(spec["chunks"]):
        if adopt is None and (c == spec["warm"] or (recal is not None and c == recal + warm2)):
            switch_now()
        if recal is not None and c == recal:
            st.recalibrate(c)
            st.reserve_switch()
        for layer in range(N):
            k, v = si.kv(layer, c)
            st.write_kv(layer, c, k, v)
            qbuf[layer].copy_(si.q(layer, c))
            del k, v
        warm = c < spec["warm"] or (recal is not None and recal <= c < recal + warm2)
        marks = []
        e_start = ev()
        e_start.record(stream)
        for layer in range(N):
            if warm:
                st.warmup(layer, c, qbuf[layer])
            else:
                st.post(layer, c, qbuf[layer])
            e = ev()
            e.record(stream)
            marks.append(e)
        last_warm = warm and (c + 1 == spec["warm"] or (recal is not None and c + 1 == recal + warm2))
        if last_warm and adopt is None:
            # the statistics of the chunks still waiting for their update belong
            # to the warmup, not to the switch that follows
            st.flush_statistics()
            e = ev()
            e.record(stream)
            marks.append(e)
        if spec.get("evaluate_at") and c + 1 in spec["evaluate_at"]:
            Ks = [round(x * N) for x in spec["xs"]]
            v0, v1 = ev(), ev()
            v0.record(stream)
            eps_e, sels_e, _, _, _ = st.evaluate(Ks)
            v1.record(stream)
            evaluations.append(dict(chunks=c + 1, eps=eps_e, sels=sels_e, ev=(v0, v1)))
        # keys each layer's call attends to (local + history during warmup)
        n_keys = st.keys_held(c)
        recs.append(dict(c=c, warm=warm, phase=0 if recal is None or c < recal else 1,
                         start=e_start, marks=marks, n_keys=n_keys,
                         kv_held=st.kv_bytes_held(c), kv_alloc=st.kv_bytes_allocated()))
    if spec["warm"] == spec["chunks"] and adopt is None:  # warmup-only pass ends in the switch
        switch_now(evict=False)
    torch.cuda.synchronize()
    for r in recs:
        t, prev = [], r["start"]
        for e in r["marks"]:
            t.append(prev.elapsed_time(e))
            prev = e
        r["layer_ms"] = t
        r["ms"] = sum(t)
        del r["start"], r["marks"]
    switch_ms = [a.elapsed_time(b) for a, b in switch_ev]
    st.quantize_ms = [a.elapsed_time(b) for a, b in quant_ev]
    st.selection_history = selections
    st.evaluations = [dict(chunks=e["chunks"], ms=e["ev"][0].elapsed_time(e["ev"][1]),
                           eps=[float(x) for x in e["eps"].cpu()],
                           sels={K: sorted(v.cpu().tolist()) for K, v in e["sels"].items()})
                      for e in evaluations]
    return recs, (switch_ms[0] if switch_ms else None), st, switch_ms


def _preload_kernels(dev):
    """One tiny untimed call of every entry point a stream uses, so that the
    first timed call of each does not include loading its kernels."""
    import torch
    import kv_cache_absorption_amd as K
    H, d, n = 2, 128, 64
    g = torch.Generator(device="cpu").manual_seed(0)
    r = lambda *sh: torch.randn(*sh, generator=g).to(dev)  # noqa: E731
    q, k, v = (r(n, H, d).to(torch.bfloat16) for _ in range(3))
    w = (r(H * d, H * d) * 0.05).to(torch.bfloat16)
    a_loc, delta, _ = K.ispa_dual_attn_merge(q, [(k, v)], [(k, v)])
    G = torch.zeros((H * d, H * d), dtype=torch.float32, device=dev)
    C = torch.zeros_like(G)
    r2 = torch.zeros(1, dtype=torch.float64, device=dev)
    K.ispa_accum_stats(a_loc, delta, w, G, C, r2)
    state = K.gram_state(H * d, device=dev)
    K.ispa_accum_gram(a_loc, delta, state)
    K.ispa_gram_finalize(state, w)
    G += torch.eye(H * d, device=dev)
    _, eps, _, _ = K.ispa_solve_dw(G, C, r2, 0.0, 1e-3, w=w)
    K.ispa_select_layers(eps, 1)
    K.ispa_local_attn_proj(q, [(k, v)], w)
    c8 = K.ispa_quantize_kv_fp8(k, v)
    qc8, qs8 = K.ispa_quantize_q_fp8(q)
    K.ispa_local_attn_fp8(qc8, qs8, [c8])
    wc, wsc = K.ispa_quantize_w_fp8(w)
    K.ispa_local_attn_fp8_proj(q, [c8], wc, wsc)
    K.ispa_local_attn_proj_fp8(q, [(k, v)], wc, wsc)
    torch.cuda.synchronize()


def _kv_stream_bytes(recs, spec):
    """K and V bytes the pass's attention calls read, each key's K and V row
    once per call (the kernels read them again for every query tile of a head,
    from L2 or HBM: this is the algorithmic KV stream, not counter traffic)."""
    D = spec["H"] * spec["d"]
    elem = 1 if spec.get("fp8attn") else 2  # the fp8 cache holds 1-byte codes
    return sum(2.0 * nk * D * elem for r in recs for nk in r["n_keys"])


def _pass_figures(recs, spec):
    """ms per chunk and TFLOP/s (attention + statistics + projection flops over
    the ISPA time) of one stream pass, and its KV streaming rate."""
    N, H, d, T = spec["N"], spec["H"], spec["d"], TOKENS_PER_CHUNK
    D = H * d
    flops = 0.0
    for r in recs:
        for nk in r["n_keys"]:
            flops += 4.0 * T * nk * D
        flops += N * ((4.0 * T * D * D + 2.0 * T * D) if r["warm"] else 2.0 * T * D * D)
    ms = sum(r["ms"] for r in recs)
    tf = flops / (ms * 1e-3) / 1e12
    kv_gbs = _kv_stream_bytes(recs, spec) / (ms * 1e-3) / 1e9
    out = {"ms/chunk (mean)": round(ms / len(recs), 3), "last chunk ms": round(recs[-1]["ms"], 3),
           "pass TFLOP/s": round(tf, 1),
           "KV streaming GB/s (K, V bytes read once per call / ISPA time)": round(kv_gbs, 1),
           "KV streaming frac of HBM 8 TB/s": round(kv_gbs / PEAK_HBM_GBS, 4)}
    if spec.get("fp8attn"):
        out["pass roofline frac (fp8 5 PFLOP/s)"] = round(tf / PEAK_FP8_TFLOPS, 4)
    else:
        out["pass roofline frac (bf16 2.5 PFLOP/s)"] = round(tf / PEAK_BF16_TFLOPS, 4)
    return out


def wan14b_figures(seed, dev):
    """One Wan-14B warmup pass (40 layers x 40 heads, 19 warmup chunks, switch
    with K = 20) and two 40-chunk post-switch passes with its selection (bf16,
    and quantised: fp8 attention for the L-Layers and W8A8 projections), each
    timed per chunk with HIP events around the ISPA calls."""
    import torch
    _preload_kernels(dev)
    t0 = time.perf_counter()
    recs_w, switch_ms, st4, _ = _stream_pass(STREAMS["wan14b_warmup"], dev, seed)
    out = {"wan14b_warmup": {**_pass_figures(recs_w, STREAMS["wan14b_warmup"]),
                             "switch ms (finalize + 40 solves at D = 5120 + select)": round(switch_ms, 3),
                             "traffic": _traffic("attn_dual_single_pass_wan14b_counters.txt", "attn.hip"),
                             "traffic_kernel": "HBM bytes per launch of the single-pass dual attention at the last "
                                               "warmup chunk (88920 keys), from counters"}}
    adopt = (list(st4.is_local_host), st4.W, st4.w_eff)
    st4.kv = []
    st4.G = st4.C = st4.dW = st4.state = None
    torch.cuda.empty_cache()
    recs_p, _, st5, _ = _stream_pass(STREAMS["wan14b_post"], dev, seed, adopt)
    last = recs_p[-1]
    full = 2 * STREAMS["wan14b_post"]["N"] * (last["c"] + 1) * TOKENS_PER_CHUNK * 5120 * 2
    out["wan14b_post"] = {**_pass_figures(recs_p, STREAMS["wan14b_post"]),
                          "kv_held_fraction_last_chunk": round(last["kv_held"] / full, 4),
                          "traffic": _traffic("attn_fpost_wan14b_traffic.txt", "attn.hip"),
                          "traffic_kernel": "HBM bytes per launch of an F-Layer's attention at the last chunk "
                                            "(187200 keys), from counters"}
    del st5
    torch.cuda.empty_cache()
    recs_8, _, st6, _ = _stream_pass(STREAMS["wan14b_post_fp8"], dev, seed, adopt)
    out["wan14b_post_fp8"] = {**_pass_figures(recs_8, STREAMS["wan14b_post_fp8"]),
                              "note": "every layer: new chunks to the fp8 cache, fp8 attention, W8A8 projection; "
                                      "flops counted as for wan14b_post"}
    out["wan14b wall s (three passes, input generation included)"] = round(time.perf_counter() - t0, 1)
    del st4, st6
    torch.cuda.empty_cache()
    return out


def _vanilla_adopt(spec, dev, seed):
    """Every layer an F-Layer from chunk 0 on, projecting with its own W: the
    stream without ISPA."""
    import torch
    import synth
    N, H, d = spec["N"], spec["H"], spec["d"]
    si = synth.StreamInputs(N, H, d, TOKENS_PER_CHUNK, torch.bfloat16, seed, dev, workload=spec["wid"])
    W = torch.stack([si.w(layer) for layer in range(N)])
    return [0] * N, W, W


def video_figures(seed, dev):
    """The 30-second video three times over the same inputs: ISPA-0.5
    (warmup chunks 0-3 with dual-stream attention and statistics, the switch,
    chunks 4-39 with 15 L-Layers on sink + current chunk and W + dW), the same
    with the quantised post-switch path (fp8 attention, W8A8 projections), and
    vanilla (every layer attends to its whole history and projects with W).
    Each chunk is timed with HIP events around the ISPA-side calls of all
    layers (attention, merge, statistics, projection); the switch and the
    quantisation at the switch are timed apart and counted on ISPA's side."""
    import torch
    _preload_kernels(dev)
    spec, spec_v = STREAMS["wan13b_video"], STREAMS["wan13b_video_vanilla"]
    recs_i, switch_ms, st, _ = _stream_pass(spec, dev, seed)
    W, selected = st.W, [i for i, f in enumerate(st.is_local_host) if f]
    st.kv = []
    st.G = st.C = st.dW = st.state = None
    del st
    torch.cuda.empty_cache()
    recs_q, switch_q, st_q, _ = _stream_pass(STREAMS["wan13b_video_fp8"], dev, seed)
    quant_ms = st_q.quantize_ms[0]
    st_q.kv = []
    st_q.f8 = st_q.sink8 = st_q.wq = None
    del st_q
    torch.cuda.empty_cache()
    recs_v, _, st_v, _ = _stream_pass(spec_v, dev, seed, adopt=([0] * spec_v["N"], W, W))
    st_v.kv = []
    del st_v, W
    torch.cuda.empty_cache()
    warm = spec["warm"]
    tot = lambda rs, lo=0, hi=None: sum(r["ms"] for r in rs[lo:hi])  # noqa: E731
    ispa_ms = tot(recs_i) + switch_ms
    ispa8_ms = tot(recs_q) + switch_q + quant_ms
    van_ms = tot(recs_v)
    return {
        "layers x heads, chunks, warmup chunks, K": f"{spec['N']} x {spec['H']}, {spec['chunks']}, "
                                                    f"{warm} (12 latent frames), {spec['K']}",
        "ISPA ms (warmup chunks + switch + post-switch chunks)": round(ispa_ms, 2),
        "vanilla ms (all chunks)": round(van_ms, 2),
        "speed-up over the video (vanilla / ISPA)": round(van_ms / ispa_ms, 3),
        "speed-up over the post-switch chunks": round(tot(recs_v, warm) / tot(recs_i, warm), 3),
        "speed-up at the last chunk": round(recs_v[-1]["ms"] / recs_i[-1]["ms"], 3),
        "warmup chunks, ISPA ms / vanilla ms (dual-stream attention + statistics against plain attention)":
            round(tot(recs_i, 0, warm) / tot(recs_v, 0, warm), 3),
        "switch ms (finalize + 30 solves + select)": round(switch_ms, 3),
        "KV held at the last chunk, ISPA / vanilla": round(recs_i[-1]["kv_held"] / recs_v[-1]["kv_held"], 4),
        "quantised ISPA ms (fp8 attention and W8A8 projections after the switch)": round(ispa8_ms, 2),
        "quantisation at the switch ms (30 projections, 15 sinks)": round(quant_ms, 3),
        "speed-up over the video, quantised ISPA against vanilla bf16": round(van_ms / ispa8_ms, 3),
        "speed-up over the post-switch chunks, quantised ISPA against vanilla bf16":
            round(tot(recs_v, warm) / tot(recs_q, warm), 3),
        "L-Layers": selected,
        "note": "ISPA-side work only (attention, merge, statistics, output projection); the pages report "
                "1.89x within attention, 1.35x for the whole model and 1.86x for the whole model with W8A8, "
                "on their GPU and backbones (EN review, Key Findings)",
    }


def wan14b_counter_calls(kind, n_calls, seed, dev):
    """The dominant attention call of a Wan-14B pass at its largest key set,
    repeated for counter runs: ``fused`` = the last warmup chunk's
    ispa_dual_attn_merge (40 heads, 9360 local keys, 17 history chunks =
    79560 keys); ``fpost`` = the last post-switch chunk of an F-Layer,
    ispa_local_attn_proj over all 40 chunks (187200 keys) with W.  Prints the
    mean call time by HIP events over the calls (unprofiled runs)."""
    import torch
    import synth
    import kv_cache_absorption_amd as K
    from kv_cache_absorption_amd import _lib as B
    T, H, d = TOKENS_PER_CHUNK, 40, 128
    n_hist = (17 if kind == "fused" else 38) * T
    g = synth.GroupInputs(T, H, d, T, n_hist, torch.bfloat16, seed, dev, workload=4)
    q, kc, vc = g.step(0)
    L = B.lib()
    sh = torch.cuda.current_stream(dev).cuda_stream
    if kind == "fused":
        ls, nl = B._segs([(g.sink_k, g.sink_v), (kc, vc)], H, d)
        hs, nh = B._segs([(g.hist_k, g.hist_v)], H, d)
        need = L.ispa_dual_attn_merge_workspace_bytes(B.ISPA_BF16, T, H, d, ls, nl, hs, nh)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        a_loc = torch.empty((T, H * d), dtype=torch.float16, device=dev)
        delta = torch.empty_like(a_loc)

        def call():
            st = L.ispa_dual_attn_merge(B.ISPA_BF16, T, H, d, d ** -0.5, q.data_ptr(), q.stride(0), ls, nl, hs, nh,
                                        a_loc.data_ptr(), delta.data_ptr(), B.ISPA_F16, None, ws.data_ptr(),
                                        ws.numel(), sh)
            if st:
                raise B.IspaError(st, L.ispa_last_error().decode())
        n_keys = 2 * T + n_hist
    else:
        # one contiguous run of keys, as a stream's layer cache holds them
        segs = [(torch.cat([g.sink_k, g.hist_k, kc]), torch.cat([g.sink_v, g.hist_v, vc]))]
        del g.hist_k, g.hist_v

        def call():
            K.ispa_local_attn_proj(q, segs, g.w)
        n_keys = 2 * T + n_hist
    call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n_calls):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n_calls
    return {"kind": kind, "calls": n_calls, "heads": H, "keys": n_keys, "call_us": round(ms * 1e3, 1),
            "attention TFLOP/s": round(4.0 * T * n_keys * H * d / (ms * 1e-3) / 1e12, 1)}


def run_stream(args, name, dev):
    import torch
    spec = STREAMS[name]
    _preload_kernels(dev)
    N, H, d, T = spec["N"], spec["H"], spec["d"], TOKENS_PER_CHUNK
    D = H * d
    adopt = None
    pre = {}
    if spec.get("vanilla"):
        adopt = _vanilla_adopt(spec, dev, args.seed)
        pre = {"vanilla": "every layer attends to its whole history and projects with W"}
    if name in ("wan14b_post", "wan14b_post_w8a8", "wan14b_post_fp8"):
        t0 = time.perf_counter()
        _, pre_switch_ms, st4, _ = _stream_pass(STREAMS["wan14b_warmup"], dev, args.seed)
        adopt = (list(st4.is_local_host), st4.W, st4.w_eff)
        pre = {"switch_source": "untimed wan14b_warmup pass (same seed)",
               "switch_ms": round(pre_switch_ms, 3), "setup_s": round(time.perf_counter() - t0, 1)}
        st4.kv = []
        st4.G = st4.C = st4.dW = None
        torch.cuda.empty_cache()
    for _ in range(args.warmup):
        _stream_pass(spec, dev, args.seed, adopt)
        torch.cuda.empty_cache()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    passes = []
    for _ in range(args.steps):
        passes.append(_stream_pass(spec, dev, args.seed, adopt))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    recs, switch_ms, st, switches = passes[-1]
    if st.quantize_ms:
        pre["quantisation at the switch ms (projections, L-Layer sinks)"] = [round(x, 3) for x in st.quantize_ms]
    all_recs = [r for p in passes for r in p[0]]
    chunk_ms = [r["ms"] for r in all_recs]
    mean = lambda xs: sum(xs) / len(xs) if xs else None  # noqa: E731
    warm_ms = [r["ms"] for r in all_recs if r["warm"]]
    post_ms = [r["ms"] for r in all_recs if not r["warm"]]
    # attention flops of every call in the pass (QK^T and PV only)
    attn_flops, proj_flops, stats_flops = 0.0, 0.0, 0.0
    for r in recs:
        for nk in r["n_keys"]:
            attn_flops += 4.0 * T * nk * D
        if r["warm"]:
            stats_flops += N * (4.0 * T * D * D + 2.0 * T * D)
        else:
            proj_flops += N * 2.0 * T * D * D
    pass_ms = sum(r["ms"] for r in recs)
    if spec.get("recal") is not None:
        for ph, tag in ((0, "before"), (1, "after")):
            w = [r["ms"] for r in all_recs if r["phase"] == ph and r["warm"]]
            p_ = [r["ms"] for r in all_recs if r["phase"] == ph and not r["warm"]]
            pre[f"warmup ms/chunk {tag} re-entry"] = round(mean(w), 3) if w else None
            pre[f"post-switch ms/chunk {tag} re-entry"] = round(mean(p_), 3) if p_ else None
        pre["warmup re-entered at chunk"] = spec["recal"]
        pre["switch ms (each switch)"] = [round(x, 3) for x in switches]
        pre["L-Layers (each switch)"] = st.selection_history
    if spec.get("evaluate_at"):
        r20 = 2 / 20  # local share of the keys at chunk 19 of a 20-chunk stream
        sweep = []
        for e in st.evaluations:
            eps_sorted = sorted(e["eps"])
            for x, K in zip(spec["xs"], sorted(e["sels"])):
                sweep.append({"warmup_frames": 3 * e["chunks"], "x": x, "K": K,
                              "L-Layers": e["sels"][K],
                              "eps_sum_selected": sum(eps_sorted[:K]),
                              "kv_fraction_at_chunk_19": round(1 - x * (1 - r20), 4)})
        pre["sweep"] = sweep
        pre["evaluate ms (solve all layers + 4 selections)"] = [round(e["ms"], 3) for e in st.evaluations]
        pre["selection overlap (x=0.5) with the 24-frame selection"] = [
            len(set(e["sels"][15]) & set(st.evaluations[-1]["sels"][15])) for e in st.evaluations]
    last = recs[-1]
    c_last = last["c"]
    full_bytes = 2 * N * (c_last + 1) * T * D * 2
    value = mean(chunk_ms)
    achieved = (attn_flops + proj_flops + stats_flops) / (pass_ms * 1e-3) / 1e12
    peak = PEAK_FP8_TFLOPS if spec.get("fp8attn") else PEAK_BF16_TFLOPS
    out = {
        "metric": "ms/chunk (1 GPU)",
        "value": round(value, 3),
        "unit": "ms/chunk",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "layers": N, "heads": H, "head_dim": d, "tokens_per_chunk": T,
                   "chunks": spec["chunks"], "warmup_chunks": spec["warm"], "K": spec["K"],
                   "stats_operands": "fp16" if spec["warm"] else None,
                   "statistics": "grouped (accum_gram)" if spec["warm"] else "none (no warmup chunk in the pass)",
                   "seed": args.seed,
                   "timing": "HIP events around each chunk's ISPA calls of all layers; the chunk's "
                             "synthetic Q/K/V generation sits outside them (ms_per_step is the wall "
                             "time of the whole pass including that generation)"},
        "also": {
            "warmup ms/chunk (mean)": round(mean(warm_ms), 3) if warm_ms else None,
            "post-switch ms/chunk (mean)": round(mean(post_ms), 3) if post_ms else None,
            "last chunk ms": round(last["ms"], 3),
            "switch ms (solve all layers + select)": round(switch_ms, 3) if switch_ms else None,
            "pass TFLOP/s (attention + statistics + projection flops / ISPA time)": round(achieved, 2),
            "KV streaming GB/s (K, V bytes read once per call / ISPA time)":
                round(_kv_stream_bytes(recs, spec) / (pass_ms * 1e-3) / 1e9, 1),
            "kv_bytes_held_last_chunk": last["kv_held"],
            "kv_bytes_all_full_last_chunk": full_bytes,
            "kv_held_fraction": round(last["kv_held"] / full_bytes, 4),
            "kv_bytes_allocated_last_chunk": last["kv_alloc"],
            "L-Layers": [i for i, f in enumerate(st.is_local_host or []) if f],
            **pre,
        },
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None,
                     "kernel": "all ISPA calls of the pass (attention dominates)"
                               + ("; priced against the fp8 peak: the attention and the projections run on the "
                                  "fp8 matrix core" if spec.get("fp8attn") else "")},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def ceilings(n_calls, dev):
    """What the machine reaches on plain library work, beside the published
    peaks the rooflines divide by: large GEMMs through torch (hipBLASLt /
    rocBLAS) in bf16, fp64 and, where torch offers it, fp8 E4M3 with unit
    scales; and a 4 GiB device-to-device copy (bytes read + bytes written per
    second).  Mean over n_calls after one untimed call, HIP events on the
    current stream.  Operands are contiguous 2-D tensors."""
    import torch
    out = {"calls": n_calls}
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(n_calls):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n_calls * 1e-3

    g = torch.Generator(device=dev).manual_seed(5)
    for name, dt, n, peak in (("bf16 GEMM 8192^3", torch.bfloat16, 8192, PEAK_BF16_TFLOPS),
                              ("fp64 GEMM 4096^3", torch.float64, 4096, PEAK_FP64_TFLOPS)):
        x = torch.randn((n, n), device=dev, generator=g).to(dt)
        y = torch.randn((n, n), device=dev, generator=g).to(dt)
        t = timed(lambda: torch.matmul(x, y))
        tf = 2.0 * n ** 3 / t / 1e12
        out[name] = {"TFLOP/s": round(tf, 1), "frac of published peak": round(tf / peak, 4)}
        del x, y
    try:  # fp8 through torch's scaled matmul (second operand column-major, as it requires)
        n = 8192
        x = torch.randn((n, n), device=dev, generator=g).to(torch.float8_e4m3fn)
        y = torch.randn((n, n), device=dev, generator=g).to(torch.float8_e4m3fn).t().contiguous().t()
        one = torch.ones((), device=dev)
        t = timed(lambda: torch._scaled_mm(x, y, scale_a=one, scale_b=one, out_dtype=torch.bfloat16))
        tf = 2.0 * n ** 3 / t / 1e12
        out["fp8 GEMM 8192^3 (torch._scaled_mm)"] = {"TFLOP/s": round(tf, 1),
                                                    "frac of published peak": round(tf / PEAK_FP8_TFLOPS, 4)}
        del x, y
    except (RuntimeError, AttributeError, TypeError) as e:  # reported, never replaced
        out["fp8 GEMM 8192^3 (torch._scaled_mm)"] = {"unavailable": str(e).splitlines()[0][:200]}
    src = torch.empty(1 << 30, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    t = timed(lambda: dst.copy_(src))
    gbs = 2.0 * src.numel() * 4 / t / 1e9
    out["device copy 4 GiB (read + write)"] = {"GB/s": round(gbs, 1), "frac of published peak": round(gbs / PEAK_HBM_GBS, 4)}
    return out


def sdpa_compare(n_calls, seed, dev):
    """The benchmark chunk's attention through torch's fused scaled-dot-product
    attention (the vendor path: flash, else memory-efficient backend; the math
    backend is never used) beside ispa_dual_attn_merge on the same inputs: one
    key set of sink + current + history (37440 keys) against our two groups
    and their merge.  Same flops (4 n_q n_k D); mean ms per call with HIP
    events on the current stream, after one untimed call of each."""
    import torch
    import torch.nn.functional as F
    import synth
    from kv_cache_absorption_amd import _lib as B
    L = B.lib()
    g = synth.wan13b_single_layer(seed=seed, device=dev)
    n_q, H, d, D = g.n_q, g.H, g.d, g.D
    q, kc, vc = g.step(0)
    k_all = torch.cat([g.sink_k, kc, g.hist_k])
    v_all = torch.cat([g.sink_v, vc, g.hist_v])
    n_k = k_all.shape[0]
    flops = 4.0 * n_q * n_k * D
    qh = q.permute(1, 0, 2).unsqueeze(0).contiguous()
    kh = k_all.permute(1, 0, 2).unsqueeze(0).contiguous()
    vh = v_all.permute(1, 0, 2).unsqueeze(0).contiguous()
    out = {"calls": n_calls, "n_q": n_q, "n_k": n_k, "heads": H, "head_dim": d, "flops_per_call": flops}
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(n_calls):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / n_calls
        return {"ms": round(ms, 4), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1)}

    from torch.nn.attention import SDPBackend, sdpa_kernel
    for name, be in (("flash", SDPBackend.FLASH_ATTENTION), ("efficient", SDPBackend.EFFICIENT_ATTENTION)):
        try:
            with sdpa_kernel([be]):
                out["torch_sdpa_" + name] = timed(lambda: F.scaled_dot_product_attention(qh, kh, vh,
                                                                                         scale=d ** -0.5))
        except RuntimeError as e:  # backend not available for these inputs: reported, never replaced
            out["torch_sdpa_" + name] = {"unavailable": str(e).splitlines()[0][:200]}
    a_loc = torch.empty((n_q, D), dtype=torch.float16, device=dev)
    delta = torch.empty_like(a_loc)
    ls, nl = B._segs([(g.sink_k, g.sink_v), (kc, vc)], H, d)
    hs, nh = B._segs([(g.hist_k, g.hist_v)], H, d)
    wsb = L.ispa_dual_attn_merge_workspace_bytes(B.ISPA_BF16, n_q, H, d, ls, nl, hs, nh)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    sh = torch.cuda.current_stream(dev).cuda_stream

    def ours():
        st = L.ispa_dual_attn_merge(B.ISPA_BF16, n_q, H, d, d ** -0.5, q.data_ptr(), q.stride(0), ls, nl, hs, nh,
                                    a_loc.data_ptr(), delta.data_ptr(), B.ISPA_F16, None, ws.data_ptr(),
                                    ws.numel(), sh)
        if st:
            raise B.IspaError(st, L.ispa_last_error().decode())
    out["ispa_dual_attn_merge"] = timed(ours)
    return out


def proj_compare(n_calls, dev):
    """Post-switch attention + projection of one chunk (4680 queries over the
    sink and current chunk, 9360 keys) with the bf16 projection and with the
    W8A8 one, and the W8A8 product alone on fp32 activations, at D = 1536
    (12 heads) and D = 5120 (40 heads).  Mean ms per call with HIP events on
    the current stream."""
    import torch
    import synth
    import kv_cache_absorption_amd as K
    out = {"calls": n_calls}
    for H in (12, 40):
        D = H * 128
        g = synth.GroupInputs(TOKENS_PER_CHUNK, H, 128, TOKENS_PER_CHUNK, 0, torch.bfloat16, 1, dev, workload=2)
        q, kc, vc = g.step(0)
        w = synth.normal((D, D), 5, dev, std=D ** -0.5, dtype=torch.bfloat16)
        segs = [(g.sink_k, g.sink_v), (kc, vc)]
        codes, scales = K.ispa_quantize_w_fp8(w)
        x = synth.normal((TOKENS_PER_CHUNK, D), 6, dev, dtype=torch.float32)
        for name, f in (("bf16 attention + projection", lambda: K.ispa_local_attn_proj(q, segs, w)),
                        ("attention + W8A8 projection", lambda: K.ispa_local_attn_proj_fp8(q, segs, codes, scales)),
                        ("W8A8 product", lambda: K.ispa_w8a8_linear(x, codes, scales)),
                        ("weight quantisation", lambda: K.ispa_quantize_w_fp8(w))):
            for _ in range(2):
                f()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(n_calls):
                f()
            e1.record()
            torch.cuda.synchronize()
            out[f"D={D} {name} ms"] = round(e0.elapsed_time(e1) / n_calls, 4)
        del g, q, kc, vc, w, codes, scales, x
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="default 3 (1 for stream workloads)")
    ap.add_argument("--warmup", type=int, default=None, help="default 1 (0 for stream workloads)")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--workload", default="wan13b_layer", choices=["wan13b_layer"] + sorted(STREAMS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-14b", action="store_true", help="skip the Wan-14B stream passes of the default run")
    ap.add_argument("--no-video", action="store_true",
                    help="skip the ISPA-against-vanilla video passes of the default run")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes (counter calibration)")
    ap.add_argument("--attn-only", type=int, default=0,
                    help="only run this many dual-attention calls of the workload (counter runs)")
    ap.add_argument("--fused-only", type=int, default=0,
                    help="only run this many fused dual-attention + merge calls of the workload (counter runs)")
    ap.add_argument("--gram-only", type=int, default=0,
                    help="only run this many statistics updates (ispa_accum_gram) of the workload (counter runs)")
    ap.add_argument("--attn8-only", type=int, default=0,
                    help="only run this many fp8 local-attention calls (post-switch L-Layer) of the workload "
                         "(counter runs)")
    ap.add_argument("--w14-fused-only", type=int, default=0,
                    help="only run this many Wan-14B last-warmup-chunk dual-attention calls (counter runs)")
    ap.add_argument("--w14-fpost-only", type=int, default=0,
                    help="only run this many Wan-14B last-chunk F-Layer attention + projection calls (counter runs)")
    ap.add_argument("--merge-only", type=int, default=0,
                    help="only run this many two-part LSE merges of the workload (counter runs)")
    ap.add_argument("--ceilings", type=int, default=0,
                    help="only time large library GEMMs (bf16, fp64, fp8) and a 4 GiB device copy, this many calls "
                         "each: what the machine reaches on plain library work")
    ap.add_argument("--sdpa-compare", type=int, default=0,
                    help="only time torch's fused attention (flash / memory-efficient backend) and "
                         "ispa_dual_attn_merge on the benchmark chunk, this many calls each")
    ap.add_argument("--proj-compare", type=int, default=0,
                    help="only time the post-switch projection paths (bf16 and W8A8) at the Wan-1.3B "
                         "and Wan-14B widths, this many calls each")
    args = ap.parse_args()
    is_stream = args.workload != "wan13b_layer"
    if args.steps is None:
        args.steps = 1 if is_stream else 3
    if args.warmup is None:
        args.warmup = 0 if is_stream else 1
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        _fail_multi(max(args.gpus, world))

    import torch
    sys.path.insert(0, ROOT)
    import kv_cache_absorption_amd as K
    from kv_cache_absorption_amd import _lib as B
    import synth

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_bytes:
        src = torch.ones(args.copy_bytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes}))
        return
    L = B.lib()  # raises if libispa.so is missing: no fallback path exists
    if args.w14_fused_only or args.w14_fpost_only:
        kind = "fused" if args.w14_fused_only else "fpost"
        print(json.dumps(wan14b_counter_calls(kind, args.w14_fused_only or args.w14_fpost_only, args.seed, dev)))
        return
    if args.proj_compare:
        print(json.dumps(proj_compare(args.proj_compare, dev)))
        return
    if args.sdpa_compare:
        print(json.dumps(sdpa_compare(args.sdpa_compare, args.seed, dev)))
        return
    if args.ceilings:
        print(json.dumps(ceilings(args.ceilings, dev)))
        return
    if args.workload != "wan13b_layer":
        run_stream(args, args.workload, dev)
        return

    # ---------------- inputs (resident in HBM before timing)
    g = synth.wan13b_single_layer(seed=args.seed, device=dev)
    n_q, H, d, D = g.n_q, g.H, g.d, g.D
    n_warm = 8
    steps_in = [g.step(i) for i in range(n_warm)]
    q_post, k_post, v_post = g.step(n_warm)
    scale = d ** -0.5
    n_loc, n_hist = 2 * n_q, g.hist_k.shape[0]
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    # ---------------- preallocated outputs, state and workspaces
    f32 = dict(dtype=torch.float32, device=dev)
    o_loc = torch.empty((n_q, H, d), **f32)
    o_hist = torch.empty_like(o_loc)
    lse_loc = torch.empty((n_q, H), **f32)
    lse_hist = torch.empty_like(lse_loc)
    # A_loc and dA rows of STATS_CHUNKS chunks: one statistics update for them
    a_loc = torch.empty((STATS_CHUNKS * n_q, D), dtype=torch.float16, device=dev)
    delta = torch.empty_like(a_loc)
    G = torch.zeros((D, D), **f32)
    C = torch.zeros((D, D), **f32)
    r2 = torch.zeros(1, dtype=torch.float64, device=dev)
    state = K.gram_state(D, device=dev)
    dW = torch.empty((D, D), **f32)
    eps = torch.empty(1, dtype=torch.float64, device=dev)
    info = torch.empty(1, dtype=torch.int32, device=dev)
    w_eff = torch.empty_like(g.w)
    sel = torch.empty(1, dtype=torch.int32, device=dev)
    is_local = torch.empty(1, dtype=torch.uint8, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    y_post = torch.empty((n_q, D), dtype=torch.bfloat16, device=dev)

    def segs(pairs):
        return B._segs(pairs, H, d)

    seg_tables = []
    for (q, kc, vc) in steps_in:
        ls, nl = segs([(g.sink_k, g.sink_v), (kc, vc)])
        hs, nh = segs([(g.hist_k, g.hist_v)])
        seg_tables.append((q, ls, nl, hs, nh))
    ws_attn_b = max(L.ispa_dual_attn_workspace_bytes(B.ISPA_BF16, n_q, H, d, seg_tables[0][1], 2,
                                                     seg_tables[0][3], 1),
                    L.ispa_dual_attn_merge_workspace_bytes(B.ISPA_BF16, n_q, H, d, seg_tables[0][1], 2,
                                                           seg_tables[0][3], 1))
    ws_stats_b = max(L.ispa_accum_stats_workspace_bytes(B.ISPA_F16, n_q, D), L.ispa_gram_finalize_workspace_bytes(D))
    ws_solve_b = L.ispa_solve_dw_workspace_bytes(1, D)
    post_segs, post_n = segs([(g.sink_k, g.sink_v), (k_post, v_post)])
    ws_post_b = L.ispa_local_attn_proj_workspace_bytes(B.ISPA_BF16, n_q, H, d, post_segs, post_n)
    ws = torch.empty(max(ws_attn_b, ws_stats_b, ws_solve_b, ws_post_b, 256), dtype=torch.uint8, device=dev)
    wsp, wsn = ws.data_ptr(), ws.numel()
    if args.fused_only or args.gram_only or args.merge_only:
        q, ls, nl, hs, nh = seg_tables[0]
        fo = (ctypes.c_void_p * 2)(o_loc.data_ptr(), o_hist.data_ptr())
        fl = (ctypes.c_void_p * 2)(lse_loc.data_ptr(), lse_hist.data_ptr())
        if args.gram_only or args.merge_only:  # inputs of one chunk
            L.ispa_dual_attn(B.ISPA_BF16, n_q, H, d, scale, q.data_ptr(), q.stride(0), ls, nl, hs, nh,
                             o_loc.data_ptr(), lse_loc.data_ptr(), o_hist.data_ptr(), lse_hist.data_ptr(), wsp, wsn, sh)
            L.ispa_lse_merge(2, fo, fl, n_q, H, d, None, None, a_loc.data_ptr(), delta.data_ptr(), B.ISPA_F16, sh)
        for _ in range(args.fused_only):
            st = L.ispa_dual_attn_merge(B.ISPA_BF16, n_q, H, d, scale, q.data_ptr(), q.stride(0), ls, nl, hs, nh,
                                        a_loc.data_ptr(), delta.data_ptr(), B.ISPA_F16, None, wsp, wsn, sh)
            if st:
                raise B.IspaError(st, L.ispa_last_error().decode())
        if args.gram_only:  # the benchmark's call: the rows of STATS_CHUNKS chunks (this chunk repeated)
            for c in range(1, STATS_CHUNKS):
                a_loc[c * n_q:(c + 1) * n_q].copy_(a_loc[:n_q])
                delta[c * n_q:(c + 1) * n_q].copy_(delta[:n_q])
        for _ in range(args.gram_only):
            st = L.ispa_accum_gram(B.ISPA_F16, STATS_CHUNKS * n_q, D, a_loc.data_ptr(), delta.data_ptr(),
                                   state.data_ptr(), sh)
            if st:
                raise B.IspaError(st, L.ispa_last_error().decode())
        for _ in range(args.merge_only):
            st = L.ispa_lse_merge(2, fo, fl, n_q, H, d, None, None, a_loc.data_ptr(), delta.data_ptr(),
                                  B.ISPA_F16, sh)
            if st:
                raise B.IspaError(st, L.ispa_last_error().decode())
        torch.cuda.synchronize()
        print(json.dumps({"fused_only_calls": args.fused_only, "gram_only_calls": args.gram_only,
                          "merge_only_calls": args.merge_only}))
        return
    if args.attn8_only:
        sink8 = K.ispa_quantize_kv_fp8(g.sink_k, g.sink_v)
        cur8 = K.ispa_quantize_kv_fp8(k_post, v_post)
        qc8, qs8 = K.ispa_quantize_q_fp8(q_post)
        o8 = torch.empty((n_q, H, d), dtype=torch.float32, device=dev)
        segs8, ns8 = B._segs_fp8([sink8, cur8])
        for _ in range(args.attn8_only):
            st = L.ispa_local_attn_fp8(n_q, H, d, scale, qc8.data_ptr(), qs8.data_ptr(), segs8, ns8, o8.data_ptr(),
                                       B.ISPA_F32, None, sh)
            if st:
                raise B.IspaError(st, L.ispa_last_error().decode())
        torch.cuda.synchronize()
        print(json.dumps({"attn8_only_calls": args.attn8_only}))
        return
    if args.attn_only:
        q, ls, nl, hs, nh = seg_tables[0]
        for _ in range(args.attn_only):
            st = L.ispa_dual_attn(B.ISPA_BF16, n_q, H, d, scale, q.data_ptr(), q.stride(0), ls, nl, hs, nh,
                                  o_loc.data_ptr(), lse_loc.data_ptr(), o_hist.data_ptr(), lse_hist.data_ptr(),
                                  wsp, wsn, sh)
            if st:
                raise B.IspaError(st, L.ispa_last_error().decode())
        torch.cuda.synchronize()
        print(json.dumps({"attn_only_calls": args.attn_only}))
        return
    op = (ctypes.c_void_p * 2)(o_loc.data_ptr(), o_hist.data_ptr())
    lp = (ctypes.c_void_p * 2)(lse_loc.data_ptr(), lse_hist.data_ptr())

    def ck(st):
        if st != 0:
            raise B.IspaError(st, L.ispa_last_error().decode())

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    rec = {"fused": [], "attn": [], "merge": [], "stats": [], "stats_direct": [], "switch": [], "post": []}

    def cycle(timed):
        state.zero_()
        marks = []
        for i, (q, ls, nl, hs, nh) in enumerate(seg_tables):
            e0, e1, e2 = ev(), ev(), ev()
            off = (i % STATS_CHUNKS) * n_q * D * 2  # this chunk's rows in the update buffers
            last = i % STATS_CHUNKS == STATS_CHUNKS - 1
            e0.record(stream)
            ck(L.ispa_dual_attn_merge(B.ISPA_BF16, n_q, H, d, scale, q.data_ptr(), q.stride(0), ls, nl, hs,
                                      nh, a_loc.data_ptr() + off, delta.data_ptr() + off, B.ISPA_F16, None,
                                      wsp, wsn, sh))
            e1.record(stream)
            if last:
                ck(L.ispa_accum_gram(B.ISPA_F16, STATS_CHUNKS * n_q, D, a_loc.data_ptr(), delta.data_ptr(),
                                     state.data_ptr(), sh))
            e2.record(stream)
            marks.append((e0, e1, e2, last))
        s0, s1, s2 = ev(), ev(), ev()
        s0.record(stream)
        ck(L.ispa_gram_finalize(1, D, state.data_ptr(), state.numel(), g.w.data_ptr(), B.ISPA_BF16, D * D,
                                G.data_ptr(), C.data_ptr(), r2.data_ptr(), D * D, wsp, wsn, sh))
        ck(L.ispa_solve_dw(1, D, G.data_ptr(), C.data_ptr(), r2.data_ptr(), D * D, 0.0, 1e-3, dW.data_ptr(),
                           eps.data_ptr(), info.data_ptr(), g.w.data_ptr(), B.ISPA_BF16, w_eff.data_ptr(),
                           wsp, wsn, sh))
        ck(L.ispa_select_layers(1, 1, eps.data_ptr(), sel.data_ptr(), is_local.data_ptr(), status.data_ptr(), sh))
        s1.record(stream)
        ck(L.ispa_local_attn_proj(B.ISPA_BF16, n_q, H, d, scale, q_post.data_ptr(), q_post.stride(0), post_segs,
                                  post_n, w_eff.data_ptr(), B.ISPA_BF16, y_post.data_ptr(), B.ISPA_BF16, wsp,
                                  wsn, sh))
        s2.record(stream)
        if timed:
            rec["_pending"] = rec.get("_pending", []) + [(marks, (s0, s1, s2))]

    for _ in range(args.warmup):
        cycle(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        cycle(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the same warmup chunks through the two separate calls, and the statistics
    # through ispa_accum_stats (after the timed steps)
    two_call = []
    G2 = torch.zeros((D, D), **f32)
    C2 = torch.zeros((D, D), **f32)
    r22 = torch.zeros(1, dtype=torch.float64, device=dev)
    for (q, ls, nl, hs, nh) in seg_tables:
        e0, e1, e2, e3 = ev(), ev(), ev(), ev()
        e0.record(stream)
        ck(L.ispa_dual_attn(B.ISPA_BF16, n_q, H, d, scale, q.data_ptr(), q.stride(0), ls, nl, hs, nh,
                            o_loc.data_ptr(), lse_loc.data_ptr(), o_hist.data_ptr(), lse_hist.data_ptr(),
                            wsp, wsn, sh))
        e1.record(stream)
        ck(L.ispa_lse_merge(2, op, lp, n_q, H, d, None, None, a_loc.data_ptr(), delta.data_ptr(),
                            B.ISPA_F16, sh))
        e2.record(stream)
        ck(L.ispa_accum_stats(B.ISPA_F16, B.ISPA_BF16, n_q, D, a_loc.data_ptr(), delta.data_ptr(),
                              g.w.data_ptr(), G2.data_ptr(), C2.data_ptr(), r22.data_ptr(), wsp, wsn, sh))
        e3.record(stream)
        two_call.append((e0, e1, e2, e3))
    # the post-switch chunk with the L-Layer's attention quantised: the sink in
    # the fp8 cache and W + dW's codes once per switch (untimed), then per call
    # the current chunk's quantisation and ispa_local_attn_fp8_proj; and the
    # fp8 attention kernel alone on quantised queries
    wq, wqs = K.ispa_quantize_w_fp8(w_eff)
    sink8 = K.ispa_quantize_kv_fp8(g.sink_k, g.sink_v)
    cur8 = K.ispa_quantize_kv_fp8(k_post, v_post)
    qc8, qs8 = K.ispa_quantize_q_fp8(q_post)
    o8 = torch.empty((n_q, H, d), **f32)
    segs8, ns8 = B._segs_fp8([sink8, cur8])
    ws8_b = max(L.ispa_local_attn_fp8_proj_workspace_bytes(n_q, H, d), L.ispa_quantize_kv_fp8_workspace_bytes(n_q, H, d))
    ws8 = torch.empty(ws8_b, dtype=torch.uint8, device=dev)
    kv8_b = L.ispa_quantize_kv_fp8_workspace_bytes(n_q, H, d)
    fp8_marks = []
    for _ in range(args.steps):
        e0, e1, e2, e3 = ev(), ev(), ev(), ev()
        e0.record(stream)
        ck(L.ispa_quantize_kv_fp8(B.ISPA_BF16, n_q, H, d, k_post.data_ptr(), k_post.stride(0), v_post.data_ptr(),
                                  v_post.stride(0), cur8.k_codes.data_ptr(), cur8.v_codes.data_ptr(),
                                  cur8.k_scales.data_ptr(), cur8.v_scales.data_ptr(), ws8.data_ptr(), kv8_b, sh))
        ck(L.ispa_local_attn_fp8_proj(n_q, H, d, scale, B.ISPA_BF16, q_post.data_ptr(), q_post.stride(0), segs8, ns8,
                                      wq.data_ptr(), wqs.data_ptr(), y_post.data_ptr(), B.ISPA_BF16, ws8.data_ptr(),
                                      ws8_b, sh))
        e1.record(stream)
        e2.record(stream)
        ck(L.ispa_local_attn_fp8(n_q, H, d, scale, qc8.data_ptr(), qs8.data_ptr(), segs8, ns8, o8.data_ptr(),
                                 B.ISPA_F32, None, sh))
        e3.record(stream)
        fp8_marks.append((e0, e1, e2, e3))
    torch.cuda.synchronize()
    rec["post_fp8"] = [e0.elapsed_time(e1) for e0, e1, _, _ in fp8_marks]
    rec["attn8"] = [e2.elapsed_time(e3) for _, _, e2, e3 in fp8_marks]
    for e0, e1, e2, e3 in two_call:
        rec["attn"].append(e0.elapsed_time(e1))
        rec["merge"].append(e1.elapsed_time(e2))
        rec["stats_direct"].append(e2.elapsed_time(e3))
    for marks, (s0, s1, s2) in rec.pop("_pending", []):
        for e0, e1, e2, last in marks:
            rec["fused"].append(e0.elapsed_time(e1))
            if last:
                rec["stats"].append(e1.elapsed_time(e2))
        rec["switch"].append(s0.elapsed_time(s1))
        rec["post"].append(s1.elapsed_time(s2))
    if int(info[0]) != 0 or int(status[0]) != 0 or not torch.isfinite(eps).all():
        raise RuntimeError(f"solve failed: info={int(info[0])} status={int(status[0])} eps={float(eps[0])}")

    mean = lambda xs: sum(xs) / len(xs)  # noqa: E731
    attn_flops = 4.0 * n_q * (n_loc + n_hist) * D
    stats_flops = (4.0 * n_q * D * D + 2.0 * n_q * D) * STATS_CHUNKS  # G, H as triangles, M; per update call
    direct_flops = 5.0 * n_q * D * D + 3.0 * n_q * D  # R = dA W, C = A_loc^T R, G as a triangle, ||R||^2
    merge_bytes = 2 * (4 * n_q * D + 4 * n_q * H) + 2 * 2 * n_q * D
    attn8_flops = 4.0 * n_q * n_loc * D
    t_attn8 = mean(rec["attn8"]) * 1e-3
    t_fused = mean(rec["fused"]) * 1e-3
    t_attn = mean(rec["attn"]) * 1e-3
    t_merge = mean(rec["merge"]) * 1e-3
    t_stats = mean(rec["stats"]) * 1e-3
    t_direct = mean(rec["stats_direct"]) * 1e-3
    value = attn_flops / t_fused / 1e12
    achieved = attn_flops / t_fused / 1e12
    traffic = _traffic("attn_dual_single_pass_wan13b_counters.txt", "attn.hip")
    out = {
        "metric": "dual-stream attn+LSE-merge TFLOP/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Wan-1.3B-shaped layer, full ISPA cycle: 8 warmup chunks (4680 queries, "
                               "12 heads x 128, 9360 local + 28080 history keys) + ridge solve + "
                               "selection + 1 post-switch local chunk",
                   "n_q": n_q, "heads": H, "head_dim": d, "local_keys": n_loc, "history_keys": n_hist,
                   "warmup_chunks": n_warm, "stats_operands": "fp16", "stats_chunks_per_update": STATS_CHUNKS,
                   "seed": args.seed},
        "also": {
            "Gram-stat TFLOP/s": round(stats_flops / t_stats / 1e12, 2),
            "Gram-stat TFLOP/s counted as the direct form (5nD^2 + 3nD per chunk)":
                round(direct_flops * STATS_CHUNKS / t_stats / 1e12, 2),
            "accum_stats (direct form) call ms": round(t_direct * 1e3, 4),
            "accum_stats (direct form) TFLOP/s": round(direct_flops / t_direct / 1e12, 2),
            "ms/chunk (1 GPU)": round((t_fused + t_stats / STATS_CHUNKS) * 1e3, 4),
            "dual_attn_merge call ms": round(t_fused * 1e3, 4),
            "two-call path TFLOP/s (ispa_dual_attn + ispa_lse_merge)": round(attn_flops / (t_attn + t_merge) / 1e12, 2),
            "merge GB/s": round(merge_bytes / t_merge / 1e9, 1),
            "switch ms (finalize statistics + solve + select)": round(mean(rec["switch"]), 4),
            "post-switch chunk ms (local attn + W+dW)": round(mean(rec["post"]), 4),
            "post-switch chunk ms, quantised (current chunk to fp8, fp8 attention, W8A8 projection)":
                round(mean(rec["post_fp8"]), 4),
            "fp8 local attention call ms (sink + current, 9360 keys)": round(mean(rec["attn8"]), 4),
            "dual_attn call ms": round(t_attn * 1e3, 4),
            "merge call ms": round(t_merge * 1e3, 4),
            f"accum_gram call ms ({STATS_CHUNKS} chunks, {STATS_CHUNKS * n_q} rows)": round(t_stats * 1e3, 4),
            "accum_gram ms per chunk": round(t_stats / STATS_CHUNKS * 1e3, 4),
            "eps": float(eps[0]),
        },
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "kernel": "ispa_dual_attn_merge (single-pass attn_bf16_d128_kernel: both groups and the merge)"},
        "roofline_other": [
            {"kernel": "ispa_dual_attn (split pieces + history combine; the two-call path's attention)",
             "bound": "mfma", "achieved": round(attn_flops / t_attn / 1e12, 2), "peak": PEAK_BF16_TFLOPS,
             "unit": "TFLOP/s", "frac": round(attn_flops / t_attn / 1e12 / PEAK_BF16_TFLOPS, 4),
             "traffic": _traffic("attn_split_wan13b_traffic.txt", "attn.hip")},
            {"kernel": "ispa_local_attn_fp8 (attn_fp8_d128_kernel, post-switch L-Layer: 4680 queries x 9360 keys)",
             "bound": "mfma", "achieved": round(attn8_flops / t_attn8 / 1e12, 2), "peak": PEAK_FP8_TFLOPS,
             "unit": "TFLOP/s", "frac": round(attn8_flops / t_attn8 / 1e12 / PEAK_FP8_TFLOPS, 4),
             "traffic": _traffic("attn_fp8_wan13b_traffic.txt", "attn8.hip")},
            {"kernel": "ispa_lse_merge", "bound": "hbm", "achieved": round(merge_bytes / t_merge / 1e9, 1),
             "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(merge_bytes / t_merge / 1e9 / PEAK_HBM_GBS, 4),
             "traffic": _traffic("merge_wan13b_traffic.txt", "attn.hip")},
            {"kernel": f"ispa_accum_gram ({STATS_CHUNKS} chunks per call; flops performed: 4nD^2 + 2nD)",
             "bound": "mfma",
             "achieved": round(stats_flops / t_stats / 1e12, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
             "frac": round(stats_flops / t_stats / 1e12 / PEAK_BF16_TFLOPS, 4),
             "traffic": _traffic("syrk_wan13b_counters.txt", "gram.hip")},
        ],
    }
    if not (args.no_14b and args.no_video):
        del steps_in, seg_tables, ws
        torch.cuda.empty_cache()
    if not args.no_14b:
        out["also"]["Wan-14B streams"] = wan14b_figures(args.seed, dev)
    if not args.no_video:
        out["also"]["Wan-1.3B 30-second video, ISPA-0.5 against vanilla"] = video_figures(args.seed, dev)
    if not args.no_cpu_baseline:
        q, kc, vc = g.step(0)
        out["cpu_baseline"] = cpu_baseline(g, q, kc, vc)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
