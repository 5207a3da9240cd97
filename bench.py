#!/usr/bin/env python3
"""Throughput of the ISPA hot path on one MI355X.

One step is one full cycle of the Wan-1.3B-shaped single-layer workload
(12 heads x 128 = 1536 wide, 4680 queries per chunk, a 4680-key sink, a
28080-key history, fresh current chunk each step):

  8 warmup chunk steps, each ispa_dual_attn_merge (dual-stream attention and
    the LSE merge into A_loc, A_full - A_loc) -> ispa_accum_stats
  the switch: ispa_solve_dw (dW, eps, W + dW) -> ispa_select_layers (K = 1 of 1)
  one post-switch chunk of the (local) layer: ispa_local_attn_proj with W + dW

All inputs are generated on the GPU before the timed region.  Prints one JSON
line; the headline value is dual-stream attention + LSE merge TFLOP/s (QK^T
and PV flops, 4 n_q n_k D per chunk, over the time of the fused call), with
Gram-statistics TFLOP/s and ms per warmup chunk beside it.  The same chunks
through the two separate calls (ispa_dual_attn, then ispa_lse_merge) are
timed after the timed steps and reported beside it; the roofline entry is the
ispa_dual_attn call.

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
  wan14b_post_w8a8  wan14b_post with the W8A8 projections: W and W + dW
                 quantised once (untimed, at the switch) to FP8 E4M3, the
                 attention output per token, the products on the fp8 matrix core
  wan13b_recal   the wan13b_stream layers with warmup re-entered: warmup 0-5,
                 switch, post-switch 6-11, warmup again at 12-17 (statistics
                 from zero, every layer over the keys it still holds), switch,
                 post-switch 18-23
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

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


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
                rec["sha"] = line.split(":", 1)[1].strip()
    if rec.get("sha") != _src_hash(src) or "bytes" not in rec:
        return None
    return rec["bytes"]


def cpu_baseline(g, q, kc, vc, rows_target_s=15.0):
    """The oracle timed on host cores on a bounded sample: dual-stream
    attention + merge for a subset of query rows of one warmup chunk."""
    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing
        cores = os.cpu_count()
    k_loc = torch.cat([g.sink_k, kc]).cpu()
    v_loc = torch.cat([g.sink_v, vc]).cpu()
    k_h, v_h = g.hist_k.cpu(), g.hist_v.cpu()
    qh = q.cpu()
    n_k = k_loc.shape[0] + k_h.shape[0]
    D = g.D
    rows_done, t_tot, chunk = 0, 0.0, 64
    while t_tot < rows_target_s and rows_done + chunk <= qh.shape[0]:
        t0 = time.perf_counter()
        O.dual_stream_attention(qh[rows_done:rows_done + chunk], k_loc, v_loc, k_h, v_h, g.d ** -0.5)
        t_tot += time.perf_counter() - t0
        rows_done += chunk
    flops = 4.0 * rows_done * n_k * D
    return {"value": flops / t_tot / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"fp64 numpy oracle, dual-stream attention + LSE merge of {rows_done} of 4680 "
                      f"query rows (all 12 heads, {n_k} keys) of one warmup chunk; {t_tot:.1f} s",
            "seconds": t_tot}


STREAMS = {
    # name: layers, heads, head_dim, chunks in the pass, warmup chunks, K, workload id
    "wan13b_stream": dict(N=30, H=12, d=128, chunks=20, warm=6, K=15, wid=3),
    "wan14b_warmup": dict(N=40, H=40, d=128, chunks=19, warm=19, K=20, wid=4),
    "wan14b_post": dict(N=40, H=40, d=128, chunks=40, warm=0, K=20, wid=5),
    "wan14b_post_w8a8": dict(N=40, H=40, d=128, chunks=40, warm=0, K=20, wid=5, w8a8=True),
    # re-calibration: warmup 0-5, switch, post 6-11, warmup re-entered at 12
    # (12-17), switch again, post 18-23
    "wan13b_recal": dict(N=30, H=12, d=128, chunks=24, warm=6, K=15, wid=3, recal=12, warm2=6),
    # budget / warmup sweep: one 8-chunk (24-frame) warmup, evaluated after
    # 2, 4, 6 and 8 chunks (6-24 frames) for x = 0.3, 0.4, 0.5, 0.7
    "wan13b_sweep": dict(N=30, H=12, d=128, chunks=8, warm=8, K=15, wid=3,
                         evaluate_at=(2, 4, 6, 8), xs=(0.3, 0.4, 0.5, 0.7)),
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
    stream = torch.cuda.current_stream(dev)
    qbuf = torch.empty((N, T, H, d), dtype=torch.bfloat16, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    recs = []
    switch_ev = []
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
        if spec.get("evaluate_at") and c + 1 in spec["evaluate_at"]:
            Ks = [round(x * N) for x in spec["xs"]]
            v0, v1 = ev(), ev()
            v0.record(stream)
            eps_e, sels_e, _, _ = st.evaluate(Ks)
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
    G += torch.eye(H * d, device=dev)
    _, eps, _, _ = K.ispa_solve_dw(G, C, r2, 0.0, 1e-3, w=w)
    K.ispa_select_layers(eps, 1)
    K.ispa_local_attn_proj(q, [(k, v)], w)
    torch.cuda.synchronize()


def run_stream(args, name, dev):
    import torch
    spec = STREAMS[name]
    _preload_kernels(dev)
    N, H, d, T = spec["N"], spec["H"], spec["d"], TOKENS_PER_CHUNK
    D = H * d
    adopt = None
    pre = {}
    if name in ("wan14b_post", "wan14b_post_w8a8"):
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
            stats_flops += N * (5.0 * T * D * D + 3.0 * T * D)
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
                   "stats_operands": "fp16", "seed": args.seed,
                   "timing": "HIP events around each chunk's ISPA calls of all layers; the chunk's "
                             "synthetic Q/K/V generation sits outside them (ms_per_step is the wall "
                             "time of the whole pass including that generation)"},
        "also": {
            "warmup ms/chunk (mean)": round(mean(warm_ms), 3) if warm_ms else None,
            "post-switch ms/chunk (mean)": round(mean(post_ms), 3) if post_ms else None,
            "last chunk ms": round(last["ms"], 3),
            "switch ms (solve all layers + select)": round(switch_ms, 3) if switch_ms else None,
            "pass TFLOP/s (attention + statistics + projection flops / ISPA time)": round(achieved, 2),
            "kv_bytes_held_last_chunk": last["kv_held"],
            "kv_bytes_all_full_last_chunk": full_bytes,
            "kv_held_fraction": round(last["kv_held"] / full_bytes, 4),
            "kv_bytes_allocated_last_chunk": last["kv_alloc"],
            "L-Layers": [i for i, f in enumerate(st.is_local_host or []) if f],
            **pre,
        },
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "all ISPA calls of the pass (attention dominates)"},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


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
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes (counter calibration)")
    ap.add_argument("--attn-only", type=int, default=0,
                    help="only run this many dual-attention calls of the workload (counter runs)")
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
    if args.proj_compare:
        print(json.dumps(proj_compare(args.proj_compare, dev)))
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
    a_loc = torch.empty((n_q, D), dtype=torch.float16, device=dev)
    delta = torch.empty_like(a_loc)
    G = torch.zeros((D, D), **f32)
    C = torch.zeros((D, D), **f32)
    r2 = torch.zeros(1, dtype=torch.float64, device=dev)
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
    ws_stats_b = L.ispa_accum_stats_workspace_bytes(B.ISPA_F16, n_q, D)
    ws_solve_b = L.ispa_solve_dw_workspace_bytes(1, D)
    post_segs, post_n = segs([(g.sink_k, g.sink_v), (k_post, v_post)])
    ws_post_b = L.ispa_local_attn_proj_workspace_bytes(B.ISPA_BF16, n_q, H, d, post_segs, post_n)
    ws = torch.empty(max(ws_attn_b, ws_stats_b, ws_solve_b, ws_post_b, 256), dtype=torch.uint8, device=dev)
    wsp, wsn = ws.data_ptr(), ws.numel()
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
    rec = {"fused": [], "attn": [], "merge": [], "stats": [], "switch": [], "post": []}

    def cycle(timed):
        G.zero_()
        C.zero_()
        r2.zero_()
        marks = []
        for (q, ls, nl, hs, nh) in seg_tables:
            e0, e1, e2 = ev(), ev(), ev()
            e0.record(stream)
            ck(L.ispa_dual_attn_merge(B.ISPA_BF16, n_q, H, d, scale, q.data_ptr(), q.stride(0), ls, nl, hs,
                                      nh, a_loc.data_ptr(), delta.data_ptr(), B.ISPA_F16, None, wsp, wsn, sh))
            e1.record(stream)
            ck(L.ispa_accum_stats(B.ISPA_F16, B.ISPA_BF16, n_q, D, a_loc.data_ptr(), delta.data_ptr(),
                                  g.w.data_ptr(), G.data_ptr(), C.data_ptr(), r2.data_ptr(), wsp, wsn, sh))
            e2.record(stream)
            marks.append((e0, e1, e2))
        s0, s1, s2 = ev(), ev(), ev()
        s0.record(stream)
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
    # the same warmup chunks through the two separate calls (after the timed steps)
    two_call = []
    for (q, ls, nl, hs, nh) in seg_tables:
        e0, e1, e2 = ev(), ev(), ev()
        e0.record(stream)
        ck(L.ispa_dual_attn(B.ISPA_BF16, n_q, H, d, scale, q.data_ptr(), q.stride(0), ls, nl, hs, nh,
                            o_loc.data_ptr(), lse_loc.data_ptr(), o_hist.data_ptr(), lse_hist.data_ptr(),
                            wsp, wsn, sh))
        e1.record(stream)
        ck(L.ispa_lse_merge(2, op, lp, n_q, H, d, None, None, a_loc.data_ptr(), delta.data_ptr(),
                            B.ISPA_F16, sh))
        e2.record(stream)
        two_call.append((e0, e1, e2))
    torch.cuda.synchronize()
    for e0, e1, e2 in two_call:
        rec["attn"].append(e0.elapsed_time(e1))
        rec["merge"].append(e1.elapsed_time(e2))
    for marks, (s0, s1, s2) in rec.pop("_pending", []):
        for e0, e1, e2 in marks:
            rec["fused"].append(e0.elapsed_time(e1))
            rec["stats"].append(e1.elapsed_time(e2))
        rec["switch"].append(s0.elapsed_time(s1))
        rec["post"].append(s1.elapsed_time(s2))
    if int(info[0]) != 0 or int(status[0]) != 0 or not torch.isfinite(eps).all():
        raise RuntimeError(f"solve failed: info={int(info[0])} status={int(status[0])} eps={float(eps[0])}")

    mean = lambda xs: sum(xs) / len(xs)  # noqa: E731
    attn_flops = 4.0 * n_q * (n_loc + n_hist) * D
    stats_flops = 5.0 * n_q * D * D + 3.0 * n_q * D
    merge_bytes = 2 * (4 * n_q * D + 4 * n_q * H) + 2 * 2 * n_q * D
    t_fused = mean(rec["fused"]) * 1e-3
    t_attn = mean(rec["attn"]) * 1e-3
    t_merge = mean(rec["merge"]) * 1e-3
    t_stats = mean(rec["stats"]) * 1e-3
    value = attn_flops / t_fused / 1e12
    achieved = attn_flops / t_attn / 1e12
    traffic = _traffic("attn_bf16_wan13b_traffic.txt", "attn.hip")
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
                   "warmup_chunks": n_warm, "stats_operands": "fp16", "seed": args.seed},
        "also": {
            "Gram-stat TFLOP/s": round(stats_flops / t_stats / 1e12, 2),
            "ms/chunk (1 GPU)": round((t_fused + t_stats) * 1e3, 4),
            "dual_attn_merge call ms": round(t_fused * 1e3, 4),
            "two-call path TFLOP/s (ispa_dual_attn + ispa_lse_merge)": round(attn_flops / (t_attn + t_merge) / 1e12, 2),
            "merge GB/s": round(merge_bytes / t_merge / 1e9, 1),
            "switch ms (solve+select)": round(mean(rec["switch"]), 4),
            "post-switch chunk ms (local attn + W+dW)": round(mean(rec["post"]), 4),
            "dual_attn call ms": round(t_attn * 1e3, 4),
            "merge call ms": round(t_merge * 1e3, 4),
            "stats call ms": round(t_stats * 1e3, 4),
            "eps": float(eps[0]),
        },
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "kernel": "ispa_dual_attn call (attn_bf16_d128_kernel + history-split combine)"},
        "roofline_other": [
            {"kernel": "ispa_lse_merge", "bound": "hbm", "achieved": round(merge_bytes / t_merge / 1e9, 1),
             "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(merge_bytes / t_merge / 1e9 / PEAK_HBM_GBS, 4)},
            {"kernel": "ispa_accum_stats", "bound": "mfma",
             "achieved": round(stats_flops / t_stats / 1e12, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
             "frac": round(stats_flops / t_stats / 1e12 / PEAK_BF16_TFLOPS, 4)},
        ],
    }
    if not args.no_cpu_baseline:
        q, kc, vc = steps_in[0]
        out["cpu_baseline"] = cpu_baseline(g, q, kc, vc)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
