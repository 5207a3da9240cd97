"""Parity of the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.

Bars: attention output rel-L2 <= 5e-3 and LSE abs <= 2e-3 with bf16 inputs;
merge vs monolithic attention <= 1e-5 relative in fp32 mode; dW
rel-Frobenius <= 1e-3; identical selection wherever the eps gap at the
K-th boundary exceeds 1e-4 relative.  Other bars are derived in each test.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(autouse=True)
def _gpu():
    _need_gpu()
    torch.manual_seed(0)
    print(flush=True)


def K():
    import kv_cache_absorption_amd as k
    return k


def h64(t):
    return t.detach().to("cpu").double().numpy()


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def rel_fro_upper(G_gpu, G_ref):
    iu = np.triu_indices(G_ref.shape[0])
    return rel(G_gpu[iu], G_ref[iu])


# ---------------------------------------------------------------- attention
def _cache(n, H, d, seed, dtype=torch.bfloat16, pad=0):
    """[n, H, d] rows with row stride H*d + pad (a view into a wider buffer)."""
    x = synth.normal((n, H * d + pad), seed, DEV, dtype=dtype)
    return x[:, : H * d].unflatten(1, (H, d))


@pytest.mark.parametrize("d,H,n_q,n_sink,n_hist,pad", [
    (128, 2, 200, 70, 300, 0),     # ragged q tile, ragged key tiles
    (128, 3, 129, 64, 1000, 64),   # strided rows, one query past a tile
    (64, 4, 77, 5, 190, 0),        # d = 64, tiny sink
    (128, 1, 1, 1, 1, 0),          # degenerate single query/key
    (128, 2, 100, 64, 9000, 0),    # history split into ragged pieces + merge
])
def test_dual_attn_bf16_parity(d, H, n_q, n_sink, n_hist, pad):
    print(f"dual_attn bf16 d={d} H={H} n_q={n_q} sink={n_sink} hist={n_hist} pad={pad}", flush=True)
    seed = 1000 + d + H
    q = _cache(n_q, H, d, seed, pad=pad)
    ks, vs = _cache(n_sink, H, d, seed + 1, pad=pad), _cache(n_sink, H, d, seed + 2, pad=pad)
    kc, vc = _cache(n_q, H, d, seed + 3, pad=pad), _cache(n_q, H, d, seed + 4, pad=pad)
    kh = _cache(n_hist, H, d, seed + 5, pad=pad) + 0.5
    vh = _cache(n_hist, H, d, seed + 6, pad=pad)
    scale = d ** -0.5
    o_l, l_l, o_h, l_h = K().ispa_dual_attn(q, [(ks, vs), (kc, vc)], [(kh, vh)], scale)
    torch.cuda.synchronize()
    ref = O.dual_stream_attention(q.cpu(), torch.cat([ks, kc]).cpu(), torch.cat([vs, vc]).cpu(),
                                  kh.cpu(), vh.cpu(), scale)
    assert rel(h64(o_l), ref["o_loc"]) <= 5e-3
    assert rel(h64(o_h), ref["o_hist"]) <= 5e-3
    assert np.abs(h64(l_l) - ref["lse_loc"]).max() <= 2e-3
    assert np.abs(h64(l_h) - ref["lse_hist"]).max() <= 2e-3


def test_dual_attn_many_segments():
    """Groups of three and four segments with ragged lengths: jobs over more
    than two segments take the general tile streams (segment changes inside a
    job), the others the two-run addressing."""
    print("dual_attn many segments", flush=True)
    H, d, n_q = 2, 128, 300
    q = _cache(n_q, H, d, 51)
    lens_l, lens_h = [100, 64, 333], [1, 700, 129, 64]
    ks = [_cache(n, H, d, 60 + i) for i, n in enumerate(lens_l)]
    vs = [_cache(n, H, d, 70 + i) for i, n in enumerate(lens_l)]
    kh = [_cache(n, H, d, 80 + i) + 0.5 for i, n in enumerate(lens_h)]
    vh = [_cache(n, H, d, 90 + i) for i, n in enumerate(lens_h)]
    o_l, l_l, o_h, l_h = K().ispa_dual_attn(q, list(zip(ks, vs)), list(zip(kh, vh)), d ** -0.5)
    torch.cuda.synchronize()
    ref = O.dual_stream_attention(q.cpu(), torch.cat(ks).cpu(), torch.cat(vs).cpu(), torch.cat(kh).cpu(),
                                  torch.cat(vh).cpu(), d ** -0.5)
    assert rel(h64(o_l), ref["o_loc"]) <= 5e-3
    assert rel(h64(o_h), ref["o_hist"]) <= 5e-3
    assert np.abs(h64(l_l) - ref["lse_loc"]).max() <= 2e-3
    assert np.abs(h64(l_h) - ref["lse_hist"]).max() <= 2e-3


def _staircase_keys(steps, tail, H, d, u, seed):
    """Keys whose score against queries along u climbs (or drops) by the
    given log2 offsets tile by tile (64 keys per tile, `tail` keys after the
    last full tile)."""
    c = d ** -0.5 * math.log2(math.e)
    n = 64 * len(steps) + tail
    k = 0.5 * synth.normal((n, H, d), seed, DEV).float()
    off = torch.tensor([steps[min(j // 64, len(steps) - 1)] for j in range(n)], device=DEV)
    k += (off / (c * 4.0))[:, None, None] * u[None]
    return k.to(torch.bfloat16)


def test_dual_attn_rebase_schedule():
    """Scores planted to step up tile by tile by more and by less than the
    kernel's lazy re-basing margin, then drop and climb again, in both
    groups: exercises re-basing on later tiles, P values up to 2^8 between
    re-basings, and tiles far below the running maximum."""
    print("dual_attn planted score staircase", flush=True)
    H, d, n_q = 2, 128, 96
    u = synth.normal((H, d), 41, DEV).float()
    u = u / u.norm(dim=1, keepdim=True)
    q = (0.5 * synth.normal((n_q, H, d), 42, DEV).float() + 4.0 * u[None]).to(torch.bfloat16)
    steps_l = [0, 3, 12, 14, 40, 41, 20, 90, 91, 200, 0, 205, 210]
    steps_h = [50, 7.9, 8.1, 60, 68.5, 0, 120, 127, 3]
    kl, vl = _staircase_keys(steps_l, 20, H, d, u, 43), _cache(64 * len(steps_l) + 20, H, d, 44)
    kh, vh = _staircase_keys(steps_h, 5, H, d, u, 45), _cache(64 * len(steps_h) + 5, H, d, 46)
    o_l, l_l, o_h, l_h = K().ispa_dual_attn(q, [(kl[:300], vl[:300]), (kl[300:], vl[300:])], [(kh, vh)],
                                            d ** -0.5)
    torch.cuda.synchronize()
    ref = O.dual_stream_attention(q.cpu(), kl.cpu(), vl.cpu(), kh.cpu(), vh.cpu(), d ** -0.5)
    assert rel(h64(o_l), ref["o_loc"]) <= 5e-3
    assert rel(h64(o_h), ref["o_hist"]) <= 5e-3
    assert np.abs(h64(l_l) - ref["lse_loc"]).max() <= 2e-3
    assert np.abs(h64(l_h) - ref["lse_hist"]).max() <= 2e-3
    assert ref["lse_loc"].min() > 100  # the planted offsets dominate the scores


def test_dual_attn_empty_history_and_zero_query():
    print("dual_attn empty history / zero query", flush=True)
    H, d, n = 2, 128, 150
    q = torch.zeros((n, H, d), dtype=torch.bfloat16, device=DEV)
    k, v = _cache(300, H, d, 7), _cache(300, H, d, 8)
    o_l, l_l, o_h, l_h = K().ispa_dual_attn(q, [(k, v)], [], d ** -0.5)
    torch.cuda.synchronize()
    assert torch.all(o_h == 0) and torch.all(torch.isneginf(l_h))
    # q = 0: uniform softmax, o = mean of v, lse = ln n
    np.testing.assert_allclose(h64(l_l), math.log(300), atol=1e-5)
    mean_v = h64(v).mean(axis=0)
    assert rel(h64(o_l), np.broadcast_to(mean_v, (n, H, d))) <= 1e-5


def test_dual_attn_wan13b_sampled_rows():
    """Wan-1.3B layer at full size (4680 queries, 12 heads, 9360 local and
    28080 history keys): every output row is computed on the GPU, a sample of
    64 query rows is checked against the oracle."""
    print("dual_attn wan1.3b full size, sampled rows", flush=True)
    g = synth.wan13b_single_layer(seed=3, device=DEV)
    q, kc, vc = g.step(0)
    o_l, l_l, o_h, l_h = K().ispa_dual_attn(q, [(g.sink_k, g.sink_v), (kc, vc)], [(g.hist_k, g.hist_v)])
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(5).choice(4680, 64, replace=False))
    rows = np.concatenate([rows, [4679, 4608, 0]])  # include the ragged last q tile
    ref = O.dual_stream_attention(q[rows].cpu(), torch.cat([g.sink_k, kc]).cpu(),
                                  torch.cat([g.sink_v, vc]).cpu(), g.hist_k.cpu(), g.hist_v.cpu(),
                                  128 ** -0.5)
    assert rel(h64(o_l[rows]), ref["o_loc"]) <= 5e-3
    assert rel(h64(o_h[rows]), ref["o_hist"]) <= 5e-3
    assert np.abs(h64(l_l[rows]) - ref["lse_loc"]).max() <= 2e-3
    assert np.abs(h64(l_h[rows]) - ref["lse_hist"]).max() <= 2e-3
    # history carries substantial mass (the offset keys make the merge matter)
    s = 1 / (1 + np.exp(-(ref["lse_hist"] - ref["lse_loc"])))
    assert 0.3 < s.mean() < 0.95


def test_dual_attn_f32_and_merge_tiny():
    """fp32 mode on the tiny workload: merged output vs monolithic attention
    <= 1e-5 relative."""
    print("dual_attn f32 tiny + merge", flush=True)
    g = synth.tiny_fp32(seed=11, device=DEV)
    q, kc, vc = g.step(0)
    o_l, l_l, o_h, l_h = K().ispa_dual_attn(q, [(g.sink_k, g.sink_v), (kc, vc)], [(g.hist_k, g.hist_v)],
                                            64 ** -0.5)
    o_f, l_f, a0, dl = K().ispa_lse_merge([o_l, o_h], [l_l, l_h], torch.float32)
    torch.cuda.synchronize()
    mono_o, mono_l = O.group_attention(q.cpu(), torch.cat([g.sink_k, kc, g.hist_k]).cpu(),
                                       torch.cat([g.sink_v, vc, g.hist_v]).cpu(), 64 ** -0.5)
    assert rel(h64(o_f), mono_o) <= 1e-5
    assert np.abs(h64(l_f) - mono_l).max() <= 1e-5 * np.abs(mono_l).max()
    assert torch.equal(a0.view(-1), o_l.view(-1))
    ref_delta = mono_o.reshape(64, -1) - h64(o_l).reshape(64, -1)
    assert rel(h64(dl), ref_delta) <= 1e-4


@pytest.mark.parametrize("dt,H,d,n_q,n_sink,n_cur,n_hist,out_dt", [
    (torch.bfloat16, 2, 128, 300, 256, 300, 1700, torch.float16),   # history in several pieces
    (torch.bfloat16, 2, 128, 600, 4680, 600, 300, torch.bfloat16),  # local longer: local split
    (torch.bfloat16, 2, 128, 257, 128, 257, 0, torch.float32),      # empty history
    (torch.float32, 2, 64, 64, 64, 64, 384, torch.float32),         # fp32 mode, tiny workload
])
def test_dual_attn_merge_parity(dt, H, d, n_q, n_sink, n_cur, n_hist, out_dt):
    """The fused call against the oracle's dual-stream attention + merge, and
    against the two-call path (ispa_dual_attn then ispa_lse_merge) on the same
    inputs: A_loc equal, dA within fp32 reassociation of the merge."""
    print(f"dual_attn_merge {dt} H={H} d={d} n_q={n_q} local={n_sink}+{n_cur} hist={n_hist} -> {out_dt}",
          flush=True)
    q = _cache(n_q, H, d, 131, dtype=dt)
    loc = [(_cache(n_sink, H, d, 132, dtype=dt), _cache(n_sink, H, d, 133, dtype=dt)),
           (_cache(n_cur, H, d, 134, dtype=dt), _cache(n_cur, H, d, 135, dtype=dt))]
    hist = [(_cache(n_hist, H, d, 136, dtype=dt), _cache(n_hist, H, d, 137, dtype=dt))] if n_hist else []
    a_loc, delta, lse = K().ispa_dual_attn_merge(q, loc, hist, out_dtype=out_dt)
    o_l, l_l, o_h, l_h = K().ispa_dual_attn(q, loc, hist)
    o_f, l_f, a0, dl = K().ispa_lse_merge([o_l, o_h], [l_l, l_h], out_dtype=out_dt)
    torch.cuda.synchronize()
    # the two GPU paths
    assert torch.equal(a_loc, a0)
    ulp = {torch.float32: 2.0 ** -23, torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -10}[out_dt]
    scale_full = float(o_f.abs().max())
    assert float((delta.float() - dl.float()).abs().max()) <= 4 * ulp * scale_full + 1e-6 * scale_full
    assert float((lse - l_f).abs().max()) <= 1e-5
    # the oracle
    cat = lambda pairs, i: torch.cat([p[i] for p in pairs]).cpu() if pairs else \
        torch.zeros((0, H, d), dtype=dt)  # noqa: E731
    ref = O.dual_stream_attention(q.cpu(), cat(loc, 0), cat(loc, 1), cat(hist, 0), cat(hist, 1), d ** -0.5)
    bar = 1e-5 if dt == torch.float32 else 5e-3
    a_ref = ref["a_loc"].reshape(n_q, -1)
    full_ref = ref["a_full"].reshape(n_q, -1)
    assert rel(h64(a_loc), a_ref) <= bar + ulp
    # dA = A_full - A_loc: its error is bounded by the errors of the two activations
    err = np.linalg.norm(h64(delta) - ref["delta"].reshape(n_q, -1))
    assert err <= (bar + ulp) * np.linalg.norm(full_ref) + (bar + ulp) * np.linalg.norm(a_ref)
    assert np.abs(h64(lse) - ref["lse_full"]).max() <= (1e-5 if dt == torch.float32 else 2e-3)


@pytest.mark.parametrize("H,n_q,loc_lens,hist_lens,out_dt", [
    (12, 4680, (4680, 4680), (9360,), torch.float16),        # Wan-1.3B layout, chunk 3 of a stream
    (12, 4680, (4680, 4680), (), torch.float16),             # chunk 1: no history yet
    (8, 6000, (700, 6000), (3000, 1500), torch.bfloat16),    # four ragged runs, ragged query tile
    (12, 4680, (), (3000,), torch.float16),                  # no local keys
    (12, 4680, (), (), torch.float16),                       # no keys at all
])
def test_dual_attn_merge_single_pass(H, n_q, loc_lens, hist_lens, out_dt):
    """The single-pass form of the fused call (one workgroup per query tile
    and head over both groups, at least 192 of them, 16-bit outputs).

    Sampled rows against the oracle (the attention bars; dA's own bound as
    in the split-path test), and every output against the split path on the
    same inputs (ispa_dual_attn + ispa_lse_merge).  The single pass holds the
    local output rounded to out_dt and forms dA = A_full - A_loc from that
    rounded A_loc, so dA may differ from the split path's by the rounding of
    A_loc (one unit in its last place) besides the attention's own error."""
    d, dt = 128, torch.bfloat16
    print(f"dual_attn_merge single pass H={H} n_q={n_q} local={loc_lens} hist={hist_lens} -> {out_dt}", flush=True)
    q = _cache(n_q, H, d, 141)
    loc = [(_cache(n, H, d, 142 + 2 * i), _cache(n, H, d, 143 + 2 * i)) for i, n in enumerate(loc_lens)]
    hist = [(_cache(n, H, d, 152 + 2 * i) + 0.5, _cache(n, H, d, 153 + 2 * i)) for i, n in enumerate(hist_lens)]
    a_loc, delta, lse = K().ispa_dual_attn_merge(q, loc, hist, out_dtype=out_dt)
    o_l, l_l, o_h, l_h = K().ispa_dual_attn(q, loc, hist)
    o_f, l_f, a0, dl = K().ispa_lse_merge([o_l, o_h], [l_l, l_h], out_dtype=out_dt)
    torch.cuda.synchronize()
    ulp = 2.0 ** -8 if out_dt == torch.bfloat16 else 2.0 ** -10
    # against the split path: A_loc within a rounding and the attention's own
    # difference (both from bf16 P), LSE, dA
    assert bool(torch.isfinite(a_loc.float()).all() and torch.isfinite(delta.float()).all())
    ea = rel(h64(a_loc), h64(a0)) if a0.abs().max() > 0 else float(a_loc.abs().max())
    ed = float((delta.float() - dl.float()).norm() / max(float(o_f.norm()), 1e-30))
    el = float((lse - l_f).abs().max()) if bool(torch.isfinite(l_f).any()) else 0.0
    print(f"vs split path: A_loc rel {ea:.2e}, dA rel (to |A_full|) {ed:.2e}, lse {el:.2e}", flush=True)
    assert ea <= 5e-3 and ed <= 5e-3
    assert torch.equal(torch.isinf(lse), torch.isinf(l_f))
    if not loc_lens and not hist_lens:
        assert not a_loc.float().any() and not delta.float().any() and bool(torch.isneginf(lse).all())
        return
    assert el <= 2e-3
    # sampled rows against the oracle
    rows = [0, 1, 255, 256, 2047, n_q // 2, n_q - 1]
    cat = lambda pairs, i: torch.cat([p[i] for p in pairs]).cpu() if pairs else \
        torch.zeros((0, H, d), dtype=dt)  # noqa: E731
    ref = O.dual_stream_attention(q[rows].cpu(), cat(loc, 0), cat(loc, 1), cat(hist, 0), cat(hist, 1), d ** -0.5)
    n = len(rows)
    a_ref, full_ref = ref["a_loc"].reshape(n, -1), ref["a_full"].reshape(n, -1)
    ar = h64(a_loc[rows])
    assert np.linalg.norm(ar - a_ref) <= (5e-3 + ulp) * max(np.linalg.norm(a_ref), 1e-30) + 1e-30
    err = np.linalg.norm(h64(delta[rows]) - ref["delta"].reshape(n, -1))
    assert err <= (5e-3 + 2 * ulp) * (np.linalg.norm(full_ref) + np.linalg.norm(a_ref))
    assert np.nanmax(np.abs(np.where(np.isinf(ref["lse_full"]), 0, h64(lse[rows]) - ref["lse_full"]))) <= 2e-3


# ---------------------------------------------------------------- merge
def test_merge_parts_from_oracle():
    print("merge: oracle parts, 3-way and empty", flush=True)
    rng = np.random.default_rng(21)
    n_q, H, d = 37, 3, 128
    qn = rng.normal(size=(n_q, H, d))
    ks = [rng.normal(size=(n, H, d)) + s for n, s in ((20, 0.0), (50, 0.5), (7, -0.3))]
    vs = [rng.normal(size=(n, H, d)) for n in (20, 50, 7)]
    parts = [O.group_attention(qn, k, v, 0.09) for k, v in zip(ks, vs)]
    mono_o, mono_l = O.group_attention(qn, np.concatenate(ks), np.concatenate(vs), 0.09)
    t = lambda a: torch.tensor(a, dtype=torch.float32, device=DEV).contiguous()  # noqa: E731
    o_f, l_f, a0, dl = K().ispa_lse_merge([t(p[0]) for p in parts], [t(p[1]) for p in parts],
                                          torch.float32)
    torch.cuda.synchronize()
    assert rel(h64(o_f), mono_o) <= 1e-5
    assert np.abs(h64(l_f) - mono_l).max() <= 1e-5 * np.abs(mono_l).max()
    # bf16 / f16 outputs are the fp32 values rounded once
    for dt in (torch.bfloat16, torch.float16):
        _, _, a0h, dlh = K().ispa_lse_merge([t(p[0]) for p in parts], [t(p[1]) for p in parts], dt,
                                            want_full=False)
        torch.cuda.synchronize()
        assert torch.equal(a0h.cpu(), a0.cpu().to(dt))
        assert torch.equal(dlh.cpu(), dl.cpu().to(dt))
    # empty parts get no weight; all-empty gives o = 0, lse = -inf
    z = torch.zeros((n_q, H, d), device=DEV)
    ninf = torch.full((n_q, H), -math.inf, device=DEV)
    o2, l2, _, d2 = K().ispa_lse_merge([t(parts[0][0]), z], [t(parts[0][1]), ninf])
    o3, l3, _, _ = K().ispa_lse_merge([z, z], [ninf, ninf])
    torch.cuda.synchronize()
    assert torch.allclose(o2, t(parts[0][0]), rtol=1e-6, atol=0) and torch.all(d2 == 0)
    assert torch.all(o3 == 0) and torch.all(torch.isneginf(l3))


# ---------------------------------------------------------------- statistics
@pytest.mark.parametrize("dt,n,D,steps", [
    (torch.bfloat16, 300, 256, 2),
    (torch.float16, 777, 128, 3),
    (torch.float16, 4680, 1536, 1),   # one Wan-1.3B warmup step
    (torch.float16, 4680, 5120, 1),   # one Wan-14B warmup step (no token split)
    (torch.float32, 64, 128, 4),      # tiny fp32 workload
])
def test_accum_stats_parity(dt, n, D, steps):
    print(f"accum_stats {dt} n={n} D={D} steps={steps}", flush=True)
    G = torch.zeros((D, D), dtype=torch.float32, device=DEV)
    C = torch.zeros_like(G)
    r2 = torch.zeros(1, dtype=torch.float64, device=DEV)
    w = synth.normal((D, D), 77, DEV, std=D ** -0.5, dtype=torch.bfloat16 if dt != torch.float32 else dt)
    Gr = np.zeros((D, D)); Cr = np.zeros((D, D)); rr = 0.0
    for s in range(steps):
        a = synth.normal((n, D), 100 + s, DEV, std=0.3, dtype=dt)
        dl = synth.normal((n, D), 200 + s, DEV, std=0.1, dtype=dt)
        K().ispa_accum_stats(a, dl, w, G, C, r2)
        g, c, r = O.accumulate_stats(a.cpu(), dl.cpu(), w.cpu())
        Gr += g; Cr += c; rr += r
    torch.cuda.synchronize()
    Gg = h64(G)
    assert rel_fro_upper(Gg, Gr) <= 1e-5
    assert np.all(np.tril(Gg, -1) == 0)  # lower triangle untouched
    # C: R is rounded to the operand type before A^T R (derived bar: one
    # rounding of R, 2^-9 relative for bf16, 2^-12 for f16, averaged over n)
    assert rel(h64(C), Cr) <= (2e-3 if dt == torch.bfloat16 else 5e-4)
    assert abs(float(r2.item()) - rr) <= 1e-5 * rr


@pytest.mark.parametrize("dt,n,D,steps", [
    (torch.float16, 4680, 1536, 2),   # two Wan-1.3B warmup chunks
    (torch.bfloat16, 300, 320, 3),    # ragged rows, a width that is not a multiple of 256
    (torch.float16, 33, 64, 2),       # one 64-wide block, a 1-row last stage
    (torch.float16, 4680, 5120, 1),   # one Wan-14B warmup chunk (no token split)
])
def test_accum_gram_parity(dt, n, D, steps):
    """The grouped statistics (one rank-k update of [A_loc | dA] per chunk,
    C = M W and r2 = <H, W W^T> at the switch) against the oracle's
    accumulate_gram and stats_from_gram on the same 16-bit operands.  The
    products are exact and summed in fp32 on both sides of the fp64 oracle,
    and M W runs on three bf16 planes of M (fp32 accuracy): bar 1e-5 for G,
    C and r2 (no operand is rounded on the way, unlike ispa_accum_stats's R)."""
    print(f"accum_gram {dt} n={n} D={D} steps={steps}", flush=True)
    state = K().gram_state(D, device=DEV)
    w = synth.normal((D, D), 77, DEV, std=D ** -0.5, dtype=torch.bfloat16)
    Gr = np.zeros((D, D)); Mr = np.zeros((D, D)); Hr = np.zeros((D, D))
    for s in range(steps):
        a = synth.normal((n, D), 100 + s, DEV, std=0.3, dtype=dt)
        dl = synth.normal((n, D), 200 + s, DEV, std=0.1, dtype=dt)
        K().ispa_accum_gram(a, dl, state)
        g, m, hh = O.accumulate_gram(a.cpu(), dl.cpu())
        Gr += g; Mr += m; Hr += hh
    st0 = state.clone()
    G, C, r2 = K().ispa_gram_finalize(state, w)
    torch.cuda.synchronize()
    assert torch.equal(state, st0)  # the finalize leaves the state as it was
    Gref, Cref, rref = O.stats_from_gram(Gr, Mr, Hr, w.cpu())
    Gg = h64(G)
    eg, ec, er = rel_fro_upper(Gg, Gref), rel(h64(C), Cref), abs(float(r2.item()) - rref) / rref
    print(f"G {eg:.2e}  C {ec:.2e}  r2 {er:.2e}", flush=True)
    assert eg <= 1e-5 and ec <= 1e-5 and er <= 1e-5
    assert np.all(np.tril(Gg, -1) == 0)  # below the diagonal untouched (zeros from gram_finalize's G)
    # n = 0 is a no-op
    K().ispa_accum_gram(a[:0], dl[:0], state)
    torch.cuda.synchronize()
    assert torch.equal(state, st0)


# ---------------------------------------------------------------- solve
def _stats_for_solve(D, n, seed, planted=False):
    rng = np.random.default_rng(seed)
    a = rng.normal(size=(n, D)) * 0.5
    w = rng.normal(size=(D, D)) / math.sqrt(D)
    dl = rng.normal(size=(n, D)) * 0.2 + 0.3 * a @ (rng.normal(size=(D, D)) / math.sqrt(D))
    G, C, r2 = O.accumulate_stats(a, dl, w)
    return G.astype(np.float32), C.astype(np.float32), r2, w


@pytest.mark.parametrize("D,L", [(64, 2), (128, 3), (256, 1), (1536, 1)])
def test_solve_parity(D, L):
    print(f"solve_dw D={D} layers={L}", flush=True)
    Gs, Cs, rs, ws = zip(*[_stats_for_solve(D, 3 * D, 50 + l) for l in range(L)])
    G = torch.tensor(np.stack(Gs), device=DEV)
    C = torch.tensor(np.stack(Cs), device=DEV)
    r2 = torch.tensor(rs, dtype=torch.float64, device=DEV)
    W = torch.tensor(np.stack(ws), dtype=torch.bfloat16, device=DEV)
    dW, eps, info, w_eff = K().ispa_solve_dw(G, C, r2, 0.0, 1e-3, w=W)
    torch.cuda.synchronize()
    assert torch.all(info == 0)
    for l in range(L):
        Gl, Cl = Gs[l].astype(np.float64), Cs[l].astype(np.float64)
        # the GPU reads the upper triangle of G: give the oracle the same matrix
        Gsym = np.triu(Gl) + np.triu(Gl, 1).T
        lam = O.ridge_lambda(Gsym, 0.0, 1e-3)
        ref, rinfo = O.solve_dw(Gsym, Cl, lam)
        assert rinfo == 0
        assert rel(h64(dW[l]), ref) <= 1e-3
        assert rel(h64(dW[l]), ref) <= 1e-6  # fp64 solve, fp32 output
        e_ref = O.epsilon_from_stats(Gsym, Cl, rs[l], ref)
        assert abs(float(eps[l]) - e_ref) <= 1e-6 * rs[l]
        weff_ref = (W[l].float().cpu() + torch.tensor(ref, dtype=torch.float32)).to(torch.bfloat16)
        assert (w_eff[l].cpu().float() - weff_ref.float()).abs().max() <= \
            2 ** -7 * weff_ref.float().abs().max()


def test_solve_grouped_batch():
    """A batch large enough for the grouped trailing updates (16 layers at
    D = 1088: 17 block columns, so the last group is partial), each layer against
    numpy's fp64 solve of the same symmetrised system."""
    D, L = 1088, 16
    print(f"solve_dw grouped D={D} layers={L}", flush=True)
    rng = np.random.default_rng(77)
    Gs, Cs = [], []
    for _ in range(L):
        a = rng.normal(size=(2 * D, D)).astype(np.float32)
        Gs.append(a.T @ a)
        Cs.append(rng.normal(size=(D, D)).astype(np.float32))
    G = torch.tensor(np.stack(Gs), device=DEV)
    C = torch.tensor(np.stack(Cs), device=DEV)
    r2 = torch.ones(L, dtype=torch.float64, device=DEV)
    dW, eps, info, _ = K().ispa_solve_dw(G, C, r2, 0.0, 1e-3)
    torch.cuda.synchronize()
    assert torch.all(info == 0)
    for l in (0, 7, L - 1):
        Gl = Gs[l].astype(np.float64)
        Gsym = np.triu(Gl) + np.triu(Gl, 1).T
        lam = 1e-3 * np.trace(Gsym) / D
        ref = np.linalg.solve(Gsym + lam * np.eye(D), Cs[l].astype(np.float64))
        assert rel(h64(dW[l]), ref) <= 1e-6, l


def test_solve_wan14b_layer():
    """One layer at the Wan-14B width (D = 5120: 80 block columns, grouped by
    8), against LAPACK's fp64 solve of the same symmetrised system; eps against
    the oracle's evaluation from the statistics."""
    D, n = 5120, 5376
    print(f"solve_dw D={D} layers=1", flush=True)
    rng = np.random.default_rng(78)
    a = rng.normal(size=(n, D)).astype(np.float32)
    Gf = a.T @ a
    Cf = (a.T @ rng.normal(size=(n, D)).astype(np.float32)).astype(np.float32)
    r2v = float(n * D)
    G = torch.tensor(Gf[None], device=DEV)
    C = torch.tensor(Cf[None], device=DEV)
    r2 = torch.tensor([r2v], dtype=torch.float64, device=DEV)
    dW, eps, info, _ = K().ispa_solve_dw(G, C, r2, 0.0, 1e-3)
    torch.cuda.synchronize()
    assert int(info[0]) == 0
    Gl = Gf.astype(np.float64)
    Gsym = np.triu(Gl) + np.triu(Gl, 1).T
    lam = 1e-3 * np.trace(Gsym) / D
    Cl = Cf.astype(np.float64)
    ref = np.linalg.solve(Gsym + lam * np.eye(D), Cl)
    assert rel(h64(dW[0]), ref) <= 1e-6
    e_ref = O.epsilon_from_stats(Gsym, Cl, r2v, ref)
    assert abs(float(eps[0]) - e_ref) <= 1e-6 * r2v


def test_solve_non_spd_reports_pivot():
    print("solve_dw non-SPD", flush=True)
    D = 128
    G = torch.eye(D, device=DEV)
    G[70, 70] = -1.0
    C = torch.ones((D, D), device=DEV)
    r2 = torch.ones(1, dtype=torch.float64, device=DEV)
    dW, eps, info, _ = K().ispa_solve_dw(G, C, r2, 0.0, 0.0)
    torch.cuda.synchronize()
    assert int(info[0]) == 71
    assert torch.isnan(eps[0]) and torch.all(torch.isnan(dW))


def test_solve_planted_and_large_lambda():
    print("solve_dw planted", flush=True)
    D, n = 256, 1024
    rng = np.random.default_rng(9)
    a = rng.normal(size=(n, D))
    dWs = 0.05 * rng.normal(size=(D, D))
    w = rng.normal(size=(D, D)) / math.sqrt(D)
    delta = a @ dWs @ np.linalg.inv(w)
    G, C, r2 = O.accumulate_stats(a, delta, w)
    t = lambda x: torch.tensor(x, dtype=torch.float32, device=DEV)  # noqa: E731
    r = torch.tensor([r2], dtype=torch.float64, device=DEV)
    dW, eps, info, _ = K().ispa_solve_dw(t(G), t(C), r, 0.0, 1e-9)
    dWb, epsb, _, _ = K().ispa_solve_dw(t(G), t(C), r, 1e12, 0.0)
    torch.cuda.synchronize()
    assert rel(h64(dW), dWs) <= 1e-3  # exactly linear target: dW* recovered
    assert float(eps[0]) <= 1e-4 * r2
    assert float(dWb.abs().max()) < 1e-6 and abs(float(epsb[0]) - r2) <= 1e-6 * r2


# ---------------------------------------------------------------- selection
def test_select_parity():
    print("select_layers", flush=True)
    rng = np.random.default_rng(3)
    for N, Kk in ((30, 15), (40, 20), (1, 1), (7, 0), (1024, 100)):
        eps = rng.uniform(size=N)
        if N > 5:
            eps[2] = eps[5]  # a tie: lower index first
        sel, is_local, st = K().ispa_select_layers(torch.tensor(eps, device=DEV), Kk)
        torch.cuda.synchronize()
        rsel, rloc, rst = O.select_layers(eps, Kk)
        assert int(st[0]) == rst == 0
        assert sel.cpu().numpy().tolist() == rsel.tolist()
        assert is_local.cpu().numpy().tolist() == rloc.tolist()
    bad = torch.tensor([0.1, float("nan"), 0.2], dtype=torch.float64, device=DEV)
    _, _, st = K().ispa_select_layers(bad, 1)
    torch.cuda.synchronize()
    assert int(st[0]) == 1


# ---------------------------------------------------------------- post-switch
@pytest.mark.parametrize("H,d,n_q,seg_lens,y_dt", [
    (2, 128, 300, [64, 300], torch.float32),        # L-layer: sink + current
    (2, 128, 130, [64, 500, 700, 130], torch.bfloat16),  # F-layer, several segments
    (4, 64, 200, [5000], torch.float32),             # long single segment (split)
    (12, 128, 600, [4680, 700], torch.bfloat16),     # D = 1536: several GEMM tiles, ragged rows
    # 8 query tiles x 16 heads = 128 workgroups, half the CUs: the key set runs
    # whole and the kernel writes its output as bf16 rows from its epilogue
    (16, 128, 2048, [4680, 700], torch.bfloat16),    # two runs of keys
    (16, 128, 2048, [1000, 2000, 3000], torch.float32),  # three runs: the segment-cursor form
])
def test_local_attn_proj_parity(H, d, n_q, seg_lens, y_dt):
    print(f"local_attn_proj H={H} d={d} n_q={n_q} segs={seg_lens} {y_dt}", flush=True)
    D = H * d
    q = _cache(n_q, H, d, 31)
    segs = [(_cache(n, H, d, 40 + i), _cache(n, H, d, 60 + i)) for i, n in enumerate(seg_lens)]
    w = synth.normal((D, D), 90, DEV, std=D ** -0.5)
    y = K().ispa_local_attn_proj(q, segs, w, d ** -0.5, out_dtype=y_dt)
    torch.cuda.synchronize()
    ref = O.local_attn_proj(q.cpu(), torch.cat([s[0] for s in segs]).cpu(),
                            torch.cat([s[1] for s in segs]).cpu(), w.cpu(), d ** -0.5)
    assert rel(h64(y), ref) <= 5e-3


def test_local_attn_proj_f16_weight():
    """W given as fp16: converted to the bf16 GEMM operand on its transpose."""
    H, d, n_q = 4, 128, 333
    print(f"local_attn_proj f16 W H={H} n_q={n_q}", flush=True)
    D = H * d
    q = _cache(n_q, H, d, 32)
    k, v = _cache(900, H, d, 41), _cache(900, H, d, 61)
    w = synth.normal((D, D), 91, DEV, std=D ** -0.5).to(torch.float16)
    y = K().ispa_local_attn_proj(q, [(k, v)], w, d ** -0.5, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = O.local_attn_proj(q.cpu(), k.cpu(), v.cpu(), w.cpu(), d ** -0.5)
    assert rel(h64(y), ref) <= 5e-3


def test_local_attn_proj_f32_tiny():
    print("local_attn_proj f32", flush=True)
    g = synth.tiny_fp32(seed=4, device=DEV)
    q, kc, vc = g.step(1)
    y = K().ispa_local_attn_proj(q, [(g.sink_k, g.sink_v), (kc, vc)], g.w, 64 ** -0.5,
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = O.local_attn_proj(q.cpu(), torch.cat([g.sink_k, kc]).cpu(), torch.cat([g.sink_v, vc]).cpu(),
                            g.w.cpu(), 64 ** -0.5)
    assert rel(h64(y), ref) <= 1e-5


# ---------------------------------------------------------------- end to end
def test_end_to_end_tiny_fp32():
    """The tiny workload through every call in fp32 mode, against the oracle
    run on the same seeded Q, K, V, W: 4 warmup steps, solve, selection, one
    post-switch chunk."""
    print("end-to-end tiny fp32", flush=True)
    k = K()
    g = synth.tiny_fp32(seed=1, device=DEV)
    D = g.D
    G = torch.zeros((D, D), device=DEV)
    C = torch.zeros_like(G)
    r2 = torch.zeros(1, dtype=torch.float64, device=DEV)
    Gr = np.zeros((D, D)); Cr = np.zeros((D, D)); rr = 0.0
    for s in range(4):
        q, kc, vc = g.step(s)
        o_l, l_l, o_h, l_h = k.ispa_dual_attn(q, [(g.sink_k, g.sink_v), (kc, vc)], [(g.hist_k, g.hist_v)],
                                              64 ** -0.5)
        _, _, a_loc, delta = k.ispa_lse_merge([o_l, o_h], [l_l, l_h], torch.float32, want_full=False)
        k.ispa_accum_stats(a_loc, delta, g.w, G, C, r2)
        ref = O.dual_stream_attention(q.cpu(), torch.cat([g.sink_k, kc]).cpu(), torch.cat([g.sink_v, vc]).cpu(),
                                      g.hist_k.cpu(), g.hist_v.cpu(), 64 ** -0.5)
        gg, cc, r = O.accumulate_stats(ref["a_loc"].reshape(64, D), ref["delta"].reshape(64, D), g.w.cpu())
        Gr += gg; Cr += cc; rr += r
    dW, eps, info, w_eff = k.ispa_solve_dw(G, C, r2, 0.0, 1e-3, w=g.w)
    sel, is_local, st = k.ispa_select_layers(eps, 1)
    torch.cuda.synchronize()
    lam = O.ridge_lambda(Gr, 0.0, 1e-3)
    dW_ref, _ = O.solve_dw(Gr, Cr, lam)
    assert int(info[0]) == 0 and int(st[0]) == 0 and int(sel[0]) == 0
    assert rel(h64(dW), dW_ref) <= 1e-3
    e_ref = O.epsilon_from_stats(Gr, Cr, rr, dW_ref)
    assert abs(float(eps[0]) - e_ref) <= 1e-3 * e_ref
    q, kc, vc = g.step(4)
    y = k.ispa_local_attn_proj(q, [(g.sink_k, g.sink_v), (kc, vc)], w_eff, 64 ** -0.5, out_dtype=torch.float32)
    torch.cuda.synchronize()
    y_ref = O.local_attn_proj(q.cpu(), torch.cat([g.sink_k, kc]).cpu(), torch.cat([g.sink_v, vc]).cpu(),
                              g.w.cpu().double().numpy() + dW_ref, 64 ** -0.5)
    assert rel(h64(y), y_ref) <= 1e-4


# ---------------------------------------------------------------- W8A8 projection
# The quantisation scheme is the oracle's (its docstrings state it): codes are
# integers decided in fp32 on both sides, so they must agree exactly.
@pytest.mark.parametrize("w_dt,d_in,d_out", [
    (torch.bfloat16, 1536, 1536),   # Wan-1.3B W_eff
    (torch.float16, 320, 196),      # ragged widths
])
def test_quantize_w_fp8_codes_exact(w_dt, d_in, d_out):
    print(f"quantize_w_fp8 {w_dt} {d_in}x{d_out}", flush=True)
    w = synth.normal((d_in, d_out), 91, DEV, std=d_in ** -0.5, dtype=w_dt)
    w[:, 5] = 0  # a zero output column: scale 0, zero codes
    codes, scales = K().ispa_quantize_w_fp8(w)
    torch.cuda.synchronize()
    rc, rs = O.quantize_weight_e4m3(w.cpu())
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy(), rs)


# The fp8 matrix core (v_mfma_scale_f32_32x32x64_f8f6f4) does not sum its
# products exactly: a GPU probe of known dot products shows each aligned group
# of 8 consecutive k added with about 12 bits below the group's largest
# product (smaller parts truncated; 448 + 2^-9 in one group gives 448, in two
# groups 448.001953125), the group sums then added in fp32.  So an output
# differs from the exact sum of the dequantised products by at most
# 7 * 2^-12 < 2^-9 of each group's largest |product|, summed over the groups,
# plus fp32 roundings.
def _w8a8_group_bound(x, w, rows, cols):
    """Per-output bound on |y_gpu - y_exact| for the sampled rows and columns:
    2^-9 * sum over 8-wide k groups of the largest |product| + 2^-20 * sum |product|."""
    qx, sx = O.quantize_rows_e4m3(x)
    qw, sw = O.quantize_weight_e4m3(w)
    xa = O.e4m3_decode(qx[rows]) * sx[rows].astype(np.float64)[:, None]
    wb = O.e4m3_decode(qw[cols]) * sw[cols].astype(np.float64)[:, None]
    prod = np.abs(xa[:, None, :] * wb[None, :, :])  # [rows, cols, d_in]
    gmax = prod.reshape(len(rows), len(cols), -1, 8).max(axis=3).sum(axis=2)
    return 2.0 ** -9 * gmax + 2.0 ** -20 * prod.sum(axis=2)


@pytest.mark.parametrize("x_dt,n,d_in,d_out,y_dt", [
    (torch.float32, 300, 320, 196, torch.float32),      # ragged: partial row and column tiles
    (torch.bfloat16, 4680, 1536, 1536, torch.float32),  # Wan-1.3B projection
    (torch.float32, 4680, 5120, 5120, torch.bfloat16),  # Wan-14B projection, bf16 output
])
def test_w8a8_linear_parity(x_dt, n, d_in, d_out, y_dt):
    print(f"w8a8_linear {x_dt} n={n} {d_in}x{d_out} -> {y_dt}", flush=True)
    x = synth.normal((n, d_in), 92, DEV, dtype=x_dt)
    x[7] = 0  # a zero row
    w = synth.normal((d_in, d_out), 93, DEV, std=d_in ** -0.5, dtype=torch.bfloat16)
    codes, scales = K().ispa_quantize_w_fp8(w)
    y = K().ispa_w8a8_linear(x, codes, scales, out_dtype=y_dt)
    torch.cuda.synchronize()
    xc, wc = x.cpu(), w.cpu()
    ref = O.w8a8_linear(xc, *O.quantize_weight_e4m3(wc))
    yg = h64(y)
    assert not yg[7].any()
    # whole output: the group truncation measured at 1.4e-5 rel-L2 (K = 320);
    # 1e-4 stays far below the ~3% the quantisation itself costs
    bf = y_dt == torch.bfloat16
    assert rel(yg, ref) <= (1e-4 + 2.0 ** -9 if bf else 1e-4)
    # sampled outputs against the elementwise bound (bf16 output: one more
    # rounding, 2^-9 of |y|)
    rows = np.unique(np.linspace(0, n - 1, 24).astype(int))
    cols = np.unique(np.linspace(0, d_out - 1, 40).astype(int))
    bound = _w8a8_group_bound(xc, wc, rows, cols)
    err = np.abs(yg[np.ix_(rows, cols)] - ref[np.ix_(rows, cols)])
    if bf:
        bound = bound + 2.0 ** -9 * np.abs(ref[np.ix_(rows, cols)])
    assert np.all(err <= bound), float(np.max(err / np.maximum(bound, 1e-300)))


def test_local_attn_proj_fp8_exact_when_attention_is():
    """Degenerate case: every key of a head has the same value row, so the
    attention output is that row whatever the scores (to fp32 rounding).  The
    rows hold values on the E4M3 grid times 2^-5 with a row maximum of 14, so
    the activation scale is 2^-5 and every code is a grid point, far from a
    rounding tie: the attention -> quantisation -> fp8 product wiring is then
    checked at the fp8 matrix core's own accuracy."""
    H, d, n_q, n_k = 12, 128, 300, 2000
    D = H * d
    print(f"local_attn_proj_fp8 degenerate H={H} n_q={n_q} keys={n_k}", flush=True)
    q = _cache(n_q, H, d, 95)
    k = _cache(n_k, H, d, 96)
    c = torch.arange(D, dtype=torch.float32)
    u = ((8 + (c * 5) % 8) / 8) * torch.exp2((c % 6) - 4) * torch.where(c % 3 == 0, -1.0, 1.0)
    u[17] = 14.0  # the row maximum: 1.75 * 2^3
    v = u.to(torch.bfloat16).reshape(1, H, d).expand(n_k, H, d).contiguous().to(DEV)
    w = synth.normal((D, D), 97, DEV, std=D ** -0.5, dtype=torch.bfloat16)
    codes, scales = K().ispa_quantize_w_fp8(w)
    y = K().ispa_local_attn_proj_fp8(q, [(k, v)], codes, scales, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = O.local_attn_proj_w8a8(q.cpu(), k.cpu(), v.cpu(), w.cpu(), d ** -0.5)
    # the fp8 matrix core's group truncation (see above) is the only error
    # left: 1e-4, as for the plain product, far below any wiring mistake
    assert rel(h64(y), ref) <= 1e-4
    o = u.double().numpy()[None, :].repeat(n_q, axis=0)
    cols = np.arange(0, D, 37)
    bound = _w8a8_group_bound(o.astype(np.float32), w.cpu(), np.arange(3), cols)
    assert np.all(np.abs(h64(y)[:3][:, cols] - ref[:3][:, cols]) <= bound + 1e-6 * np.abs(ref[:3][:, cols]))


def test_local_attn_proj_fp8_wan13b_shape():
    """Sink + current chunk of a Wan-1.3B layer (300 of the 4680 queries).

    The W8A8 stage at the matrix core's own accuracy: the call's output
    equals, bit for bit, the GPU attention's fp32 output (ispa_dual_attn over
    the same key set) put through ispa_w8a8_linear, and that product matches
    the oracle's w8a8_linear of the same fp32 activations (quantised on the
    host from the GPU's values, so the codes are the same decisions) within
    rel-L2 1e-4 and the per-element group bound.  A call that skipped or
    mis-scaled the activation quantisation would miss it by the scheme's
    few-percent cost.

    Against the oracle's W8A8 chain from the inputs: the GPU attention differs from the fp64
    one by up to 5e-3 relative; an activation whose x / scale lies that close
    to a rounding midpoint gets the neighbouring code on one side, one E4M3
    step (2^-4 .. 2^-3 relative) apart.  About 5e-3 / 2^-4 = 8% of the codes
    can flip, an rms activation difference of sqrt(0.08) * 2^-3.5 ~ 2.5%,
    which carries into y; 4e-2 leaves margin.  The quantisation itself costs
    a few percent against the unquantised projection (oracle pin: 1e-3 to
    6e-2 on Gaussian operands)."""
    H, d, n_q, n_sink, n_cur = 12, 128, 300, 1560, 300
    D = H * d
    print(f"local_attn_proj_fp8 H={H} n_q={n_q} keys={n_sink + n_cur}", flush=True)
    g = synth.GroupInputs(n_q, H, d, n_sink, 0, torch.bfloat16, 98, DEV, workload=2)
    q, kc, vc = g.step(0)
    w = synth.normal((D, D), 99, DEV, std=D ** -0.5, dtype=torch.bfloat16)
    codes, scales = K().ispa_quantize_w_fp8(w)
    segs = [(g.sink_k, g.sink_v), (kc, vc)]
    y = K().ispa_local_attn_proj_fp8(q, segs, codes, scales, out_dtype=torch.float32)
    torch.cuda.synchronize()
    kk = torch.cat([g.sink_k, kc]).cpu()
    vv = torch.cat([g.sink_v, vc]).cpu()
    ref = O.local_attn_proj_w8a8(q.cpu(), kk, vv, w.cpu(), d ** -0.5)
    ref_full = O.local_attn_proj(q.cpu(), kk, vv, w.cpu(), d ** -0.5)
    e8, ef = rel(h64(y), ref), rel(h64(y), ref_full)
    # the W8A8 stage on the GPU's own attention output
    o_gpu = K().ispa_dual_attn(q, segs, [], d ** -0.5)[0].reshape(n_q, D)
    y_comp = K().ispa_w8a8_linear(o_gpu, codes, scales, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y, y_comp)
    oc = o_gpu.cpu()
    ref_g = O.w8a8_linear(oc, *O.quantize_weight_e4m3(w.cpu()))
    eg = rel(h64(y), ref_g)
    rows = np.arange(0, n_q, 23)
    cols = np.arange(0, D, 41)
    bound = _w8a8_group_bound(oc.numpy(), w.cpu(), rows, cols)
    assert np.all(np.abs(h64(y)[np.ix_(rows, cols)] - ref_g[np.ix_(rows, cols)]) <= bound)
    print(f"rel-L2 vs oracle W8A8 on the GPU attention output {eg:.3e}; vs the oracle's W8A8 chain {e8:.3e}; "
          f"vs unquantised {ef:.3e}", flush=True)
    assert eg <= 1e-4
    assert e8 <= 4e-2
    assert ef <= 6e-2


def test_local_attn_proj_fp8_empty_keys():
    """An empty key set: attention gives 0, the activation rows are all zero
    (scale 0, zero codes), so y = 0 exactly, as on the bf16 path."""
    H, d, n_q = 2, 128, 70
    print("local_attn_proj_fp8 empty key set", flush=True)
    q = _cache(n_q, H, d, 101)
    k = _cache(1, H, d, 102)[:0]
    w = synth.normal((H * d, H * d), 103, DEV, std=(H * d) ** -0.5, dtype=torch.bfloat16)
    codes, scales = K().ispa_quantize_w_fp8(w)
    y = K().ispa_local_attn_proj_fp8(q, [(k, k)], codes, scales, out_dtype=torch.float32)
    y16 = K().ispa_local_attn_proj(q, [(k, k)], w, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert not h64(y).any() and not h64(y16).any()
