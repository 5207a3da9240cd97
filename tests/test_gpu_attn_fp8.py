"""Parity of the quantised local attention (fp8 cache, fp8 queries, the
attention on the fp8 matrix core) against the oracle's attention_fp8.

Codes and scales are integers decided in fp32 on both sides and compare bit
for bit.  The attention output differs from the oracle's (the exact softmax
attention of the dequantised operands) by the kernel's own roundings:
  * each probability p is rounded to E4M3 before the PV product, a relative
    error delta with |delta| <= 2^-4 (RNE with 3 mantissa bits); with the row
    weights w_j = p_j / sum p the output moves by sum_j w_j delta_j (v_j - o),
    whose variance is at most (2^-4)^2 / 3 * sum_j w_j^2 (v_j - o)^2 when the
    rounding errors are independent and uniform;
  * the fp8 matrix core's products are accumulated in groups of 8 with a
    truncation below 2^-9 of the group's largest product (measured for the
    W8A8 product), a far smaller effect on the scores and sums.
The bar on realistic inputs is therefore statistical: the summed squared
error over the checked outputs is at most 3x the predicted variance (rms at
most 1.73x), with the prediction computed here in fp64 from the dequantised
operands.  On inputs whose scores are integers in log2 units (every
probability a power of two, so its rounding is exact) and whose products stay
within the matrix core's exact range, the kernel must match to fp32
accumulation (1e-5)."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(flush=True)


def K():
    import kv_cache_absorption_amd as k
    return k


def h64(t):
    return t.detach().to("cpu").double().numpy()


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# ---------------------------------------------------------------- cache layout
def untile_k(codes, n, H):
    """The library's K tiles -> codes [n, H, 128] (and the padding rows)."""
    T = -(-n // 64)
    t = codes.cpu().numpy().reshape(H, T, 64, 8, 16)  # head, tile, row, stored chunk, byte
    r = np.arange(64)[:, None]
    c = np.arange(8)[None, :]
    t = t[:, :, r, c ^ ((r >> 1) & 7), :]              # stored position of logical chunk c
    full = t.reshape(H, T * 64, 128).transpose(1, 0, 2)
    return full[:n], full[n:]


def untile_v(codes, n, H):
    """The library's V^T tiles -> codes [n, H, 128] (and the padding rows)."""
    T = -(-n // 64)
    t = codes.cpu().numpy().reshape(H, T, 128, 4, 16)  # head, tile, d, stored chunk, byte
    dd = np.arange(128)[:, None]
    c = np.arange(4)[None, :]
    t = t[:, :, dd, c ^ ((dd >> 2) & 3), :].reshape(H, T, 128, 64)  # [.., d, position]
    p = np.arange(64)
    key = ((p >> 4) & 1) * 32 + ((p >> 2) & 3) * 8 + (p >> 5) * 4 + (p & 3)
    out = np.empty_like(t)
    out[..., key] = t                                   # position p holds key key[p]
    full = out.transpose(1, 3, 0, 2).reshape(T * 64, H, 128)  # [tile, key, head, d]
    return full[:n], full[n:]


@pytest.mark.parametrize("dt,n,H,pad", [
    (torch.bfloat16, 4680, 12, 0),    # a Wan-1.3B chunk: 73 full tiles and an 8-key tail
    (torch.float32, 100, 3, 8),       # strided fp32 rows
    (torch.float16, 64, 2, 0),        # exactly one tile
    (torch.bfloat16, 1, 1, 0),        # one key
])
def test_quantize_kv_fp8_bit_exact(dt, n, H, pad):
    print(f"quantize_kv_fp8 {dt} n={n} H={H} pad={pad}", flush=True)
    kb = synth.normal((n, H * 128 + pad), 301, DEV, dtype=dt)
    vb = synth.normal((n, H * 128 + pad), 302, DEV, dtype=dt)
    kb[:, :128] *= 1e3  # head 0 of K on another scale
    if H > 1:
        vb[:, 128:256] = 0  # an all-zero V head: scale 1, zero codes
    k, v = kb[:, :H * 128].unflatten(1, (H, 128)), vb[:, :H * 128].unflatten(1, (H, 128))
    ch = K().ispa_quantize_kv_fp8(k, v)
    torch.cuda.synchronize()
    kc, ks = O.quantize_chunk_e4m3(k.cpu())
    vc, vs = O.quantize_chunk_e4m3(v.cpu())
    np.testing.assert_array_equal(ch.k_scales.cpu().numpy(), ks)
    np.testing.assert_array_equal(ch.v_scales.cpu().numpy(), vs)
    gk, pk = untile_k(ch.k_codes, n, H)
    gv, pv = untile_v(ch.v_codes, n, H)
    np.testing.assert_array_equal(gk, kc)
    np.testing.assert_array_equal(gv, vc)
    assert not pk.any() and not pv.any()  # keys past n are zero codes


@pytest.mark.parametrize("dt,n_q,H", [(torch.bfloat16, 4680, 12), (torch.float32, 37, 5)])
def test_quantize_q_fp8_bit_exact(dt, n_q, H):
    print(f"quantize_q_fp8 {dt} n_q={n_q} H={H}", flush=True)
    q = synth.normal((n_q, H * 128 + 8), 303, DEV, dtype=dt)[:, : H * 128].unflatten(1, (H, 128))
    q[3, 0] = 0  # a zero (row, head)
    q[5, H - 1] *= 1e-30
    qc, qs = K().ispa_quantize_q_fp8(q)
    torch.cuda.synchronize()
    oc, os_ = O.quantize_heads_e4m3(q.cpu())
    np.testing.assert_array_equal(qs.cpu().numpy(), os_)
    np.testing.assert_array_equal(qc.cpu().numpy(), oc)


# ---------------------------------------------------------------- attention
def _deq(codes, scales_b):
    return O.e4m3_decode(codes) * scales_b


def _predicted_var(qh, kh, vh, scale, rows):
    """sum over the given rows of the predicted variance of the output error
    (see the module docstring) and the oracle output there, per head."""
    tot = 0.0
    for h in range(qh.shape[1]):
        s = scale * (qh[rows, h] @ kh[:, h].T)                 # [r, n]
        w = np.exp(s - s.max(axis=1, keepdims=True))
        w /= w.sum(axis=1, keepdims=True)
        o = w @ vh[:, h]                                       # [r, d]
        # sum_j w_j^2 (v_j - o)^2 = sum_j w_j^2 v_j^2 - 2 o sum_j w_j^2 v_j + o^2 sum_j w_j^2
        w2 = w * w
        tot += float(((w2 @ (vh[:, h] ** 2)) - 2 * o * (w2 @ vh[:, h]) + o * o * w2.sum(axis=1, keepdims=True)).sum())
    return (2.0 ** -4) ** 2 / 3.0 * tot


def _run(q, chunks_kv, scale, rows=None, out_dtype=torch.float32):
    """GPU: quantise q and the chunks, run the attention; oracle: attention_fp8.
    Returns (gpu o, gpu lse, oracle o, oracle lse, dequantised q, k, v) on rows."""
    k8 = K()
    chunks = [k8.ispa_quantize_kv_fp8(k, v) for k, v in chunks_kv]
    qc, qs = k8.ispa_quantize_q_fp8(q)
    o, lse = k8.ispa_local_attn_fp8(qc, qs, chunks, scale=scale, out_dtype=out_dtype, want_lse=True)
    torch.cuda.synchronize()
    qcpu = q.cpu()
    rows = np.arange(q.shape[0]) if rows is None else rows
    ks = [k.cpu() for k, _ in chunks_kv]
    vs = [v.cpu() for _, v in chunks_kv]
    ro, rl = O.attention_fp8(qcpu[rows], ks, vs, scale)
    qcodes, qsc = O.quantize_heads_e4m3(qcpu)
    qh = _deq(qcodes, qsc.astype(np.float64)[:, :, None])

    def deq_chunk(x):
        c, sc = O.quantize_chunk_e4m3(x)
        return _deq(c, sc.astype(np.float64)[None, :, None])

    kh = [deq_chunk(k) for k in ks]
    vh = [deq_chunk(v) for v in vs]
    H = q.shape[1]
    kh = np.concatenate(kh) if kh else np.zeros((0, H, 128))
    vh = np.concatenate(vh) if vh else np.zeros((0, H, 128))
    return h64(o)[rows], h64(lse)[rows], ro, rl, qh, kh, vh


def _grid(n, H, seed, marker_col, density=0.06):
    """Integer-valued [n, H, 128] rows: entries in {-1, 0, 1} with the given
    density, and 4 at column marker_col of every row (so every row's, and every
    chunk's, maximum magnitude is 4: scale 2^-6, codes 64 x value, exact)."""
    g = torch.Generator().manual_seed(seed)
    x = (torch.rand((n, H, 128), generator=g) < density).float() * (torch.randint(0, 2, (n, H, 128), generator=g) * 2 - 1)
    x[:, :, marker_col] = 4.0
    return x


def test_local_attn_fp8_exact_on_power_of_two_scores():
    """Scores in log2 units are the integers <q, k> in [-2, 4] (scale = ln 2):
    every probability is a power of two, exactly an E4M3 value, and every
    product on the fp8 matrix core fits its exact range, so the kernel's
    roundings vanish and it must equal the oracle to fp32 accumulation.
    Two chunks of ragged length, one of them on another V scale, a re-basing
    of the running maximum (the second chunk's scores run higher), queries in
    a partial last tile."""
    H, n_q = 2, 300
    print(f"local_attn_fp8 exact grid H={H} n_q={n_q}", flush=True)
    # q: 4 in column 0 (its maximum), 1 in column 1, sparse +-1 in columns 3..14
    # k: 4 in column 2 (its maximum), k_0 in {0, 1}, k_1 in {-1, 0}, sparse +-1 in 3..14
    # so <q, k> = 4 k_0 + k_1 + (rare +-1 overlaps of the sparse columns)
    q = _grid(n_q, H, 11, 0)
    q[:, :, 1] = 1.0
    q[:, :, 2] = 0.0
    k1 = _grid(700, H, 12, 2)           # chunk 1: k_0 = 0, scores in {-1, 0} (and rare +-1)
    k1[:, :, 0] = 0.0
    k1[:, :, 1] = torch.where(torch.arange(700)[:, None] % 3 == 0, -1.0, 0.0).expand(700, H)
    k2 = _grid(333, H, 13, 2)           # chunk 2: k_0 = 1 on a third of the keys (scores up to 4 and 5)
    k2[:, :, 0] = torch.where(torch.arange(333)[:, None] % 3 == 1, 1.0, 0.0).expand(333, H)
    k2[:, :, 1] = 0.0
    for t in (q, k1, k2):
        t[:, :, 15:] = 0.0
    v1 = _grid(700, H, 14, 5, density=0.5)
    v2 = _grid(333, H, 15, 6, density=0.5) * 0.25   # V on another scale (2^-8)
    dev = lambda t: t.to(DEV, torch.bfloat16)  # noqa: E731
    scale = float(np.float32(math.log(2.0)))
    og, lg, ro, rl, qh, kh, vh = _run(dev(q), [(dev(k1), dev(v1)), (dev(k2), dev(v2))], scale)
    s = np.einsum("qhd,khd->qhk", qh, kh)
    assert np.all(np.abs(s - np.round(s)) == 0) and s.min() >= -3 and s.max() <= 6, (s.min(), s.max())
    assert s[:, :, 700:].max() - s[:, :, :700].max() > 3  # the second chunk re-bases the running maximum
    assert rel(og, ro) <= 1e-5, rel(og, ro)
    assert np.abs(lg - rl).max() <= 1e-5 * np.abs(rl).max() + 1e-6


@pytest.mark.parametrize("H,n_q,chunks,out_dtype", [
    (2, 300, (700, 333), torch.float32),          # ragged chunks, a partial query tile
    (3, 257, (64, 1, 65, 0, 129), torch.float32), # tile-edge and empty chunks, 5 segments
    (1, 40, (5000,), torch.bfloat16),             # one long chunk, bf16 output
    (4, 100, (31,) * 8, torch.float16),           # 8 segments, f16 output
    (2, 70, (100,) * 40 + (65,) * 24, torch.float32),  # 64 segments (the limit), the F-Layer form
])
def test_local_attn_fp8_parity(H, n_q, chunks, out_dtype):
    print(f"local_attn_fp8 H={H} n_q={n_q} chunks={chunks} -> {out_dtype}", flush=True)
    q = synth.normal((n_q, H, 128), 310, DEV, dtype=torch.bfloat16)
    kv = [(synth.normal((n, H, 128), 311 + i, DEV, dtype=torch.bfloat16),
           synth.normal((n, H, 128), 411 + i, DEV, dtype=torch.bfloat16)) for i, n in enumerate(chunks)]
    scale = 128 ** -0.5
    og, lg, ro, rl, qh, kh, vh = _run(q, kv, scale, out_dtype=out_dtype)
    pred = _predicted_var(qh, kh, vh, scale, np.arange(n_q))
    err2 = float(((og - ro) ** 2).sum())
    # 16-bit outputs add one rounding of the result (2^-9 for bf16, 2^-12 f16 relative, variance /3)
    u = {torch.float32: 0.0, torch.bfloat16: 2.0 ** -9, torch.float16: 2.0 ** -12}[out_dtype]
    pred += u * u / 3.0 * float((ro ** 2).sum())
    print(f"  err^2 {err2:.3e}, predicted {pred:.3e} (ratio {err2 / max(pred, 1e-300):.3f}); rel-L2 {rel(og, ro):.3e}",
          flush=True)
    assert err2 <= 3.0 * pred
    assert np.abs(lg - rl).max() <= math.log1p(2.0 ** -4)  # the sum of rounded p within 2^-4 of the exact one


def test_local_attn_fp8_no_keys():
    H, n_q = 2, 70
    q = synth.normal((n_q, H, 128), 320, DEV, dtype=torch.bfloat16)
    qc, qs = K().ispa_quantize_q_fp8(q)
    for chunks in ([], [K().ispa_quantize_kv_fp8(q[:0], q[:0])]):
        o, lse = K().ispa_local_attn_fp8(qc, qs, chunks, want_lse=True)
        torch.cuda.synchronize()
        assert not h64(o).any()
        assert np.all(np.isneginf(h64(lse)))


def test_local_attn_fp8_wan13b_shape_sampled():
    """The post-switch L-Layer at Wan-1.3B size: 4680 queries, 12 heads,
    sink + current chunk (2 x 4680 keys), in the launch the benchmark times;
    64 sampled query rows, every head, against the oracle."""
    H, T = 12, 4680
    print(f"local_attn_fp8 Wan-1.3B H={H} n_q={T} keys=2x{T}", flush=True)
    q = synth.normal((T, H, 128), 330, DEV, dtype=torch.bfloat16)
    kv = [(synth.normal((T, H, 128), 331 + i, DEV, dtype=torch.bfloat16),
           synth.normal((T, H, 128), 431 + i, DEV, dtype=torch.bfloat16)) for i in range(2)]
    rows = np.unique(np.linspace(0, T - 1, 64).astype(int))
    scale = 128 ** -0.5
    og, lg, ro, rl, qh, kh, vh = _run(q, kv, scale, rows=rows)
    pred = _predicted_var(qh, kh, vh, scale, rows)
    err2 = float(((og - ro) ** 2).sum())
    print(f"  err^2 {err2:.3e}, predicted {pred:.3e} (ratio {err2 / pred:.3f}); rel-L2 {rel(og, ro):.3e}", flush=True)
    assert err2 <= 3.0 * pred
    assert np.abs(lg - rl).max() <= math.log1p(2.0 ** -4)


def test_local_attn_fp8_proj_matches_its_parts():
    """The fused post-switch call (fp8 attention then W8A8 projection) equals
    the two calls it combines: ispa_local_attn_fp8 into fp32, then
    ispa_w8a8_linear with the same weight codes, bit for bit."""
    H, n_q, D = 12, 600, 1536
    print(f"local_attn_fp8_proj H={H} n_q={n_q}", flush=True)
    k8 = K()
    q = synth.normal((n_q, H, 128), 340, DEV, dtype=torch.bfloat16)
    kv = [(synth.normal((n, H, 128), 341 + i, DEV, dtype=torch.bfloat16),
           synth.normal((n, H, 128), 441 + i, DEV, dtype=torch.bfloat16)) for i, n in enumerate((900, 600))]
    chunks = [k8.ispa_quantize_kv_fp8(k, v) for k, v in kv]
    w = synth.normal((D, D), 342, DEV, std=D ** -0.5, dtype=torch.bfloat16)
    wc, ws = k8.ispa_quantize_w_fp8(w)
    y = k8.ispa_local_attn_fp8_proj(q, chunks, wc, ws, out_dtype=torch.float32)
    qc, qs = k8.ispa_quantize_q_fp8(q)
    o, _ = k8.ispa_local_attn_fp8(qc, qs, chunks)
    y2 = k8.ispa_w8a8_linear(o.reshape(n_q, D), wc, ws, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


def test_stream_post_uses_fp8_attention():
    """IspaStream after quantize_attention: an L-Layer's post-switch output
    equals, bit for bit, ispa_local_attn_fp8_proj over its sink and current
    chunk with its W + dW codes, and an F-Layer's the same call over all its
    chunks (each quantised on its own) with W's codes; with
    quantize_local_attention the F-Layer keeps bf16 attention with the W8A8
    projection (ispa_local_attn_proj_fp8 over all its keys)."""
    from kv_cache_absorption_amd.stream import IspaStream
    k8 = K()
    H, d, T, N = 4, 128, 300, 2
    D = H * d
    print(f"stream fp8 post H={H} T={T}", flush=True)
    W = synth.normal((N, D, D), 350, DEV, std=D ** -0.5, dtype=torch.bfloat16)
    w_eff = W + synth.normal((N, D, D), 351, DEV, std=1e-3, dtype=torch.bfloat16)
    kv = {c: (synth.normal((T, H, d), 360 + c, DEV, dtype=torch.bfloat16),
              synth.normal((T, H, d), 370 + c, DEV, dtype=torch.bfloat16)) for c in range(5)}
    q = synth.normal((T, H, d), 380, DEV, dtype=torch.bfloat16)
    for f_layers in (True, False):
        st = IspaStream(N, H, d, T, [2, 5], DEV, with_stats=False)
        st.W = W
        st.adopt_switch([1, 0], w_eff)
        for layer in range(N):
            for c in range(3):
                if layer == 1 or c == 0:
                    st.write_kv(layer, c, *kv[c])
        st.quantize_projections()
        if f_layers:
            st.quantize_attention()
        else:
            st.quantize_local_attention()
        for c in (3, 4):  # two post-switch steps: the F-Layer's chunks are quantised as they are first read
            for layer in range(N):
                st.write_kv(layer, c, *kv[c])
            y0 = st.post(0, c, q).clone()
            y1 = st.post(1, c, q).clone()
            chunks = [k8.ispa_quantize_kv_fp8(*kv[0]), k8.ispa_quantize_kv_fp8(*kv[c])]
            ref0 = k8.ispa_local_attn_fp8_proj(q, chunks, st.wq[0], st.wq_scale[0], out_dtype=torch.bfloat16)
            if f_layers:
                all8 = [k8.ispa_quantize_kv_fp8(*kv[i]) for i in range(c + 1)]
                ref1 = k8.ispa_local_attn_fp8_proj(q, all8, st.wq[1], st.wq_scale[1], out_dtype=torch.bfloat16)
            else:
                ref1 = k8.ispa_local_attn_proj_fp8(q, [(torch.cat([kv[i][0] for i in range(c + 1)]),
                                                        torch.cat([kv[i][1] for i in range(c + 1)]))],
                                                   st.wq[1], st.wq_scale[1], out_dtype=torch.bfloat16)
            torch.cuda.synchronize()
            assert torch.equal(y0, ref0)
            assert torch.equal(y1, ref1)


def test_stream_quantised_after_warmup_and_switch():
    """The quantised post-switch path entered from a real warmup and switch
    (the order the video benchmark uses): after switch + eviction,
    quantize_projections holds the codes of W + dW for the L-Layer and of W
    for the F-Layer (bit for bit as ispa_quantize_w_fp8), and every post()
    equals ispa_local_attn_fp8_proj over the chunks the layer keeps (the
    L-Layer: its sink, kept by the eviction, and the current chunk)."""
    from kv_cache_absorption_amd.stream import IspaStream
    k8 = K()
    H, d, T, N, warm = 2, 128, 300, 2, 3
    D = H * d
    print(f"stream warmup -> switch -> fp8 post H={H} T={T}", flush=True)
    W = [synth.normal((D, D), 390 + i, DEV, std=D ** -0.5, dtype=torch.bfloat16) for i in range(N)]
    kv = {(i, c): (synth.normal((T, H, d), 400 + 10 * i + c, DEV, dtype=torch.bfloat16),
                   synth.normal((T, H, d), 500 + 10 * i + c, DEV, dtype=torch.bfloat16))
          for i in range(N) for c in range(warm + 2)}
    qs = {(i, c): synth.normal((T, H, d), 600 + 10 * i + c, DEV, dtype=torch.bfloat16)
          for i in range(N) for c in range(warm + 2)}
    st = IspaStream(N, H, d, T, warm + 2, DEV)
    for i in range(N):
        st.set_w(i, W[i])
    for c in range(warm):
        for i in range(N):
            st.write_kv(i, c, *kv[i, c])
            st.warmup(i, c, qs[i, c])
    st.switch(1)
    st.quantize_projections()
    st.quantize_attention()
    loc = [i for i in range(N) if st.is_local_host[i]]
    assert len(loc) == 1
    for i in range(N):
        wc, wsc = k8.ispa_quantize_w_fp8(st.w_eff[i] if st.is_local_host[i] else W[i])
        torch.cuda.synchronize()
        assert torch.equal(st.wq[i], wc) and torch.equal(st.wq_scale[i], wsc)
    for c in range(warm, warm + 2):
        for i in range(N):
            st.write_kv(i, c, *kv[i, c])
            y = st.post(i, c, qs[i, c]).clone()
            held = [0, c] if st.is_local_host[i] else list(range(c + 1))
            chunks = [k8.ispa_quantize_kv_fp8(*kv[i, j]) for j in held]
            ref = k8.ispa_local_attn_fp8_proj(qs[i, c], chunks, st.wq[i], st.wq_scale[i],
                                              out_dtype=torch.bfloat16)
            torch.cuda.synchronize()
            assert torch.equal(y, ref), (i, c)
