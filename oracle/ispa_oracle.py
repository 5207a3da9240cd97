"""Plain fp64 CPU oracle of the ISPA hot path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check
and the CPU-baseline leg of the benchmark may import this module.  The HIP
library does not use it, and it imports nothing from the HIP library.

Every function restates a definition from the pages about "Towards
Memory-Efficient Autoregressive Video Generation via Instance-Specific
Parametric Absorption" (arXiv 2607.00712).  Short names for the pages:

* EN review  -- the English papernotes review ("Key Designs" 1-3, "A Worked
  Example", "Loss & Training", the Table 2 excerpts under "Main Results"
  and "Ablation Study").
* ZH review  -- the Chinese papernotes review (same structure, "关键设计").
* DE summary -- the gist.science technical summary, section 2 "Methodik":
  the printed objective and the printed closed form for Delta W.
* gptget     -- the gptget.net summary ("Methodology", ZH "Methodology").

Everything is float64 on whatever the inputs hold (bf16 inputs are decoded
exactly).  Steps that are a plain library primitive (a matrix product, an
exponential, a sort) use numpy for that step only; nothing is blocked, fused
or reordered beyond the definition.  Where the pages leave a step open the
docstring states the reading taken.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "as_f64",
    "group_attention",
    "lse_merge",
    "dual_stream_attention",
    "residual_target",
    "accumulate_stats",
    "accumulate_gram",
    "stats_from_gram",
    "ridge_lambda",
    "cholesky_lower",
    "forward_substitution",
    "backward_substitution",
    "solve_dw",
    "epsilon_from_stats",
    "epsilon_direct",
    "select_layers",
    "local_attn_proj",
    "stream_groups",
    "kv_bytes_retained",
    "remaining_kv_fraction",
    "stream_groups_kept",
    "E4M3_MAX",
    "e4m3_decode",
    "e4m3_encode",
    "quantize_rows_e4m3",
    "quantize_weight_e4m3",
    "w8a8_linear",
    "local_attn_proj_w8a8",
    "pow2_scale",
    "quantize_rows_e4m3_pow2",
    "quantize_chunk_e4m3",
    "quantize_heads_e4m3",
    "attention_fp8",
]


def as_f64(x) -> np.ndarray:
    """Decode any array-like (numpy, or a CPU torch tensor of any float
    dtype including bfloat16) to a float64 numpy array, exactly."""
    if hasattr(x, "detach"):  # torch tensor: widen on the torch side first
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Attention of one key group, and the log-sum-exp merge
# ---------------------------------------------------------------------------

def group_attention(q, k, v, scale: float):
    """Softmax attention of every query over ONE group of keys, returning the
    value-weighted output and the group's log-sum-exp.

    EN review, Key Design 1 (ZH review, 关键设计 1): the same current query
    attends to each disjoint KV group, and each group returns its weighted
    value output together with the LSE of its softmax normalisation.

    q: [n_q, H, d]; k, v: [n_k, H, d].  Returns (o [n_q, H, d],
    lse [n_q, H]) with s_j = scale * <q, k_j>, lse = ln sum_j exp(s_j) and
    o = sum_j exp(s_j - lse) v_j.  An empty group gives o = 0, lse = -inf
    (its softmax mass is zero).
    """
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    n_q, H, d = q.shape
    n_k = k.shape[0]
    if n_k == 0:
        return np.zeros((n_q, H, d)), np.full((n_q, H), -np.inf)
    # scores per head: [H, n_q, n_k]  (matrix product primitive)
    s = scale * np.matmul(q.transpose(1, 0, 2), k.transpose(1, 2, 0))
    m = s.max(axis=2, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=2, keepdims=True)
    o = np.matmul(e / l, v.transpose(1, 0, 2))  # [H, n_q, d]
    lse = (m + np.log(l))[:, :, 0]  # [H, n_q]
    return o.transpose(1, 0, 2), lse.T


def lse_merge(o_parts, lse_parts):
    """Combine per-group attention results into attention over their union.

    EN review, Key Design 1: the full activation is recovered from the two
    branches with weights given by their normalisation constants, not by a
    plain average.  Written out: lse = ln sum_p exp(lse_p) and
    o = sum_p exp(lse_p - lse) o_p.  Parts with lse = -inf carry no mass;
    if every part is empty the result is o = 0, lse = -inf.

    Returns (o_full, lse_full, a0, delta) where a0 = o_parts[0] (the local
    activation A_loc when part 0 is the local group) and
    delta = o_full - a0 (A_full - A_loc).
    """
    os_ = [as_f64(o) for o in o_parts]
    ls_ = [as_f64(l) for l in lse_parts]
    stack_l = np.stack(ls_)  # [P, n_q, H]
    m = stack_l.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    tot = np.zeros_like(m)
    for l in ls_:
        tot += np.where(np.isfinite(l), np.exp(l - m_safe), 0.0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, tot, 1.0)), -np.inf)
    o = np.zeros_like(os_[0])
    for op, l in zip(os_, ls_):
        wgt = np.where(np.isfinite(l) & finite, np.exp(l - np.where(finite, lse, 0.0)), 0.0)
        o += wgt[..., None] * op
    return o, lse, os_[0], o - os_[0]


def dual_stream_attention(q, k_loc, v_loc, k_hist, v_hist, scale: float):
    """Dual-stream warmup attention (EN review, Key Design 1; DE summary,
    "Dual-Stream Warmup"): attention over the local group and the history
    group separately, then the LSE merge.  Returns a dict with o_loc,
    lse_loc, o_hist, lse_hist, a_full, lse_full, a_loc and delta."""
    o_l, l_l = group_attention(q, k_loc, v_loc, scale)
    o_h, l_h = group_attention(q, k_hist, v_hist, scale)
    a_full, lse_full, a_loc, delta = lse_merge([o_l, o_h], [l_l, l_h])
    return dict(o_loc=o_l, lse_loc=l_l, o_hist=o_h, lse_hist=l_h,
                a_full=a_full, lse_full=lse_full, a_loc=a_loc, delta=delta)


# ---------------------------------------------------------------------------
# Regression statistics
# ---------------------------------------------------------------------------

def residual_target(a_loc, a_full, w):
    """R = (A_full - A_loc) W (EN review, Key Design 2, the residual
    equation).  Rows are tokens; W is [D_in, D_out] acting on row vectors."""
    return (as_f64(a_full) - as_f64(a_loc)) @ as_f64(w)


def accumulate_stats(a_loc, delta_a, w):
    """One step's contribution to the sufficient statistics.

    EN review, Key Design 2: activation outer products and activation-residual
    cross statistics can be accumulated during the forward passes.  With rows
    a_i of A_loc (one per query token, all heads concatenated, width D) and
    r_i = delta_i W the matching residual rows:
        G = sum_i a_i a_i^T = A_loc^T A_loc       (D x D)
        C = sum_i a_i r_i^T = A_loc^T R           (D x D)
        r2 = sum_i |r_i|^2  = ||R||_F^2
    Statistics are sums over rows (not means); the warmup total is the sum of
    the per-step contributions.  Returns (G, C, r2).
    """
    a = as_f64(a_loc)
    r = as_f64(delta_a) @ as_f64(w)
    return a.T @ a, a.T @ r, float(np.sum(r * r))


def accumulate_gram(a_loc, delta_a):
    """One step's contribution to the statistics in the grouping of the
    printed closed form.

    DE summary, Methodik: Delta W = (A_loc^T A_loc + lambda I)^-1
    A_loc^T (A_full - A_loc) W.  The factor A_loc^T (A_full - A_loc) does
    not involve W, so it can be summed over the warmup rows on its own and
    multiplied by W once at the switch; the same holds for the residual
    energy, ||(A_full - A_loc) W||_F^2 = <dA^T dA, W W^T>.  With rows a_i of
    A_loc and d_i of A_full - A_loc:
        G = sum_i a_i a_i^T = A_loc^T A_loc      (D x D)
        M = sum_i a_i d_i^T = A_loc^T dA         (D x D)
        H = sum_i d_i d_i^T = dA^T dA            (D x D)
    Sums over rows; the warmup total is the sum of the per-step
    contributions.  Returns (G, M, H)."""
    a, dl = as_f64(a_loc), as_f64(delta_a)
    return a.T @ a, a.T @ dl, dl.T @ dl


def stats_from_gram(G, M, H, w):
    """The statistics the solve takes, from the grouped sums of
    accumulate_gram: G unchanged, C = M W (= A_loc^T R) and
    r2 = <H, W W^T> = trace(W^T H W) (= ||R||_F^2), with R = dA W the
    residual target (EN review, Key Design 2).  Returns (G, C, r2)."""
    G, M, H, w = as_f64(G), as_f64(M), as_f64(H), as_f64(w)
    return G, M @ w, float(np.sum(H * (w @ w.T)))


# ---------------------------------------------------------------------------
# Ridge solve
# ---------------------------------------------------------------------------

def ridge_lambda(G, lambda_abs: float, lambda_rel: float) -> float:
    """Regularisation weight.  The pages give lambda = 0.001 (EN review, Loss &
    Training) without saying whether G is a sum or a mean; the reading taken
    is lambda = lambda_abs + lambda_rel * tr(G) / D, with lambda_rel = 1e-3 and
    lambda_abs = 0 for the workloads (the relative form makes Delta W the same
    for summed or averaged statistics)."""
    G = as_f64(G)
    return float(lambda_abs + lambda_rel * np.trace(G) / G.shape[0])


def cholesky_lower(a):
    """Lower-triangular L with L L^T = a, column by column (Cholesky-Crout).

    Returns (L, info): info = 0 on success, else the 1-based index of the
    first pivot that is not positive (L is then incomplete)."""
    a = as_f64(a)
    n = a.shape[0]
    L = np.zeros_like(a)
    for j in range(n):
        piv = a[j, j] - np.dot(L[j, :j], L[j, :j])
        if not piv > 0.0:
            return L, j + 1
        L[j, j] = math.sqrt(piv)
        if j + 1 < n:
            L[j + 1:, j] = (a[j + 1:, j] - L[j + 1:, :j] @ L[j, :j]) / L[j, j]
    return L, 0


def forward_substitution(L, B):
    """Solve L Y = B for lower-triangular L, one row at a time."""
    L, B = as_f64(L), as_f64(B)
    Y = np.zeros_like(B)
    for i in range(L.shape[0]):
        Y[i] = (B[i] - L[i, :i] @ Y[:i]) / L[i, i]
    return Y


def backward_substitution(L, Y):
    """Solve L^T X = Y for lower-triangular L, one row at a time."""
    L, Y = as_f64(L), as_f64(Y)
    n = L.shape[0]
    X = np.zeros_like(Y)
    for i in range(n - 1, -1, -1):
        X[i] = (Y[i] - L[i + 1:, i] @ X[i + 1:]) / L[i, i]
    return X


def solve_dw(G, C, lam: float):
    """Closed-form ridge absorption.

    DE summary, Methodik: Delta W minimises
    ||A_loc (W + Delta W) - A_full W||^2 + lambda ||Delta W||^2, and the
    printed closed form is Delta W = (A_loc^T A_loc + lambda I)^-1
    A_loc^T (A_full - A_loc) W = (G + lambda I)^-1 C.  The pages call this a
    single D x D inversion (EN review, Key Design 2); it is solved here as
    (G + lambda I) = L L^T followed by two triangular solves, which gives the
    same matrix without forming the inverse.

    Returns (dW, info); info > 0 means G + lambda I was not positive
    definite (first failing pivot, 1-based) and dW is NaN.
    """
    G, C = as_f64(G), as_f64(C)
    A = G + lam * np.eye(G.shape[0])
    L, info = cholesky_lower(A)
    if info:
        return np.full_like(C, np.nan), info
    return backward_substitution(L, forward_substitution(L, C)), 0


def epsilon_from_stats(G, C, r2: float, dW) -> float:
    """Reconstruction error from the statistics.

    EN review, Key Design 2 defines eps = ||A_loc (W + dW) - A_full W||_F^2 =
    ||A_loc dW - R||_F^2.  Expanding the square over the warmup rows:
    eps = r2 - 2 <dW, C> + <dW, G dW>, with the unregularised G (the penalty
    term is not part of eps)."""
    G, C, dW = as_f64(G), as_f64(C), as_f64(dW)
    return float(r2 - 2.0 * np.sum(dW * C) + np.sum(dW * (G @ dW)))


def epsilon_direct(a_loc, a_full, w, dW) -> float:
    """eps straight from its definition on stored rows (EN review, Key
    Design 2): ||A_loc (W + dW) - A_full W||_F^2."""
    a_loc, a_full, w, dW = as_f64(a_loc), as_f64(a_full), as_f64(w), as_f64(dW)
    e = a_loc @ (w + dW) - a_full @ w
    return float(np.sum(e * e))


# ---------------------------------------------------------------------------
# Layer selection
# ---------------------------------------------------------------------------

def select_layers(eps, K: int):
    """Instance-specific layer selection (EN review, Key Design 3): sort the N
    layers by increasing eps and take the K lowest as L-Layers.  Ties go to
    the lower layer index (stable sort).  A NaN eps is an error.

    Returns (selected [K] int32 in ascending-eps order, is_local [N] uint8,
    status): status 0 on success, 1 if any eps is NaN (outputs then zero)."""
    eps = [float(e) for e in as_f64(eps).ravel()]
    N = len(eps)
    if any(math.isnan(e) for e in eps):
        return np.zeros(K, np.int32), np.zeros(N, np.uint8), 1
    order = sorted(range(N), key=lambda i: (eps[i], i))
    sel = np.array(order[:K], dtype=np.int32)
    is_local = np.zeros(N, np.uint8)
    is_local[sel] = 1
    return sel, is_local, 0


# ---------------------------------------------------------------------------
# Post-switch layers
# ---------------------------------------------------------------------------

def local_attn_proj(q, k, v, w_proj, scale: float):
    """Post-switch layer output (EN review, Key Design 2 and 3; DE summary,
    "Speichereffiziente Inferenz"): attention over the retained keys, then the
    output projection.  An L-Layer passes its local keys (sink + current) and
    W + Delta W; an F-Layer passes all its keys and W.  Returns [n_q, D]."""
    o, _ = group_attention(q, k, v, scale)
    n_q = o.shape[0]
    return o.reshape(n_q, -1) @ as_f64(w_proj)


# ---------------------------------------------------------------------------
# W8A8 post-switch projection
#
# The pages report a 1.86x overall speed-up when ISPA is combined with W8A8
# post-training quantisation (EN review, Key Findings, the Figure 7 item; DE
# summary, section 4 "Experimentelle Ergebnisse", the acceleration item), and
# give no scheme: no format, granularity or scale rule.  The reading taken
# here is the plainest W8A8 for the one linear layer the method changes, the
# output projection with W (F-Layers) or W + Delta W (L-Layers): 8-bit
# floating point (OCP FP8 E4M3) for both operands, one symmetric scale per
# activation row (token) and per weight output column, fp32 accumulation.
# Attention itself stays in its own precision.
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Values of OCP FP8 E4M3 codes: 1 sign bit, 4 exponent bits with bias 7,
    3 mantissa bits.  Exponent field 0 holds subnormals m * 2^-9; codes 0x7f
    and 0xff are NaN; there is no infinity, so the largest finite magnitude
    is 1.75 * 2^8 = 448."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(c >> 7, -mag, mag)


_E4M3_POS = e4m3_decode(np.arange(0x7F, dtype=np.uint8))  # codes 0x00..0x7e, increasing


def e4m3_encode(x) -> np.ndarray:
    """E4M3 code of each value with |x| <= 448: the nearest finite magnitude,
    a tie going to the even code (even mantissa), the sign from the sign of x.
    A magnitude that rounds to zero is encoded as +0 (0x00), whatever the sign
    of x: the scheme has a single zero code."""
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any() or (np.abs(x) > E4M3_MAX).any():
        raise ValueError("e4m3_encode: values must be finite and within +-448")
    a = np.abs(x)
    hi = np.minimum(np.searchsorted(_E4M3_POS, a, side="left"), len(_E4M3_POS) - 1)  # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)), hi, lo)
    code = np.where((x < 0) & (code != 0), code | 0x80, code)
    return code.astype(np.uint8)


def quantize_rows_e4m3(x):
    """Symmetric per-row E4M3 quantisation (the scheme stated above).

    Row i: amax_i = max_k |x_ik|, scale_i = amax_i / 448 and
    code_ik = E4M3(clamp(x_ik / scale_i, -448, 448)).  The two divisions are
    fp32 operations rounded to nearest: the codes are integers decided by
    floating point, so the oracle takes the decision in the kernel's
    precision.  Inputs are fp32 or 16-bit values (exact in fp32).  A row of
    zeros gets scale 0 and zero codes.  Returns (codes uint8, scales fp32)."""
    x32 = np.asarray(as_f64(x), dtype=np.float32)
    if x32.ndim != 2:
        raise ValueError("quantize_rows_e4m3: 2-D input")
    amax = np.max(np.abs(x32), axis=1) if x32.shape[1] else np.zeros(x32.shape[0], np.float32)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    y = (x32 / safe[:, None]).astype(np.float32)
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    codes = np.where(scale[:, None] > 0, e4m3_encode(y), 0).astype(np.uint8)
    return codes, scale


def quantize_weight_e4m3(w):
    """W [D_in, D_out] -> (codes [D_out, D_in], scales [D_out]): one scale per
    output column, the codes of a column stored as a row (input index
    contiguous)."""
    return quantize_rows_e4m3(as_f64(w).T)


def w8a8_linear(x, w_codes, w_scales):
    """y = (x quantised per row) times (W quantised per output column), in
    fp64 on the dequantised operands: y_ij = sx_i sw_j sum_k dec(qx_ik)
    dec(qw_jk).  x [n, D_in]; w_codes [D_out, D_in]; returns [n, D_out]."""
    qx, sx = quantize_rows_e4m3(x)
    xa = e4m3_decode(qx) * sx.astype(np.float64)[:, None]
    wb = e4m3_decode(w_codes) * np.asarray(w_scales, dtype=np.float64)[:, None]
    return xa @ wb.T


def local_attn_proj_w8a8(q, k, v, w_proj, scale: float):
    """Post-switch layer output with the W8A8 projection: attention over the
    retained keys (fp64, as local_attn_proj), its output rounded to fp32 (the
    attention's output type) and quantised per token, times W quantised per
    output column.  Returns [n_q, D_out]."""
    o, _ = group_attention(q, k, v, scale)
    o32 = o.reshape(o.shape[0], -1).astype(np.float32)
    wq, ws = quantize_weight_e4m3(w_proj)
    return w8a8_linear(o32, wq, ws)


# ---------------------------------------------------------------------------
# Quantised local attention (the post-switch L-Layer on the fp8 matrix core)
#
# The pages name W8A8 quantisation beside ISPA and nothing more (EN review,
# Key Findings, the Figure 7 item).  The reading here for the attention
# itself: its three operands in OCP FP8 E4M3 with symmetric scales, K and V
# once per cache chunk and head (a chunk's rows are written once and then
# only read, so they are quantised when written), Q per query row and head;
# the attention is then the exact softmax attention of the dequantised
# operands.  Each scale is a power of two, the smallest 2^e with
# amax <= 448 * 2^e (the shared-exponent convention of the OCP microscaling
# formats, whose E8M0 block scales the fp8 matrix core applies itself), so
# x / scale is exact and each code is the E4M3 rounding of it; a group of
# zeros takes scale 1 and zero codes.
# ---------------------------------------------------------------------------

def pow2_scale(amax):
    """The smallest power of two 2^e with amax <= 448 * 2^e and e >= -126
    (the least normal fp32 power of two, so that every scale is a normal
    fp32 number), per element of amax (fp32 magnitudes); 1.0 where amax is
    0.  Decided by exact comparisons in fp64 (448 * 2^e and every fp32 value
    are exact there)."""
    a = np.asarray(amax, dtype=np.float64)
    out = np.ones(a.shape, dtype=np.float64)
    nz = a > 0
    if nz.any():
        e = np.ceil(np.log2(a[nz] / E4M3_MAX)).astype(np.int64)
        # log2 is rounded: step to the exact smallest e
        e = np.where(a[nz] <= E4M3_MAX * np.ldexp(1.0, e - 1), e - 1, e)
        e = np.where(a[nz] > E4M3_MAX * np.ldexp(1.0, e), e + 1, e)
        out[nz] = np.ldexp(1.0, np.maximum(e, -126))
    return out.astype(np.float32)


def quantize_rows_e4m3_pow2(x):
    """Per-row E4M3 quantisation with power-of-two scales: scale_i =
    pow2_scale(max_k |x_ik|), code_ik = E4M3(x_ik / scale_i) (the quotient is
    exact and within +-448).  Returns (codes uint8, scales fp32)."""
    x32 = np.asarray(as_f64(x), dtype=np.float32)
    if x32.ndim != 2:
        raise ValueError("quantize_rows_e4m3_pow2: 2-D input")
    amax = np.max(np.abs(x32), axis=1) if x32.shape[1] else np.zeros(x32.shape[0], np.float32)
    scale = pow2_scale(amax)
    y = x32.astype(np.float64) / scale.astype(np.float64)[:, None]
    return e4m3_encode(y), scale


def quantize_chunk_e4m3(x):
    """One cache chunk [n, H, d] -> (codes uint8 [n, H, d], scales fp32 [H]):
    one symmetric scale per head over all n x d values of the chunk."""
    x32 = np.asarray(as_f64(x), dtype=np.float32)
    n, H, d = x32.shape
    per_head = x32.transpose(1, 0, 2).reshape(H, n * d)
    codes, scales = quantize_rows_e4m3_pow2(per_head)
    return codes.reshape(H, n, d).transpose(1, 0, 2).copy(), scales


def quantize_heads_e4m3(q):
    """Queries [n, H, d] -> (codes uint8 [n, H, d], scales fp32 [n, H]): one
    scale per query row and head."""
    q32 = np.asarray(as_f64(q), dtype=np.float32)
    n, H, d = q32.shape
    codes, scales = quantize_rows_e4m3_pow2(q32.reshape(n * H, d))
    return codes.reshape(n, H, d), scales.reshape(n, H)


def attention_fp8(q, k_chunks, v_chunks, scale: float):
    """Attention of every query over the keys of the given chunks with the
    operands quantised as stated above: Q per (row, head), each chunk's K
    and V per head; the softmax attention of the dequantised values in fp64.
    k_chunks, v_chunks: lists of [n_c, H, d].  Returns (o [n_q, H, d],
    lse [n_q, H])."""
    qc, sq = quantize_heads_e4m3(q)
    q_hat = e4m3_decode(qc) * sq.astype(np.float64)[:, :, None]
    ks, vs = [], []
    for k, v in zip(k_chunks, v_chunks):
        kc, sk = quantize_chunk_e4m3(k)
        vc, sv = quantize_chunk_e4m3(v)
        ks.append(e4m3_decode(kc) * sk.astype(np.float64)[None, :, None])
        vs.append(e4m3_decode(vc) * sv.astype(np.float64)[None, :, None])
    H, d = q_hat.shape[1], q_hat.shape[2]
    k_hat = np.concatenate(ks) if ks else np.zeros((0, H, d))
    v_hat = np.concatenate(vs) if vs else np.zeros((0, H, d))
    return group_attention(q_hat, k_hat, v_hat, scale)


# ---------------------------------------------------------------------------
# Key grouping and KV accounting
# ---------------------------------------------------------------------------

def stream_groups(c: int, chunk_tokens: int):
    """Key groups at chunk step c of a chunked stream (EN review, Overall
    Architecture and Key Design 1): the local group is the initial sink plus
    the current chunk, history is everything in between.

    Reading taken: chunk 0 is the sink; at c = 0 the local group is chunk 0
    alone and history is empty; at c >= 1 local = {chunk 0, chunk c} and
    history = chunks 1 .. c-1.  Returns (local, history) as lists of
    half-open token ranges (start, stop) into the layer's key sequence."""
    T = chunk_tokens
    if c == 0:
        return [(0, T)], []
    local = [(0, T), (c * T, (c + 1) * T)]
    hist = [(T, c * T)] if c >= 2 else []
    return local, hist


def stream_groups_kept(c: int, chunk_tokens: int, first_kept: int):
    """Key groups at chunk step c for a layer that holds its sink and the
    chunks first_kept .. c, and no history before first_kept.

    This is the state after re-entering warmup (EN review, Limitations: the
    method re-enters warmup after a major scene change to refresh the
    selection and the weight corrections; it gives no detector).  Reading
    taken: a layer re-enters warmup with the keys it still holds.  An F-Layer
    holds everything, so first_kept = 1 and the groups are those of
    stream_groups.  An L-Layer holds its sink and its last current chunk, so
    first_kept is that chunk's index.  Chunks arriving from then on are kept.
    Local = {sink, chunk c}, history = chunks first_kept .. c-1 (empty when
    c <= first_kept).  Ranges index the original key sequence, as in
    stream_groups."""
    T = chunk_tokens
    if first_kept < 1:
        raise ValueError("first_kept counts from chunk 1 (chunk 0 is the sink)")
    if c == 0:
        return [(0, T)], []
    local = [(0, T), (c * T, (c + 1) * T)]
    hist = [(first_kept * T, c * T)] if c > first_kept else []
    return local, hist


def kv_bytes_retained(n_keys_per_layer, D: int, bytes_per_elem: int = 2) -> int:
    """KV bytes held: K and V of width D for every retained key of every
    layer (EN review, Key Design 3: L-Layers keep sink and current entries,
    F-Layers keep their whole history)."""
    return int(sum(2 * int(n) * D * bytes_per_elem for n in n_keys_per_layer))


def remaining_kv_fraction(x: float, r: float) -> float:
    """Remaining KV relative to keeping every layer full, when a fraction x of
    the layers keep only a fraction r of their keys: 1 - x (1 - r).  (EN
    review, Key Design 3: ISPA-x converts K = xN layers; converted layers
    still keep sink and current entries.)"""
    return 1.0 - x * (1.0 - r)
