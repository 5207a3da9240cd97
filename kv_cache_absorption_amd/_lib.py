"""ctypes binding of libispa.

Thin marshalling only: every function takes torch tensors that live on the
GPU, allocates its outputs and workspace with torch, passes raw device
pointers and the current HIP stream to the C ABI declared in include/ispa.h,
and raises IspaError on a non-zero status.  All arithmetic happens in the
HIP kernels of libispa.so; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libispa.so")

ISPA_OK, ISPA_ERR_INVALID_ARG, ISPA_ERR_UNSUPPORTED, ISPA_ERR_WORKSPACE, ISPA_ERR_HIP = range(5)
ISPA_F32, ISPA_BF16, ISPA_F16 = 0, 1, 2
ISPA_MAX_SEGS = 8
ISPA_NOALLOC_SCRATCH_BYTES = 32 << 20

EXPORTED = [
    "ispa_version", "ispa_status_str", "ispa_last_error",
    "ispa_dual_attn_workspace_bytes", "ispa_dual_attn",
    "ispa_dual_attn_merge_workspace_bytes", "ispa_dual_attn_merge",
    "ispa_lse_merge",
    "ispa_accum_stats_workspace_bytes", "ispa_accum_stats",
    "ispa_gram_state_bytes", "ispa_accum_gram", "ispa_gram_finalize_workspace_bytes", "ispa_gram_finalize",
    "ispa_solve_dw_workspace_bytes", "ispa_solve_dw",
    "ispa_select_layers",
    "ispa_local_attn_proj_workspace_bytes", "ispa_local_attn_proj",
    "ispa_quantize_w_fp8_workspace_bytes", "ispa_quantize_w_fp8",
    "ispa_w8a8_linear_workspace_bytes", "ispa_w8a8_linear", "ispa_w8a8_linear_noalloc",
    "ispa_local_attn_proj_fp8_workspace_bytes", "ispa_local_attn_proj_fp8",
    "ispa_kv_fp8_bytes", "ispa_quantize_kv_fp8_workspace_bytes", "ispa_quantize_kv_fp8",
    "ispa_quantize_q_fp8", "ispa_local_attn_fp8",
    "ispa_local_attn_fp8_proj_workspace_bytes", "ispa_local_attn_fp8_proj",
]
ISPA_FP8_TILE_KEYS = 64
ISPA_MAX_SEGS_FP8 = 64

_DT = {torch.float32: ISPA_F32, torch.bfloat16: ISPA_BF16, torch.float16: ISPA_F16}
_TORCH_DT = {v: k for k, v in _DT.items()}


class IspaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libispa status {status}: {msg}")
        self.status = status


class Seg(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("n", ctypes.c_int64),
                ("k_stride", ctypes.c_int64), ("v_stride", ctypes.c_int64)]


class SegFp8(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p),
                ("v_scales", ctypes.c_void_p), ("n", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libispa.so (built in-tree by kv_cache_absorption_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run `python -m kv_cache_absorption_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
        f32, f64 = ctypes.c_float, ctypes.c_double
        segp = ctypes.POINTER(Seg)
        seg8p = ctypes.POINTER(SegFp8)
        sig = {
            "ispa_version": (i32, []),
            "ispa_status_str": (ctypes.c_char_p, [i32]),
            "ispa_last_error": (ctypes.c_char_p, []),
            "ispa_dual_attn_workspace_bytes": (sz, [i32, i64, i32, i32, segp, i32, segp, i32]),
            "ispa_dual_attn": (i32, [i32, i64, i32, i32, f32, vp, i64, segp, i32, segp, i32,
                                     vp, vp, vp, vp, vp, sz, vp]),
            "ispa_dual_attn_merge_workspace_bytes": (sz, [i32, i64, i32, i32, segp, i32, segp, i32]),
            "ispa_dual_attn_merge": (i32, [i32, i64, i32, i32, f32, vp, i64, segp, i32, segp, i32,
                                           vp, vp, i32, vp, vp, sz, vp]),
            "ispa_lse_merge": (i32, [i32, ctypes.POINTER(vp), ctypes.POINTER(vp), i64, i32, i32,
                                     vp, vp, vp, vp, i32, vp]),
            "ispa_accum_stats_workspace_bytes": (sz, [i32, i64, i32]),
            "ispa_accum_stats": (i32, [i32, i32, i64, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "ispa_gram_state_bytes": (sz, [i32]),
            "ispa_accum_gram": (i32, [i32, i64, i32, vp, vp, vp, vp]),
            "ispa_gram_finalize_workspace_bytes": (sz, [i32]),
            "ispa_gram_finalize": (i32, [i32, i32, vp, i64, vp, i32, i64, vp, vp, vp, i64, vp, sz, vp]),
            "ispa_solve_dw_workspace_bytes": (sz, [i32, i32]),
            "ispa_solve_dw": (i32, [i32, i32, vp, vp, vp, i64, f64, f64, vp, vp, vp, vp, i32, vp,
                                    vp, sz, vp]),
            "ispa_select_layers": (i32, [i32, i32, vp, vp, vp, vp, vp]),
            "ispa_local_attn_proj_workspace_bytes": (sz, [i32, i64, i32, i32, segp, i32]),
            "ispa_local_attn_proj": (i32, [i32, i64, i32, i32, f32, vp, i64, segp, i32, vp, i32,
                                           vp, i32, vp, sz, vp]),
            "ispa_quantize_w_fp8_workspace_bytes": (sz, [i32, i32]),
            "ispa_quantize_w_fp8": (i32, [i32, i32, i32, vp, vp, vp, vp, sz, vp]),
            "ispa_w8a8_linear_workspace_bytes": (sz, [i64, i32]),
            "ispa_w8a8_linear": (i32, [i32, i64, i32, i32, vp, i64, vp, vp, vp, i32, vp, sz, vp]),
            "ispa_w8a8_linear_noalloc": (i32, [i32, i64, i32, i32, vp, i64, vp, vp, vp, i32, vp]),
            "ispa_local_attn_proj_fp8_workspace_bytes": (sz, [i64, i32, i32, segp, i32]),
            "ispa_local_attn_proj_fp8": (i32, [i64, i32, i32, f32, vp, i64, segp, i32, vp, vp, vp, i32,
                                               vp, sz, vp]),
            "ispa_kv_fp8_bytes": (sz, [i64, i32, i32]),
            "ispa_quantize_kv_fp8_workspace_bytes": (sz, [i64, i32, i32]),
            "ispa_quantize_kv_fp8": (i32, [i32, i64, i32, i32, vp, i64, vp, i64, vp, vp, vp, vp, vp, sz, vp]),
            "ispa_quantize_q_fp8": (i32, [i32, i64, i32, i32, vp, i64, vp, vp, vp]),
            "ispa_local_attn_fp8": (i32, [i64, i32, i32, f32, vp, vp, seg8p, i32, vp, i32, vp, vp]),
            "ispa_local_attn_fp8_proj_workspace_bytes": (sz, [i64, i32, i32]),
            "ispa_local_attn_fp8_proj": (i32, [i64, i32, i32, f32, i32, vp, i64, seg8p, i32, vp, vp, vp, i32,
                                               vp, sz, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def _check(status: int):
    if status != ISPA_OK:
        raise IspaError(status, lib().ispa_last_error().decode())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _segs(pairs, H: int, d: int):
    """[(k, v), ...] with k, v of shape [n, H, d] (rows may be strided) -> Seg array."""
    arr = (Seg * max(1, len(pairs)))()
    for i, (k, v) in enumerate(pairs):
        for t in (k, v):
            if t.dim() != 3 or t.shape[1] != H or t.shape[2] != d or t.stride(2) != 1 or t.stride(1) != d:
                raise ValueError("segments must be [n, H, d] with contiguous [H, d] rows")
        if k.shape[0] != v.shape[0]:
            raise ValueError("k and v of a segment differ in length")
        arr[i] = Seg(k.data_ptr(), v.data_ptr(), k.shape[0], k.stride(0), v.stride(0))
    return arr, len(pairs)


def _workspace(nbytes: int, device) -> torch.Tensor | None:
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _q_args(q: torch.Tensor):
    if q.dim() != 3 or q.stride(2) != 1 or q.stride(1) != q.shape[2]:
        raise ValueError("q must be [n_q, H, d] with contiguous [H, d] rows")
    return q.shape[0], q.shape[1], q.shape[2], q.stride(0)


# ---------------------------------------------------------------------------
def ispa_dual_attn(q, loc, hist, scale: float | None = None):
    """Dual-stream attention.  q [n_q, H, d]; loc / hist lists of (k, v)
    segments.  Returns (o_loc, lse_loc, o_hist, lse_hist), fp32."""
    n_q, H, d, qs = _q_args(q)
    dt = _DT[q.dtype]
    scale = d ** -0.5 if scale is None else scale
    ls, nl = _segs(loc, H, d)
    hs, nh = _segs(hist, H, d)
    dev = q.device
    o_loc = torch.empty((n_q, H, d), dtype=torch.float32, device=dev)
    o_hist = torch.empty_like(o_loc)
    lse_loc = torch.empty((n_q, H), dtype=torch.float32, device=dev)
    lse_hist = torch.empty_like(lse_loc)
    L = lib()
    wsb = L.ispa_dual_attn_workspace_bytes(dt, n_q, H, d, ls, nl, hs, nh)
    ws = _workspace(wsb, dev)
    _check(L.ispa_dual_attn(dt, n_q, H, d, scale, q.data_ptr(), qs, ls, nl, hs, nh,
                            o_loc.data_ptr(), lse_loc.data_ptr(), o_hist.data_ptr(),
                            lse_hist.data_ptr(), _ptr(ws), wsb, _stream(dev)))
    return o_loc, lse_loc, o_hist, lse_hist


def ispa_dual_attn_merge(q, loc, hist, scale: float | None = None, out_dtype=torch.float16,
                         want_lse=True):
    """Dual-stream attention and the LSE merge in one call.  Returns (a_loc,
    delta, lse_full): a_loc = o_loc and delta = o_full - o_loc as [n_q, D] of
    out_dtype, lse_full fp32 [n_q, H] (None unless requested)."""
    n_q, H, d, qs = _q_args(q)
    dt = _DT[q.dtype]
    scale = d ** -0.5 if scale is None else scale
    ls, nl = _segs(loc, H, d)
    hs, nh = _segs(hist, H, d)
    dev = q.device
    a_loc = torch.empty((n_q, H * d), dtype=out_dtype, device=dev)
    delta = torch.empty_like(a_loc)
    lse = torch.empty((n_q, H), dtype=torch.float32, device=dev) if want_lse else None
    L = lib()
    wsb = L.ispa_dual_attn_merge_workspace_bytes(dt, n_q, H, d, ls, nl, hs, nh)
    ws = _workspace(wsb, dev)
    _check(L.ispa_dual_attn_merge(dt, n_q, H, d, scale, q.data_ptr(), qs, ls, nl, hs, nh,
                                  a_loc.data_ptr(), delta.data_ptr(), _DT[out_dtype], _ptr(lse),
                                  _ptr(ws), wsb, _stream(dev)))
    return a_loc, delta, lse


def ispa_lse_merge(o_parts: Sequence[torch.Tensor], lse_parts: Sequence[torch.Tensor],
                   out_dtype=torch.float32, want_full=True, want_a0=True, want_delta=True):
    """n-way LSE merge.  Returns (o_full, lse_full, a0, delta); a0/delta are
    [n_q, D] of out_dtype, any of them None when not requested."""
    o0 = o_parts[0]
    n_q, H, d = o0.shape
    dev = o0.device
    for t in list(o_parts) + list(lse_parts):
        if not t.is_contiguous() or t.dtype != torch.float32:
            raise ValueError("parts must be contiguous fp32")
    P = len(o_parts)
    op = (ctypes.c_void_p * P)(*[t.data_ptr() for t in o_parts])
    lp = (ctypes.c_void_p * P)(*[t.data_ptr() for t in lse_parts])
    o_full = torch.empty((n_q, H, d), dtype=torch.float32, device=dev) if want_full else None
    lse_full = torch.empty((n_q, H), dtype=torch.float32, device=dev) if want_full else None
    a0 = torch.empty((n_q, H * d), dtype=out_dtype, device=dev) if want_a0 else None
    delta = torch.empty((n_q, H * d), dtype=out_dtype, device=dev) if want_delta else None
    _check(lib().ispa_lse_merge(P, op, lp, n_q, H, d, _ptr(o_full), _ptr(lse_full), _ptr(a0),
                                _ptr(delta), _DT[out_dtype], _stream(dev)))
    return o_full, lse_full, a0, delta


def ispa_accum_stats(a_loc, delta_a, w, G, C, r2):
    """In place: G (upper triangle) += a^T a, C += a^T (delta W), r2 += ||delta W||^2."""
    n, D = a_loc.shape
    for t in (a_loc, delta_a, w, G, C, r2):
        if not t.is_contiguous():
            raise ValueError("accum_stats operands must be contiguous")
    if G.dtype != torch.float32 or C.dtype != torch.float32 or r2.dtype != torch.float64:
        raise ValueError("G, C must be fp32 and r2 fp64")
    dev = a_loc.device
    L = lib()
    adt = _DT[a_loc.dtype]
    wsb = L.ispa_accum_stats_workspace_bytes(adt, n, D)
    ws = _workspace(wsb, dev)
    _check(L.ispa_accum_stats(adt, _DT[w.dtype], n, D, a_loc.data_ptr(), delta_a.data_ptr(),
                              w.data_ptr(), G.data_ptr(), C.data_ptr(), r2.data_ptr(), _ptr(ws), wsb,
                              _stream(dev)))


def gram_state(D: int, n_layers: int | None = None, device="cuda"):
    """A zeroed statistics state (fp32 words, opaque layout) for one layer, or
    [n_layers, ...] for several."""
    nb = lib().ispa_gram_state_bytes(D)
    if nb == 0:
        raise ValueError("D must be a positive multiple of 64")
    shape = (nb // 4,) if n_layers is None else (n_layers, nb // 4)
    return torch.zeros(shape, dtype=torch.float32, device=device)


def ispa_accum_gram(a_loc, delta_a, state):
    """In place: the layer's statistics state += this chunk's rows
    (G += a^T a, M += a^T delta, H += delta^T delta)."""
    n, D = a_loc.shape
    for t in (a_loc, delta_a, state):
        if not t.is_contiguous():
            raise ValueError("accum_gram operands must be contiguous")
    if delta_a.shape != a_loc.shape or delta_a.dtype != a_loc.dtype:
        raise ValueError("a_loc and delta_a must match")
    if state.dtype != torch.float32 or state.numel() * 4 < lib().ispa_gram_state_bytes(D):
        raise ValueError("state too small (see gram_state)")
    _check(lib().ispa_accum_gram(_DT[a_loc.dtype], n, D, a_loc.data_ptr(), delta_a.data_ptr(),
                                 state.data_ptr(), _stream(a_loc.device)))


def ispa_gram_finalize(state, w, G=None, C=None, r2=None):
    """G (upper triangle), C = M W and r2 = <H, W W^T> of one state ([S]) and
    W ([D, D]) or of a batch ([L, S] and [L, D, D]).  Returns (G, C, r2)."""
    squeeze = state.dim() == 1
    if squeeze:
        state, w = state.unsqueeze(0), w.unsqueeze(0)
    nl, D = w.shape[0], w.shape[1]
    dev = w.device
    if not state.is_contiguous() or not w.is_contiguous() or w.dtype != torch.bfloat16:
        raise ValueError("state and w (bf16) must be contiguous")
    G = torch.zeros((nl, D, D), dtype=torch.float32, device=dev) if G is None else G
    C = torch.empty((nl, D, D), dtype=torch.float32, device=dev) if C is None else C
    r2 = torch.empty(nl, dtype=torch.float64, device=dev) if r2 is None else r2
    L = lib()
    wsb = L.ispa_gram_finalize_workspace_bytes(D)
    ws = _workspace(wsb, dev)
    _check(L.ispa_gram_finalize(nl, D, state.data_ptr(), state.shape[1], w.data_ptr(), ISPA_BF16, D * D,
                                G.data_ptr(), C.data_ptr(), r2.data_ptr(), D * D, _ptr(ws), wsb, _stream(dev)))
    if squeeze:
        return G[0], C[0], r2
    return G, C, r2


def ispa_solve_dw(G, C, r2, lambda_abs=0.0, lambda_rel=1e-3, w=None, w_eff_dtype=None):
    """Batched ridge solve.  G, C fp32 [L, D, D] (or [D, D]); r2 fp64 [L].
    Returns (dW fp32, eps fp64 [L], info int32 [L], w_eff or None)."""
    squeeze = G.dim() == 2
    if squeeze:
        G, C = G.unsqueeze(0), C.unsqueeze(0)
        r2 = r2.reshape(1)
        if w is not None:
            w = w.unsqueeze(0)
    nl, D, _ = G.shape
    dev = G.device
    for t in (G, C, r2):
        if not t.is_contiguous():
            raise ValueError("solve operands must be contiguous")
    dW = torch.empty_like(G)
    eps = torch.empty(nl, dtype=torch.float64, device=dev)
    info = torch.empty(nl, dtype=torch.int32, device=dev)
    w_eff = None
    if w is not None:
        w = w.contiguous()
        w_eff = torch.empty_like(w, dtype=w_eff_dtype or w.dtype)
        if w_eff.dtype != w.dtype:
            raise ValueError("w_eff has the dtype of w")
    L = lib()
    wsb = L.ispa_solve_dw_workspace_bytes(nl, D)
    ws = _workspace(wsb, dev)
    _check(L.ispa_solve_dw(nl, D, G.data_ptr(), C.data_ptr(), r2.data_ptr(), D * D, lambda_abs,
                           lambda_rel, dW.data_ptr(), eps.data_ptr(), info.data_ptr(), _ptr(w),
                           _DT[w.dtype] if w is not None else 0, _ptr(w_eff), _ptr(ws), wsb,
                           _stream(dev)))
    if squeeze:
        dW = dW[0]
        if w_eff is not None:
            w_eff = w_eff[0]
    return dW, eps, info, w_eff


def ispa_select_layers(eps, K: int):
    """Returns (selected int32 [K], is_local uint8 [N], status int32 [1])."""
    N = eps.shape[0]
    dev = eps.device
    eps = eps.contiguous()
    sel = torch.empty(max(K, 1), dtype=torch.int32, device=dev)
    is_local = torch.empty(N, dtype=torch.uint8, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    _check(lib().ispa_select_layers(N, K, eps.data_ptr(), sel.data_ptr(), is_local.data_ptr(),
                                    status.data_ptr(), _stream(dev)))
    return sel[:K], is_local, status


def ispa_local_attn_proj(q, segs, w_proj, scale: float | None = None, out_dtype=torch.bfloat16):
    """Attention over the segments then y @ w_proj.  Returns y [n_q, D]."""
    n_q, H, d, qs = _q_args(q)
    dt = _DT[q.dtype]
    scale = d ** -0.5 if scale is None else scale
    ss, ns = _segs(segs, H, d)
    dev = q.device
    if not w_proj.is_contiguous():
        raise ValueError("w_proj must be contiguous")
    y = torch.empty((n_q, H * d), dtype=out_dtype, device=dev)
    L = lib()
    wsb = L.ispa_local_attn_proj_workspace_bytes(dt, n_q, H, d, ss, ns)
    ws = _workspace(wsb, dev)
    _check(L.ispa_local_attn_proj(dt, n_q, H, d, scale, q.data_ptr(), qs, ss, ns,
                                  w_proj.data_ptr(), _DT[w_proj.dtype], y.data_ptr(),
                                  _DT[out_dtype], _ptr(ws), wsb, _stream(dev)))
    return y


def ispa_quantize_w_fp8(w):
    """W8A8 weight step: w [d_in, d_out] (bf16 or f16) -> (codes uint8
    [d_out, d_in], scales fp32 [d_out]), one scale per output column."""
    if not w.is_contiguous() or w.dim() != 2:
        raise ValueError("w must be a contiguous [d_in, d_out] matrix")
    d_in, d_out = w.shape
    dev = w.device
    codes = torch.empty((d_out, d_in), dtype=torch.uint8, device=dev)
    scales = torch.empty(d_out, dtype=torch.float32, device=dev)
    L = lib()
    wsb = L.ispa_quantize_w_fp8_workspace_bytes(d_in, d_out)
    ws = _workspace(wsb, dev)
    _check(L.ispa_quantize_w_fp8(_DT[w.dtype], d_in, d_out, w.data_ptr(), codes.data_ptr(),
                                 scales.data_ptr(), _ptr(ws), wsb, _stream(dev)))
    return codes, scales


def ispa_w8a8_linear(x, w_codes, w_scales, out_dtype=torch.bfloat16):
    """y = Q(x) Q(W): x [n, d_in] (rows may be strided) quantised per row,
    (w_codes, w_scales) from ispa_quantize_w_fp8.  Returns y [n, d_out]."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [n, d_in] with contiguous rows")
    n, d_in = x.shape
    d_out = w_codes.shape[0]
    if not w_codes.is_contiguous() or not w_scales.is_contiguous() or w_codes.shape[1] != d_in:
        raise ValueError("w_codes [d_out, d_in] and w_scales [d_out] must be contiguous")
    dev = x.device
    y = torch.empty((n, d_out), dtype=out_dtype, device=dev)
    L = lib()
    wsb = L.ispa_w8a8_linear_workspace_bytes(n, d_in)
    ws = _workspace(wsb, dev)
    _check(L.ispa_w8a8_linear(_DT[x.dtype], n, d_in, d_out, x.data_ptr(), x.stride(0),
                              w_codes.data_ptr(), w_scales.data_ptr(), y.data_ptr(), _DT[out_dtype],
                              _ptr(ws), wsb, _stream(dev)))
    return y


def ispa_w8a8_linear_noalloc(x, w_codes, w_scales, y):
    """ispa_w8a8_linear into a caller-allocated y [n, d_out] (bf16, f16 or
    fp32), with the library's fixed per-device scratch instead of a
    workspace: the call allocates nothing on the device."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [n, d_in] with contiguous rows")
    n, d_in = x.shape
    d_out = w_codes.shape[0]
    if not w_codes.is_contiguous() or not w_scales.is_contiguous() or w_codes.shape[1] != d_in:
        raise ValueError("w_codes [d_out, d_in] and w_scales [d_out] must be contiguous")
    if not y.is_contiguous() or tuple(y.shape) != (n, d_out):
        raise ValueError("y must be a contiguous [n, d_out] tensor")
    _check(lib().ispa_w8a8_linear_noalloc(_DT[x.dtype], n, d_in, d_out, x.data_ptr(), x.stride(0),
                                          w_codes.data_ptr(), w_scales.data_ptr(), y.data_ptr(),
                                          _DT[y.dtype], _stream(x.device)))
    return y


def ispa_local_attn_proj_fp8(q, segs, w_codes, w_scales, scale: float | None = None,
                             out_dtype=torch.bfloat16):
    """bf16 attention over the segments, then the W8A8 projection with
    (w_codes, w_scales) from ispa_quantize_w_fp8.  Returns y [n_q, D]."""
    n_q, H, d, qs = _q_args(q)
    if q.dtype != torch.bfloat16:
        raise ValueError("the fp8 projection path takes bf16 attention inputs")
    scale = d ** -0.5 if scale is None else scale
    ss, ns = _segs(segs, H, d)
    dev = q.device
    if not w_codes.is_contiguous() or not w_scales.is_contiguous():
        raise ValueError("w_codes and w_scales must be contiguous")
    y = torch.empty((n_q, H * d), dtype=out_dtype, device=dev)
    L = lib()
    wsb = L.ispa_local_attn_proj_fp8_workspace_bytes(n_q, H, d, ss, ns)
    ws = _workspace(wsb, dev)
    _check(L.ispa_local_attn_proj_fp8(n_q, H, d, scale, q.data_ptr(), qs, ss, ns, w_codes.data_ptr(),
                                      w_scales.data_ptr(), y.data_ptr(), _DT[out_dtype], _ptr(ws), wsb,
                                      _stream(dev)))
    return y


# ---------------------------------------------------------------- quantised local attention
class Fp8Chunk:
    """One chunk of the fp8 key/value cache as ispa_quantize_kv_fp8 wrote it:
    k_codes and v_codes (uint8, the library's tiled layout), k_scales and
    v_scales (fp32 [H], powers of two), n keys."""

    def __init__(self, k_codes, v_codes, k_scales, v_scales, n: int, H: int):
        self.k_codes, self.v_codes, self.k_scales, self.v_scales = k_codes, v_codes, k_scales, v_scales
        self.n, self.H = int(n), int(H)


def ispa_quantize_kv_fp8(k, v) -> Fp8Chunk:
    """A chunk's k, v ([n, H, 128] with contiguous [H, 128] rows, fp32, bf16
    or f16) into the fp8 cache format."""
    n, H, d = k.shape
    for t in (k, v):
        if t.dim() != 3 or t.shape != k.shape or t.stride(2) != 1 or t.stride(1) != d:
            raise ValueError("k and v must be [n, H, d] with contiguous [H, d] rows")
    if v.dtype != k.dtype:
        raise ValueError("k and v must have one dtype")
    dev = k.device
    L = lib()
    nb = L.ispa_kv_fp8_bytes(n, H, d)
    kc = torch.empty(nb, dtype=torch.uint8, device=dev)
    vc = torch.empty(nb, dtype=torch.uint8, device=dev)
    ks = torch.empty(H, dtype=torch.float32, device=dev)
    vs = torch.empty(H, dtype=torch.float32, device=dev)
    wsb = L.ispa_quantize_kv_fp8_workspace_bytes(n, H, d)
    ws = _workspace(wsb, dev)
    _check(L.ispa_quantize_kv_fp8(_DT[k.dtype], n, H, d, k.data_ptr(), k.stride(0), v.data_ptr(), v.stride(0),
                                  kc.data_ptr(), vc.data_ptr(), ks.data_ptr(), vs.data_ptr(), _ptr(ws), wsb,
                                  _stream(dev)))
    return Fp8Chunk(kc, vc, ks, vs, n, H)


def ispa_quantize_q_fp8(q):
    """Queries [n_q, H, 128] -> (codes uint8 [n_q, H, 128], scales fp32 [n_q, H])."""
    n_q, H, d, qs = _q_args(q)
    dev = q.device
    qc = torch.empty((n_q, H, d), dtype=torch.uint8, device=dev)
    sc = torch.empty((n_q, H), dtype=torch.float32, device=dev)
    _check(lib().ispa_quantize_q_fp8(_DT[q.dtype], n_q, H, d, q.data_ptr(), qs, qc.data_ptr(), sc.data_ptr(),
                                     _stream(dev)))
    return qc, sc


def _segs_fp8(chunks):
    if len(chunks) > ISPA_MAX_SEGS_FP8:
        raise ValueError(f"at most {ISPA_MAX_SEGS_FP8} chunks")
    arr = (SegFp8 * max(1, len(chunks)))()
    for i, c in enumerate(chunks):
        arr[i] = SegFp8(c.k_codes.data_ptr(), c.v_codes.data_ptr(), c.k_scales.data_ptr(), c.v_scales.data_ptr(),
                        c.n)
    return arr, len(chunks)


def ispa_local_attn_fp8(q_codes, q_scales, chunks, scale: float | None = None, out_dtype=torch.float32,
                        want_lse=False):
    """Attention of the quantised queries over the keys of the fp8 chunks.
    Returns (o [n_q, H, 128] of out_dtype, lse fp32 [n_q, H] or None)."""
    n_q, H, d = q_codes.shape
    if not q_codes.is_contiguous() or not q_scales.is_contiguous() or q_codes.dtype != torch.uint8:
        raise ValueError("q_codes (uint8) and q_scales must be contiguous")
    scale = d ** -0.5 if scale is None else scale
    ss, ns = _segs_fp8(chunks)
    dev = q_codes.device
    o = torch.empty((n_q, H, d), dtype=out_dtype, device=dev)
    lse = torch.empty((n_q, H), dtype=torch.float32, device=dev) if want_lse else None
    _check(lib().ispa_local_attn_fp8(n_q, H, d, scale, q_codes.data_ptr(), q_scales.data_ptr(), ss, ns,
                                     o.data_ptr(), _DT[out_dtype], _ptr(lse), _stream(dev)))
    return o, lse


def ispa_local_attn_fp8_proj(q, chunks, w_codes, w_scales, scale: float | None = None, out_dtype=torch.bfloat16):
    """The post-switch layer output with fp8 attention over the chunks and the
    W8A8 projection with (w_codes, w_scales) from ispa_quantize_w_fp8.
    q [n_q, H, 128].  Returns y [n_q, D]."""
    n_q, H, d, qs = _q_args(q)
    scale = d ** -0.5 if scale is None else scale
    ss, ns = _segs_fp8(chunks)
    dev = q.device
    if not w_codes.is_contiguous() or not w_scales.is_contiguous():
        raise ValueError("w_codes and w_scales must be contiguous")
    y = torch.empty((n_q, H * d), dtype=out_dtype, device=dev)
    L = lib()
    wsb = L.ispa_local_attn_fp8_proj_workspace_bytes(n_q, H, d)
    ws = _workspace(wsb, dev)
    _check(L.ispa_local_attn_fp8_proj(n_q, H, d, scale, _DT[q.dtype], q.data_ptr(), qs, ss, ns, w_codes.data_ptr(),
                                      w_scales.data_ptr(), y.data_ptr(), _DT[out_dtype], _ptr(ws), wsb,
                                      _stream(dev)))
    return y
