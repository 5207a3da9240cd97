"""CPU checks of the C ABI: the library loads, exports what include/ispa.h
declares, and rejects bad arguments on the host before launching anything.
Also the host-side stream layout against the oracle's grouping."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    try:
        from kv_cache_absorption_amd import _lib as m
        return m, m.lib()
    except (ImportError, OSError) as e:  # libamdhip64 missing or library not built
        pytest.skip(f"libispa not loadable here: {e}")


def test_exports_match_header():
    m, L = _lib()
    hdr = open(os.path.join(ROOT, "include", "ispa.h")).read()
    declared = set(re.findall(r"\b(ispa_[a-z0-9_]+)\s*\(", hdr))
    assert declared == set(m.EXPORTED)
    for name in declared:
        assert hasattr(L, name), name
    assert L.ispa_version() == 10000
    assert L.ispa_status_str(m.ISPA_ERR_WORKSPACE) == b"workspace too small"


def _seg(n, H=2, d=128, ptr=256):
    return (n and ptr, n and ptr, n, H * d, H * d)


def _segarr(m, specs):
    arr = (m.Seg * max(1, len(specs)))()
    for i, s in enumerate(specs):
        arr[i] = m.Seg(*s)
    return arr


FAKE = 4096  # a non-null, aligned address that is never dereferenced


def test_dual_attn_rejects_bad_args():
    m, L = _lib()
    segs = _segarr(m, [_seg(10, ptr=FAKE)])
    args = dict(dt=m.ISPA_BF16, n_q=4, H=2, d=128, scale=0.1, q=FAKE, qs=256)

    def call(**kw):
        a = {**args, **kw}
        return L.ispa_dual_attn(a["dt"], a["n_q"], a["H"], a["d"], a["scale"], a["q"], a["qs"],
                                segs, kw.get("nl", 1), segs, kw.get("nh", 1), FAKE, FAKE, FAKE, FAKE,
                                None, 0, None)
    assert call(d=96) == m.ISPA_ERR_UNSUPPORTED
    assert call(dt=m.ISPA_F16) == m.ISPA_ERR_UNSUPPORTED
    assert call(q=None) == m.ISPA_ERR_INVALID_ARG
    assert call(qs=100) == m.ISPA_ERR_INVALID_ARG
    assert call(nl=9) == m.ISPA_ERR_INVALID_ARG
    assert call(q=FAKE + 2) == m.ISPA_ERR_INVALID_ARG  # misaligned bf16 rows
    assert call(scale=float("nan")) == m.ISPA_ERR_INVALID_ARG
    assert b"finite" in L.ispa_last_error()
    bad = _segarr(m, [(0, FAKE, 10, 256, 256)])
    assert L.ispa_dual_attn(m.ISPA_BF16, 4, 2, 128, 0.1, FAKE, 256, bad, 1, segs, 1,
                            FAKE, FAKE, FAKE, FAKE, None, 0, None) == m.ISPA_ERR_INVALID_ARG


def test_dual_attn_merge_rejects_bad_args():
    """The fused attention + merge call validates like ispa_dual_attn, plus
    its output type and alignment; every error returns before any launch."""
    m, L = _lib()
    segs = _segarr(m, [_seg(10, ptr=FAKE)])

    def call(out_dt=m.ISPA_F16, a_loc=FAKE, delta=FAKE, nl=1, ws=None, wsb=0, d=128):
        return L.ispa_dual_attn_merge(m.ISPA_BF16, 4, 2, d, 0.1, FAKE, 256, segs, nl, segs, 1,
                                      a_loc, delta, out_dt, None, ws, wsb, None)
    assert call(d=96) == m.ISPA_ERR_UNSUPPORTED
    assert call(nl=9) == m.ISPA_ERR_INVALID_ARG
    assert call(out_dt=7) == m.ISPA_ERR_UNSUPPORTED
    assert call(a_loc=None) == m.ISPA_ERR_INVALID_ARG
    assert call(delta=FAKE + 4) == m.ISPA_ERR_INVALID_ARG            # 8-byte alignment for fp16
    assert call(out_dt=m.ISPA_F32, a_loc=FAKE + 8) == m.ISPA_ERR_INVALID_ARG  # 16 for fp32
    need = L.ispa_dual_attn_merge_workspace_bytes(m.ISPA_BF16, 4, 2, 128, segs, 1, segs, 1)
    assert need > 0  # every piece goes through the workspace, split or not
    assert call(ws=FAKE, wsb=need - 1) == m.ISPA_ERR_WORKSPACE


def test_workspace_queries_and_errors():
    m, L = _lib()
    # Wan-1.3B layer: 37 q-tiles x 12 heads x 2 groups is below the split target,
    # so the history group is split and needs workspace
    loc = _segarr(m, [_seg(4680, 12, 128, FAKE), _seg(4680, 12, 128, FAKE)])
    hist = _segarr(m, [_seg(28080, 12, 128, FAKE)])
    need = L.ispa_dual_attn_workspace_bytes(m.ISPA_BF16, 4680, 12, 128, loc, 2, hist, 1)
    assert need > 0
    st = L.ispa_dual_attn(m.ISPA_BF16, 4680, 12, 128, 0.1, FAKE, 1536, loc, 2, hist, 1,
                          FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None)
    assert st == m.ISPA_ERR_WORKSPACE
    # enough work units (many heads, short history): no split, no workspace
    loc64 = _segarr(m, [_seg(4680, 64, 128, FAKE), _seg(4680, 64, 128, FAKE)])
    hist64 = _segarr(m, [_seg(9360, 64, 128, FAKE)])
    assert L.ispa_dual_attn_workspace_bytes(m.ISPA_BF16, 4680, 64, 128, loc64, 2, hist64, 1) == 0
    assert L.ispa_accum_stats_workspace_bytes(m.ISPA_F16, 4680, 1536) >= 1536 * 4680 * 2
    assert L.ispa_solve_dw_workspace_bytes(2, 128) >= 2 * 2 * 128 * 128 * 8


def test_header_compiles_as_c_and_links(tmp_path):
    """include/ispa.h is a C header: a C11 program that includes it compiles
    with gcc, links against the built library and calls its host-side entry
    points (version, status strings, a size query)."""
    import shutil
    import subprocess
    m, L = _lib()
    gcc = shutil.which("gcc")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    if gcc is None or not os.path.isdir(os.path.join(rocm, "include", "hip")):
        pytest.skip("gcc or the ROCm headers are not available")
    src = tmp_path / "t.c"
    src.write_text('#include "ispa.h"\n#include <stdio.h>\n'
                   'int main(void) {\n'
                   '  printf("%d\\n%s\\n%zu\\n", ispa_version(), ispa_status_str(ISPA_ERR_WORKSPACE),\n'
                   '         ispa_gram_state_bytes(1536));\n'
                   '  return 0;\n}\n')
    libdir = os.path.dirname(m.LIB_PATH)
    exe = tmp_path / "t"
    subprocess.run([gcc, "-std=c11", "-Wall", "-Werror=implicit-function-declaration", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"), str(src),
                    "-L", libdir, "-lispa", f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True,
                   capture_output=True, timeout=120)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, timeout=60).stdout.splitlines()
    assert int(out[0]) == L.ispa_version()
    assert out[1] == L.ispa_status_str(m.ISPA_ERR_WORKSPACE).decode()
    assert int(out[2]) == L.ispa_gram_state_bytes(1536)


def test_local_attn_proj_split_rule():
    """A single key set runs whole when its launch already gives half the CUs a
    workgroup (no split parts in the workspace), and is split into merged
    pieces when the launch would leave most CUs idle."""
    m, L = _lib()
    a = lambda b: (b + 255) // 256 * 256  # noqa: E731

    def base(n_q, H, d=128):  # fp32 O and LSE, bf16 O, bf16 W^T
        D = H * d
        return a(n_q * D * 4) + a(n_q * H * 4) + a(n_q * D * 2) + a(D * D * 2)

    # Wan-1.3B F-Layer at its last chunk: 19 query tiles x 12 heads = 228 workgroups
    segs = _segarr(m, [_seg(93600, 12, 128, FAKE)])
    assert L.ispa_local_attn_proj_workspace_bytes(m.ISPA_BF16, 4680, 12, 128, segs, 1) == base(4680, 12)
    # 8 query tiles x 16 heads = 128: still whole
    segs16 = _segarr(m, [_seg(93600, 16, 128, FAKE)])
    assert L.ispa_local_attn_proj_workspace_bytes(m.ISPA_BF16, 2048, 16, 128, segs16, 1) == base(2048, 16)
    # 3 query tiles x 12 heads = 36: split, each piece with its fp32 (o, lse) part
    part = a(600 * 12 * 128 * 4) + a(600 * 12 * 4)
    need = L.ispa_local_attn_proj_workspace_bytes(m.ISPA_BF16, 600, 12, 128, segs, 1)
    assert need > base(600, 12) and (need - base(600, 12)) % part == 0 and (need - base(600, 12)) // part >= 2


def test_stats_solve_select_reject_bad_args():
    m, L = _lib()
    F = FAKE
    assert L.ispa_accum_stats(m.ISPA_BF16, m.ISPA_BF16, 10, 100, F, F, F, F, F, F, F, 1 << 20, None) \
        == m.ISPA_ERR_INVALID_ARG  # D not a multiple of 64
    assert L.ispa_accum_stats(m.ISPA_F32, m.ISPA_BF16, 10, 128, F, F, F, F, F, F, F, 1 << 20, None) \
        == m.ISPA_ERR_UNSUPPORTED
    assert L.ispa_accum_stats(m.ISPA_BF16, m.ISPA_BF16, 10, 128, F, F, F, F, F, F, None, 0, None) \
        == m.ISPA_ERR_WORKSPACE
    assert L.ispa_accum_stats(m.ISPA_BF16, m.ISPA_BF16, 0, 128, F, F, F, F, F, F, None, 0, None) \
        == m.ISPA_OK  # empty step: nothing to do, nothing launched
    assert L.ispa_solve_dw(1, 128, F, F, F, 128 * 128, 0.0, 1e-3, F, F, F, None, 0, None, None, 0,
                           None) == m.ISPA_ERR_WORKSPACE
    assert L.ispa_solve_dw(1, 128, F, F, F, 100, 0.0, 1e-3, F, F, F, None, 0, None, F, 1 << 30,
                           None) == m.ISPA_ERR_INVALID_ARG
    assert L.ispa_solve_dw(1, 128, F, F, F, 128 * 128, 0.0, -1.0, F, F, F, None, 0, None, F, 1 << 30,
                           None) == m.ISPA_ERR_INVALID_ARG
    assert L.ispa_solve_dw(1, 128, F, F, F, 128 * 128, 0.0, 1e-3, F, F, F, F, m.ISPA_BF16, None, F,
                           1 << 30, None) == m.ISPA_ERR_INVALID_ARG  # w without w_eff
    assert L.ispa_select_layers(30, 31, F, F, F, F, None) == m.ISPA_ERR_INVALID_ARG
    assert L.ispa_select_layers(0, 0, F, F, F, F, None) == m.ISPA_ERR_INVALID_ARG
    assert L.ispa_select_layers(2000, 1, F, F, F, F, None) == m.ISPA_ERR_INVALID_ARG
    op = (ctypes.c_void_p * 1)(F)
    assert L.ispa_lse_merge(0, op, op, 4, 2, 128, F, F, F, F, m.ISPA_F32, None) == m.ISPA_ERR_INVALID_ARG
    assert L.ispa_lse_merge(1, op, op, 4, 2, 6, F, F, F, F, m.ISPA_F32, None) == m.ISPA_ERR_INVALID_ARG
    assert L.ispa_lse_merge(1, op, op, 4, 2, 128, F, F, F, F, 7, None) == m.ISPA_ERR_UNSUPPORTED
    segs = _segarr(m, [_seg(10, ptr=F)])
    assert L.ispa_local_attn_proj(m.ISPA_BF16, 4, 2, 128, 0.1, F, 256, segs, 1, F, m.ISPA_F32, F,
                                  m.ISPA_BF16, F, 1 << 20, None) == m.ISPA_ERR_UNSUPPORTED
    assert L.ispa_local_attn_proj(m.ISPA_BF16, 4, 2, 128, 0.1, F, 256, segs, 0, F, m.ISPA_BF16, F,
                                  m.ISPA_BF16, F, 1 << 20, None) == m.ISPA_ERR_INVALID_ARG


def test_stream_layout_matches_oracle_grouping():
    from kv_cache_absorption_amd.stream import chunk_segments, keys_retained, kv_bytes
    from oracle import kv_bytes_retained, stream_groups
    T, H, d = 5, 2, 4
    cache = torch.arange(12 * T * H * d, dtype=torch.float32).reshape(12 * T, H, d)
    for c in range(12):
        loc, hist = chunk_segments(cache, cache, c, T)
        oloc, ohist = stream_groups(c, T)
        for got, want in ((loc, oloc), (hist, ohist)):
            assert len(got) == len(want)
            for (k, v), (a, b) in zip(got, want):
                assert torch.equal(k, cache[a:b]) and k.data_ptr() == cache[a:b].data_ptr()
    flags = [1, 0, 1, 1, 0]
    for c in (0, 1, 7):
        n = keys_retained(c, T, flags)
        assert kv_bytes(n, 1536) == kv_bytes_retained(n, 1536)


def test_w8a8_calls_reject_bad_args():
    m, L = _lib()
    F = FAKE
    big = 1 << 30
    # weight quantisation: 16-bit W only, dims multiples of 4, workspace checked
    assert L.ispa_quantize_w_fp8_workspace_bytes(1536, 1536) >= 1536 * 1536 * 2
    assert L.ispa_quantize_w_fp8(m.ISPA_F32, 128, 128, F, F, F, F, big, None) == m.ISPA_ERR_UNSUPPORTED
    assert L.ispa_quantize_w_fp8(m.ISPA_BF16, 130, 128, F, F, F, F, big, None) == m.ISPA_ERR_INVALID_ARG
    assert L.ispa_quantize_w_fp8(m.ISPA_BF16, 128, 128, None, F, F, F, big, None) == m.ISPA_ERR_INVALID_ARG
    assert L.ispa_quantize_w_fp8(m.ISPA_BF16, 128, 128, F, F, F, F, 10, None) == m.ISPA_ERR_WORKSPACE
    # the W8A8 product: d_in a multiple of 64, ld_x >= d_in, 16-byte aligned codes and scales
    assert L.ispa_w8a8_linear_workspace_bytes(4680, 1536) >= 4680 * 1536 + 4680 * 4
    assert L.ispa_w8a8_linear(m.ISPA_F32, 8, 96, 64, F, 96, F, F, F, m.ISPA_F32, F, big, None) \
        == m.ISPA_ERR_INVALID_ARG  # d_in not a multiple of 64
    assert L.ispa_w8a8_linear(m.ISPA_F32, 8, 128, 64, F, 64, F, F, F, m.ISPA_F32, F, big, None) \
        == m.ISPA_ERR_INVALID_ARG  # ld_x < d_in
    assert L.ispa_w8a8_linear(m.ISPA_F32, 8, 128, 64, F, 128, F + 4, F, F, m.ISPA_F32, F, big, None) \
        == m.ISPA_ERR_INVALID_ARG  # misaligned codes
    assert L.ispa_w8a8_linear(9, 8, 128, 64, F, 128, F, F, F, m.ISPA_F32, F, big, None) \
        == m.ISPA_ERR_UNSUPPORTED
    assert L.ispa_w8a8_linear(m.ISPA_F32, 8, 128, 64, F, 128, F, F, F, m.ISPA_F32, F, 10, None) \
        == m.ISPA_ERR_WORKSPACE
    assert L.ispa_w8a8_linear(m.ISPA_F32, 0, 128, 64, None, 128, F, F, None, m.ISPA_F32, None, 0, None) \
        == m.ISPA_OK  # no rows: nothing launched
    # attention + W8A8 projection: bf16 attention arguments, D = H d
    segs = _segarr(m, [_seg(10, ptr=F)])
    assert L.ispa_local_attn_proj_fp8_workspace_bytes(4, 2, 128, segs, 1) > 4 * 256 * 4
    assert L.ispa_local_attn_proj_fp8(4, 2, 96, 0.1, F, 256, segs, 1, F, F, F, m.ISPA_BF16, F, big,
                                      None) == m.ISPA_ERR_UNSUPPORTED  # head_dim
    assert L.ispa_local_attn_proj_fp8(4, 2, 128, 0.1, F, 256, segs, 0, F, F, F, m.ISPA_BF16, F, big,
                                      None) == m.ISPA_ERR_INVALID_ARG  # no segments
    assert L.ispa_local_attn_proj_fp8(4, 2, 128, 0.1, F, 256, segs, 1, None, F, F, m.ISPA_BF16, F, big,
                                      None) == m.ISPA_ERR_INVALID_ARG  # no weight codes
    assert L.ispa_local_attn_proj_fp8(4, 2, 128, float("nan"), F, 256, segs, 1, F, F, F, m.ISPA_BF16, F,
                                      big, None) == m.ISPA_ERR_INVALID_ARG
    assert L.ispa_local_attn_proj_fp8(4, 2, 128, 0.1, F, 256, segs, 1, F, F, F, m.ISPA_BF16, F, 10,
                                      None) == m.ISPA_ERR_WORKSPACE


def test_w8a8_noalloc_rejects_bad_args():
    """The allocation-free W8A8 product validates on the host: a scratch need
    above the fixed array is an argument error returned before any device
    work, as are the usual shape, alignment and pointer errors."""
    m, L = _lib()
    lim = m.ISPA_NOALLOC_SCRATCH_BYTES

    def call(n=64, d_in=1536, d_out=1536, x=FAKE, ld=1536, wc=FAKE, ws=FAKE, y=FAKE, xdt=m.ISPA_F32,
             ydt=m.ISPA_BF16):
        return L.ispa_w8a8_linear_noalloc(xdt, n, d_in, d_out, x, ld, wc, ws, y, ydt, None)

    def need(n, d_in):
        return L.ispa_w8a8_linear_workspace_bytes(n, d_in)

    assert call(n=0) == m.ISPA_OK                        # nothing to do
    assert need(6548, 5120) <= lim < need(6549, 5120)      # the documented limit
    assert call(n=6560, d_in=5120, d_out=5120, ld=5120) == m.ISPA_ERR_INVALID_ARG
    assert b"scratch" in L.ispa_last_error()
    assert call(n=-1) == m.ISPA_ERR_INVALID_ARG
    assert call(d_in=100, ld=100) == m.ISPA_ERR_INVALID_ARG  # not a multiple of 64
    assert call(ld=1000) == m.ISPA_ERR_INVALID_ARG
    assert call(x=None) == m.ISPA_ERR_INVALID_ARG
    assert call(wc=None) == m.ISPA_ERR_INVALID_ARG
    assert call(y=FAKE + 4) == m.ISPA_ERR_INVALID_ARG      # bf16 y must be 8-byte aligned
    assert call(xdt=7) == m.ISPA_ERR_UNSUPPORTED


def test_fp8_attention_calls_reject_bad_args():
    """The quantised local attention path validates on the host: head_dim 128
    only, positive finite scale, segment table limits, alignment of codes and
    scales, workspace size; empty work returns at once."""
    m, L = _lib()
    F = FAKE
    big = 1 << 30
    assert L.ispa_kv_fp8_bytes(4680, 12, 128) == 12 * 74 * 64 * 128
    assert L.ispa_kv_fp8_bytes(4680, 12, 64) == 0
    assert L.ispa_quantize_kv_fp8_workspace_bytes(4680, 12, 128) >= 2 * 12 * 74 * 4
    # quantize_kv: dtype, head_dim, strides, alignment, workspace
    kv = lambda **a: L.ispa_quantize_kv_fp8(a.get("dt", m.ISPA_BF16), a.get("n", 100), a.get("H", 2),  # noqa: E731
                                            a.get("d", 128), a.get("k", F), a.get("ks", 256), F, 256,
                                            a.get("kc", F), F, F, F, F, a.get("ws", big), None)
    assert kv(d=64) == m.ISPA_ERR_UNSUPPORTED
    assert kv(dt=9) == m.ISPA_ERR_UNSUPPORTED
    assert kv(ks=200) == m.ISPA_ERR_INVALID_ARG      # stride < H * d
    assert kv(ks=258) == m.ISPA_ERR_INVALID_ARG      # stride not a multiple of 4
    assert kv(k=F + 2) == m.ISPA_ERR_INVALID_ARG     # 16-bit rows 8-byte aligned
    assert kv(kc=F + 8) == m.ISPA_ERR_INVALID_ARG    # codes 16-byte aligned
    assert kv(k=None) == m.ISPA_ERR_INVALID_ARG
    assert kv(ws=10) == m.ISPA_ERR_WORKSPACE
    assert kv(n=0, k=None, kc=None) == m.ISPA_OK
    # quantize_q
    assert L.ispa_quantize_q_fp8(m.ISPA_BF16, 10, 2, 96, F, 256, F, F, None) == m.ISPA_ERR_UNSUPPORTED
    assert L.ispa_quantize_q_fp8(m.ISPA_F32, 10, 2, 128, F + 4, 256, F, F, None) == m.ISPA_ERR_INVALID_ARG
    assert L.ispa_quantize_q_fp8(m.ISPA_BF16, 10, 2, 128, F, 256, None, F, None) == m.ISPA_ERR_INVALID_ARG
    assert L.ispa_quantize_q_fp8(m.ISPA_BF16, 0, 2, 128, None, 256, None, None, None) == m.ISPA_OK
    # attention
    arr = (m.SegFp8 * 9)()
    for i in range(9):
        arr[i] = m.SegFp8(F, F, F, F, 100)

    def att(n_q=10, d=128, scale=0.1, qc=F, segs=arr, ns=1, o=F, odt=m.ISPA_F32, lse=None):
        return L.ispa_local_attn_fp8(n_q, 2, d, scale, qc, F, segs, ns, o, odt, lse, None)

    assert att(d=64) == m.ISPA_ERR_UNSUPPORTED
    assert att(scale=0.0) == m.ISPA_ERR_INVALID_ARG
    assert att(scale=float("inf")) == m.ISPA_ERR_INVALID_ARG
    assert att(ns=65) == m.ISPA_ERR_INVALID_ARG  # above ISPA_MAX_SEGS_FP8
    assert att(ns=-1) == m.ISPA_ERR_INVALID_ARG
    assert att(qc=F + 4) == m.ISPA_ERR_INVALID_ARG
    assert att(o=F + 4) == m.ISPA_ERR_INVALID_ARG
    assert att(lse=F + 2) == m.ISPA_ERR_INVALID_ARG
    assert att(odt=7) == m.ISPA_ERR_UNSUPPORTED
    bad = (m.SegFp8 * 1)()
    bad[0] = m.SegFp8(F + 8, F, F, F, 100)
    assert att(segs=bad) == m.ISPA_ERR_INVALID_ARG
    bad[0] = m.SegFp8(None, F, F, F, 100)
    assert att(segs=bad) == m.ISPA_ERR_INVALID_ARG
    bad[0] = m.SegFp8(F, F, F, F, -1)
    assert att(segs=bad) == m.ISPA_ERR_INVALID_ARG
    assert att(n_q=0, qc=None, o=None) == m.ISPA_OK
    # attention + W8A8 projection
    assert L.ispa_local_attn_fp8_proj_workspace_bytes(4680, 12, 128) >= 4680 * 1536 * 6
    proj = lambda **a: L.ispa_local_attn_fp8_proj(a.get("n_q", 10), 2, 128, 0.1, m.ISPA_BF16, F, 256, arr, 1,  # noqa: E731
                                                 a.get("wc", F), F, F, m.ISPA_BF16, F, a.get("ws", big), None)
    assert proj(wc=None) == m.ISPA_ERR_INVALID_ARG
    assert proj(ws=10) == m.ISPA_ERR_WORKSPACE
