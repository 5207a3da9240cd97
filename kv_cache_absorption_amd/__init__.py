"""MI355X-native (gfx950) hot path of Instance-Specific Parametric Absorption.

The compute lives in libispa.so (HIP kernels behind the C ABI of
include/ispa.h); this package only marshals torch tensors to it.  Build the
library with ``python -m kv_cache_absorption_amd.build``.
"""
from ._lib import (ISPA_BF16, ISPA_F16, ISPA_F32, IspaError, gram_state, ispa_accum_gram,  # noqa: F401
                   ispa_accum_stats, ispa_gram_finalize,
                   ispa_dual_attn, ispa_dual_attn_merge, ispa_local_attn_proj,
                   ispa_local_attn_proj_fp8, ispa_lse_merge, ispa_quantize_w_fp8, ispa_select_layers,
                   ispa_solve_dw, ispa_w8a8_linear, ispa_w8a8_linear_noalloc, lib,
                   Fp8Chunk, ispa_local_attn_fp8, ispa_local_attn_fp8_proj, ispa_quantize_kv_fp8,
                   ispa_quantize_q_fp8)
from .stream import Workspace, chunk_segments, kv_bytes  # noqa: F401
