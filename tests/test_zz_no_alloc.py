"""The allocation-free W8A8 product, ispa_w8a8_linear_noalloc, through the C
ABI against the workspace call it varies, ispa_w8a8_linear: the same kernels
on the library's fixed per-device scratch, so the outputs must agree bit for
bit.  Two calls in a row share the scratch; the second is smaller and must
not see anything the first left there."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_w8a8_noalloc_matches_workspace_call():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_absorption_amd as K
    cases = [
        # (rows, width, x dtype, y dtype): the largest call the scratch takes at the
        # Wan-14B width, then a smaller Wan-1.3B-width call with ragged rows
        (6548, 5120, torch.float32, torch.bfloat16),
        (1001, 1536, torch.bfloat16, torch.float32),
    ]
    for i, (n, D, xdt, ydt) in enumerate(cases):
        print(f"w8a8 noalloc call {i}: n={n} D={D} x={xdt} y={ydt}", flush=True)
        w = synth.normal((D, D), 501 + i, DEV, std=D ** -0.5, dtype=torch.bfloat16)
        codes, scales = K.ispa_quantize_w_fp8(w)
        x = synth.normal((n, D), 511 + i, DEV, dtype=xdt)
        x[3] = 0  # a zero row: scale 0 and zero codes
        ref = K.ispa_w8a8_linear(x, codes, scales, out_dtype=ydt)
        y = torch.full((n, D), float("nan"), dtype=ydt, device=DEV)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        K.ispa_w8a8_linear_noalloc(x, codes, scales, y)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        assert torch.equal(y, ref), float((y.float() - ref.float()).abs().max())
        assert not y[3].any()
