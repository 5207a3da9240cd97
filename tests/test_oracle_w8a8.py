"""Pins of the oracle's W8A8 projection (FP8 E4M3 codes, per-row
quantisation, the quantised product), CPU only.

The pages give no quantisation scheme (EN review, Key Findings: the W8A8
figure only), so these pins fix the E4M3 format by its definition and by an
independent implementation of it (torch's float8_e4m3fn), and the scheme by
its invariants and exact small cases."""
import math

import numpy as np
import pytest
import torch

import oracle as O


def torch_decode(codes):
    t = torch.tensor(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def torch_encode(x):
    """torch's float32 -> float8_e4m3fn conversion (nearest, ties to even);
    a zero magnitude is mapped to the scheme's single zero code."""
    c = torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    c[(c & 0x7F) == 0] = 0
    return c


def test_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = O.e4m3_decode(codes), torch_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ours[~nan], ref[~nan])


def test_decode_closed_forms():
    # largest finite, smallest normal, smallest subnormal, one, a negative
    assert O.e4m3_decode([0x7E, 0x08, 0x01, 0x38, 0xC2]).tolist() == [448.0, 2.0 ** -6, 2.0 ** -9, 1.0, -2.5]
    assert O.E4M3_MAX == 448.0


def test_encode_ties_and_bounds_from_the_definition():
    # value, code: ties between neighbours go to the even mantissa
    cases = [
        (1.0625, 0x38),      # halfway 1 / 1.125 -> 1 (mantissa 0)
        (1.1875, 0x3A),      # halfway 1.125 / 1.25 -> 1.25 (mantissa 2)
        (17.0, 0x58),        # halfway 16 / 18 -> 16
        (19.0, 0x5A),        # halfway 18 / 20 -> 20
        (432.0, 0x7E),       # halfway 416 / 448 -> 448 (mantissa 6)
        (2.0 ** -10, 0x00),  # half the smallest subnormal -> 0
        (3 * 2.0 ** -11, 0x01),
        (448.0, 0x7E),
        (-448.0, 0xFE),
        (-2.5, 0xC2),
        (-1e-5, 0x00),       # rounds to zero: the single zero code
        (0.0, 0x00),
    ]
    got = O.e4m3_encode([c[0] for c in cases])
    assert [int(g) for g in got] == [c[1] for c in cases]
    with pytest.raises(ValueError):
        O.e4m3_encode([449.0])


def test_encode_matches_torch_on_random_values():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.normal(size=20000) * 3.0,
        rng.normal(size=20000) * 1e-2,
        np.exp2(rng.uniform(-12, 8.8, 20000)) * rng.choice([-1, 1], 20000),
    ]).astype(np.float32)
    x = np.clip(x, -448, 448)
    assert np.array_equal(O.e4m3_encode(x), torch_encode(x))


def test_encode_is_the_nearest_code():
    # brute force over every finite code for a few thousand values
    rng = np.random.default_rng(6)
    x = rng.uniform(-448, 448, 3000)
    vals = O.e4m3_decode(np.arange(256, dtype=np.uint8))
    finite = ~np.isnan(vals)
    best = np.min(np.abs(x[:, None] - vals[None, finite]), axis=1)
    assert np.array_equal(np.abs(O.e4m3_decode(O.e4m3_encode(x)) - x), best)


def test_quantize_rows_invariants():
    rng = np.random.default_rng(7)
    x = (rng.normal(size=(64, 320)) * np.exp(rng.normal(size=(64, 1)))).astype(np.float32)
    x[3] = 0.0
    codes, scale = O.quantize_rows_e4m3(x)
    assert codes.dtype == np.uint8 and scale.dtype == np.float32
    assert scale[3] == 0 and not codes[3].any()
    dec = O.e4m3_decode(codes)
    nz = np.arange(64) != 3
    # the row maximum maps to the largest code
    assert np.all(np.max(np.abs(dec[nz]), axis=1) == 448.0)
    # reconstruction within half a unit in the last place: 2^-4 relative for
    # normal codes, 2^-10 scale for subnormal ones (one rounding of x / scale
    # in fp32 adds at most 2^-24 relative)
    s = scale.astype(np.float64)[:, None]
    err = np.abs(dec * s - x)
    bound = 2.0 ** -4 * np.abs(x) * (1 + 2.0 ** -20) + 2.0 ** -10 * s
    assert np.all(err[nz] <= bound[nz])
    # scale is amax / 448 rounded to fp32
    amax = np.max(np.abs(x), axis=1)
    assert np.array_equal(scale, (amax / np.float32(448)).astype(np.float32))


def test_quantize_weight_is_per_output_column():
    rng = np.random.default_rng(8)
    w = rng.normal(size=(96, 40)).astype(np.float32)
    w[:, 7] *= 100.0  # one loud column does not change the others' codes
    codes, scale = O.quantize_weight_e4m3(w)
    assert codes.shape == (40, 96) and scale.shape == (40,)
    c2, s2 = O.quantize_rows_e4m3(np.delete(w, 7, axis=1).T)
    assert np.array_equal(np.delete(codes, 7, axis=0), c2)
    assert np.array_equal(np.delete(scale, 7), s2)


def test_w8a8_linear_exact_on_grid_operands():
    # operands already on the E4M3 grid with a row maximum of 448: scales are 1,
    # the codes reproduce the values, and the product is the plain one
    rng = np.random.default_rng(9)
    grid = O.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    grid = np.concatenate([grid, -grid[1:]])
    x = rng.choice(grid, size=(8, 64))
    x[:, 0] = 448.0
    w = rng.choice(grid, size=(64, 16))
    w[0, :] = -448.0
    wq, ws = O.quantize_weight_e4m3(w)
    assert np.all(ws == 1.0)
    y = O.w8a8_linear(x, wq, ws)
    ref = np.zeros((8, 16))
    for i in range(8):
        for j in range(16):
            ref[i, j] = math.fsum(x[i, k] * w[k, j] for k in range(64))
    assert np.array_equal(y, ref)


def test_w8a8_linear_close_to_the_unquantised_product():
    # each operand is within 2^-4 relative (elementwise) of its source, so the
    # product error is bounded by the sum of |x||w| terms times ~2^-3
    rng = np.random.default_rng(10)
    x = rng.normal(size=(32, 256)).astype(np.float32)
    w = (rng.normal(size=(256, 48)) / 16).astype(np.float32)
    wq, ws = O.quantize_weight_e4m3(w)
    y = O.w8a8_linear(x, wq, ws)
    ref = x.astype(np.float64) @ w.astype(np.float64)
    bound = (2.0 ** -3 + 2.0 ** -7) * (np.abs(x).astype(np.float64) @ np.abs(w).astype(np.float64)) + 1e-3
    assert np.all(np.abs(y - ref) <= bound)
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert 1e-3 < rel < 6e-2  # quantisation is visible but small


def test_local_attn_proj_w8a8_reduces_to_parts():
    rng = np.random.default_rng(11)
    q = rng.normal(size=(5, 2, 16))
    k = rng.normal(size=(9, 2, 16))
    v = rng.normal(size=(9, 2, 16))
    w = rng.normal(size=(32, 24)) / 6
    y = O.local_attn_proj_w8a8(q, k, v, w, 0.25)
    o, _ = O.group_attention(q, k, v, 0.25)
    wq, ws = O.quantize_weight_e4m3(w)
    assert np.array_equal(y, O.w8a8_linear(o.reshape(5, -1).astype(np.float32), wq, ws))


# ---------------------------------------------------------------- quantised attention
def test_pow2_scale_is_the_smallest_power_of_two():
    """Brute force over exponents in exact arithmetic: the scale is the least
    2^e >= 2^-126 with amax <= 448 * 2^e (the boundary cases 448 * 2^k and
    the fp32 values on either side included, and magnitudes so small that
    the floor decides), 1 for a zero group."""
    from fractions import Fraction
    rng = np.random.default_rng(2)
    vals = [np.float32(448.0 * 2.0 ** k) for k in (-20, -3, 0, 5)]
    vals += [np.nextafter(v, np.float32(np.inf)) for v in vals] + [np.nextafter(v, np.float32(0)) for v in vals]
    vals += list(rng.lognormal(0, 8, 200).astype(np.float32))
    vals += [np.float32(1e-40), np.float32(2e-38), np.float32(448.0 * 2.0 ** -126), np.float32(3e38)]
    amax = np.array(vals, dtype=np.float32)
    got = O.pow2_scale(amax)
    for a, s in zip(amax, got):
        e = next(e for e in range(-126, 140) if Fraction(float(a)) <= 448 * Fraction(2) ** e)
        assert Fraction(float(s)) == Fraction(2) ** e, (a, s, e)
    assert O.pow2_scale(np.zeros(3, np.float32)).tolist() == [1.0, 1.0, 1.0]


def test_quantize_chunk_scales_and_codes():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 3, 16)).astype(np.float32)
    x[:, 1, :] *= 100.0      # heads of very different ranges
    x[:, 2, :] = 0.0         # an all-zero head
    codes, scales = O.quantize_chunk_e4m3(x)
    assert codes.shape == x.shape and scales.shape == (3,)
    for h in (0, 1):
        amax = np.abs(x[:, h, :]).max()
        # a power of two that takes the head's maximum into (224, 448]
        assert math.frexp(float(scales[h]))[0] == 0.5
        assert 224.0 < amax / scales[h] <= 448.0
    assert not codes[:, 2, :].any() and scales[2] == 1.0
    # codes are torch's E4M3 rounding of the (exact) quotient, per head
    for h in (0, 1):
        y = (x[:, h, :] / scales[h]).astype(np.float32)
        assert np.array_equal(codes[:, h, :], torch_encode(y))
        assert np.array_equal(y.astype(np.float64) * 1.0, x[:, h, :].astype(np.float64) / float(scales[h]))
    # queries: one scale per (row, head)
    qc, sq = O.quantize_heads_e4m3(x[:7])
    assert sq.shape == (7, 3)
    for i in range(7):
        for h in (0, 1):
            amax = np.abs(x[i, h, :]).max()
            assert math.frexp(float(sq[i, h]))[0] == 0.5 and 224.0 < amax / sq[i, h] <= 448.0
            assert np.array_equal(qc[i, h], torch_encode((x[i, h] / sq[i, h]).astype(np.float32)))
        assert sq[i, 2] == 1.0 and not qc[i, 2].any()


def test_attention_fp8_exact_on_the_grid():
    """Operands on the E4M3 grid with a power-of-two scale per quantisation
    group (each group reaching 448 * 2^k) are quantised exactly, so the
    quantised attention equals plain attention on them."""
    rng = np.random.default_rng(4)
    pos = O.e4m3_decode(np.arange(1, 0x7F, dtype=np.uint8))

    def grid(shape, groups_axes, k):
        x = rng.choice(pos, size=shape) * rng.choice([-1.0, 1.0], size=shape)
        # force the maximum 448 once in every group
        it = np.ndindex(*[shape[a] for a in range(len(shape)) if a not in groups_axes])
        for idx in it:
            sl = [slice(None)] * len(shape)
            j = 0
            for a in range(len(shape)):
                if a not in groups_axes:
                    sl[a] = idx[j]
                    j += 1
            g = x[tuple(sl)]
            g.flat[rng.integers(g.size)] = 448.0
        return x * 2.0 ** k

    n_q, H, d = 5, 2, 8
    q = grid((n_q, H, d), (2,), -7)                 # per (row, head)
    k1, v1 = grid((6, H, d), (0, 2), -6), grid((6, H, d), (0, 2), -3)  # per head over the chunk
    k2, v2 = grid((9, H, d), (0, 2), -8), grid((9, H, d), (0, 2), -5)
    o8, l8 = O.attention_fp8(q, [k1, k2], [v1, v2], 0.3)
    o, l = O.group_attention(q, np.concatenate([k1, k2]), np.concatenate([v1, v2]), 0.3)
    np.testing.assert_allclose(o8, o, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(l8, l, rtol=1e-12, atol=1e-12)


def test_attention_fp8_scales_per_chunk():
    """The scale is per chunk: a chunk of small values next to a chunk of
    large ones keeps its own resolution, so the quantised attention stays
    near the exact one; one shared scale for both chunks would flush the
    small chunk's values (a pinned difference)."""
    rng = np.random.default_rng(5)
    n_q, H, d = 4, 1, 16
    q = rng.standard_normal((n_q, H, d))
    k1, k2 = rng.standard_normal((20, H, d)), rng.standard_normal((20, H, d))
    v1, v2 = 1e-3 * rng.standard_normal((20, H, d)), 1e3 * rng.standard_normal((20, H, d))
    # queries attend (almost) only to the first chunk
    k2 = k2 - 10.0 * np.sign(q.mean(axis=0, keepdims=True))
    o8, _ = O.attention_fp8(q, [k1, k2], [v1, v2], 1.0)
    o, _ = O.group_attention(q, np.concatenate([k1, k2]), np.concatenate([v1, v2]), 1.0)
    e_chunk = np.linalg.norm(o8 - o) / np.linalg.norm(o)
    # one scale shared by both chunks' V
    vv = np.concatenate([v1, v2])
    vc, sv = O.quantize_chunk_e4m3(vv)
    v_shared = O.e4m3_decode(vc) * sv[None, :, None]
    o_sh, _ = O.attention_fp8(q, [np.concatenate([k1, k2])], [v_shared], 1.0)
    e_shared = np.linalg.norm(o_sh - o) / np.linalg.norm(o)
    assert e_chunk < 0.1 and e_shared > 10 * e_chunk, (e_chunk, e_shared)


def test_attention_fp8_error_is_the_quantisation():
    """On Gaussian operands the quantised attention departs from the exact
    one by the E4M3 step (a few percent), neither zero nor more."""
    rng = np.random.default_rng(6)
    q, k, v = (rng.standard_normal((32, 2, 64)) for _ in range(3))
    o8, l8 = O.attention_fp8(q, [k], [v], 64 ** -0.5)
    o, l = O.group_attention(q, k, v, 64 ** -0.5)
    e = np.linalg.norm(o8 - o) / np.linalg.norm(o)
    assert 1e-3 < e < 8e-2, e
    assert np.abs(l8 - l).max() < 0.05
