"""Pins of the oracle's per-group attention and LSE merge against facts that
do not come from the oracle itself: brute force, closed forms, invariants and
a second library routine."""
import math

import numpy as np
import pytest
import torch

from oracle import dual_stream_attention, group_attention, lse_merge


def _brute_attention(q, k, v, scale):
    """Pure-Python softmax attention, one query/head at a time."""
    n_q, H, d = q.shape
    n_k = k.shape[0]
    o = np.zeros((n_q, H, d))
    lse = np.zeros((n_q, H))
    for i in range(n_q):
        for h in range(H):
            s = [scale * sum(q[i, h, t] * k[j, h, t] for t in range(d)) for j in range(n_k)]
            z = sum(math.exp(x) for x in s)
            lse[i, h] = math.log(z)
            for t in range(d):
                o[i, h, t] = sum(math.exp(s[j]) / z * v[j, h, t] for j in range(n_k))
    return o, lse


def test_brute_force_tiny(rng):
    q, k, v = rng.normal(size=(3, 2, 4)), rng.normal(size=(5, 2, 4)), rng.normal(size=(5, 2, 4))
    o, lse = group_attention(q, k, v, 0.7)
    ob, lb = _brute_attention(q, k, v, 0.7)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=1e-13, atol=1e-13)


def test_closed_form_two_keys():
    # scores 0 and ln 3 -> weights 1/4, 3/4 ; lse = ln 4
    q = np.zeros((1, 1, 2)); q[0, 0, 0] = 1.0
    k = np.zeros((2, 1, 2)); k[1, 0, 0] = math.log(3.0)
    v = np.array([[[1.0, 2.0]], [[5.0, -2.0]]])
    o, lse = group_attention(q, k, v, 1.0)
    np.testing.assert_allclose(o[0, 0], [0.25 * 1 + 0.75 * 5, 0.25 * 2 - 0.75 * 2], rtol=1e-14)
    assert abs(lse[0, 0] - math.log(4.0)) < 1e-14


def test_zero_query_is_uniform(rng):
    k, v = rng.normal(size=(7, 3, 8)), rng.normal(size=(7, 3, 8))
    o, lse = group_attention(np.zeros((2, 3, 8)), k, v, 0.3)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, math.log(7.0), rtol=1e-14)


def test_single_key(rng):
    q, k, v = rng.normal(size=(4, 2, 8)), rng.normal(size=(1, 2, 8)), rng.normal(size=(1, 2, 8))
    o, lse = group_attention(q, k, v, 0.5)
    np.testing.assert_allclose(o, np.broadcast_to(v[0], o.shape), rtol=1e-14)
    np.testing.assert_allclose(lse, 0.5 * np.einsum("qhd,hd->qh", q, k[0]), rtol=1e-13)


def test_key_permutation_invariance(rng):
    q, k, v = rng.normal(size=(5, 2, 8)), rng.normal(size=(9, 2, 8)), rng.normal(size=(9, 2, 8))
    p = rng.permutation(9)
    o1, l1 = group_attention(q, k, v, 0.4)
    o2, l2 = group_attention(q, k[p], v[p], 0.4)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)


def test_against_torch_sdpa(rng):
    q, k, v = rng.normal(size=(6, 3, 16)), rng.normal(size=(11, 3, 16)), rng.normal(size=(11, 3, 16))
    o, _ = group_attention(q, k, v, 16 ** -0.5)
    t = lambda x: torch.from_numpy(x).permute(1, 0, 2).unsqueeze(0)  # noqa: E731
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v))
    np.testing.assert_allclose(o, ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


def test_empty_group():
    o, lse = group_attention(np.ones((3, 2, 4)), np.zeros((0, 2, 4)), np.zeros((0, 2, 4)), 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def _split(rng, n_q=6, H=2, d=8, n_loc=5, n_hist=13):
    q = rng.normal(size=(n_q, H, d))
    kl, vl = rng.normal(size=(n_loc, H, d)), rng.normal(size=(n_loc, H, d))
    kh, vh = rng.normal(size=(n_hist, H, d)) + 0.5, rng.normal(size=(n_hist, H, d))
    return q, kl, vl, kh, vh


def test_merge_equals_monolithic(rng):
    q, kl, vl, kh, vh = _split(rng)
    r = dual_stream_attention(q, kl, vl, kh, vh, 0.35)
    o_m, l_m = group_attention(q, np.concatenate([kl, kh]), np.concatenate([vl, vh]), 0.35)
    np.testing.assert_allclose(r["a_full"], o_m, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["lse_full"], l_m, rtol=1e-13)
    np.testing.assert_allclose(r["a_loc"], r["o_loc"], rtol=0, atol=0)
    np.testing.assert_allclose(r["delta"], o_m - r["o_loc"], rtol=1e-12, atol=1e-14)


def test_merge_three_way_equals_monolithic(rng):
    q = rng.normal(size=(4, 2, 8))
    ks = [rng.normal(size=(n, 2, 8)) for n in (3, 7, 2)]
    vs = [rng.normal(size=(n, 2, 8)) for n in (3, 7, 2)]
    parts = [group_attention(q, k, v, 0.5) for k, v in zip(ks, vs)]
    o, lse, a0, _ = lse_merge([p[0] for p in parts], [p[1] for p in parts])
    o_m, l_m = group_attention(q, np.concatenate(ks), np.concatenate(vs), 0.5)
    np.testing.assert_allclose(o, o_m, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, l_m, rtol=1e-13)


def test_merge_sigmoid_form(rng):
    # two groups: A_full = s*O_hist + (1-s)*O_loc, s = sigmoid(lse_hist - lse_loc)
    q, kl, vl, kh, vh = _split(rng)
    r = dual_stream_attention(q, kl, vl, kh, vh, 0.35)
    s = 1.0 / (1.0 + np.exp(-(r["lse_hist"] - r["lse_loc"])))
    ref = s[..., None] * r["o_hist"] + (1 - s[..., None]) * r["o_loc"]
    np.testing.assert_allclose(r["a_full"], ref, rtol=1e-12, atol=1e-14)


def test_duplicate_history_doubles_mass(rng):
    q, kl, vl, _, _ = _split(rng)
    r = dual_stream_attention(q, kl, vl, kl.copy(), vl.copy(), 0.35)
    np.testing.assert_allclose(r["a_full"], r["a_loc"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["lse_full"], r["lse_loc"] + math.log(2.0), rtol=1e-13)


def test_merge_is_not_plain_mean(rng):
    # the groups carry different softmax mass, so averaging is wrong
    q, kl, vl, kh, vh = _split(rng)
    r = dual_stream_attention(q, kl, vl, kh, vh, 0.35)
    assert np.max(np.abs(r["lse_loc"] - r["lse_hist"])) > 0.1
    assert np.max(np.abs(r["a_full"] - 0.5 * (r["o_loc"] + r["o_hist"]))) > 1e-3


def test_merge_empty_history(rng):
    q, kl, vl, _, _ = _split(rng)
    r = dual_stream_attention(q, kl, vl, np.zeros((0, 2, 8)), np.zeros((0, 2, 8)), 0.35)
    np.testing.assert_array_equal(r["a_full"], r["a_loc"])
    np.testing.assert_array_equal(r["lse_full"], r["lse_loc"])
    assert np.all(r["delta"] == 0)


def test_merge_all_empty():
    o, lse, _, d = lse_merge([np.zeros((2, 1, 4))] * 2, [np.full((2, 1), -np.inf)] * 2)
    assert np.all(o == 0) and np.all(np.isneginf(lse)) and np.all(d == 0)


@pytest.mark.parametrize("shift", [0.0, 30.0])
def test_merge_shift_stability(rng, shift):
    # adding a constant to every score of one group shifts its lse only
    q, kl, vl, kh, vh = _split(rng)
    o1, l1 = group_attention(q, kh, vh, 0.35)
    o2, l2 = lse_merge([o1], [l1 + shift])[:2]
    np.testing.assert_allclose(o2, o1, rtol=1e-13)
    np.testing.assert_allclose(l2, l1 + shift, rtol=1e-13)
