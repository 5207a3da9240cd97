"""Pins of the oracle's layer selection, key grouping, KV accounting and
post-switch projection."""
import math
import os

import numpy as np
import pytest

from oracle import (accumulate_stats, dual_stream_attention, epsilon_from_stats,
                    group_attention, kv_bytes_retained, local_attn_proj,
                    remaining_kv_fraction, ridge_lambda, select_layers, solve_dw,
                    stream_groups, stream_groups_kept)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute_select(eps, K):
    # rank_i = number of layers strictly ahead of i (lower eps, or equal and lower index)
    N = len(eps)
    rank = [sum(1 for j in range(N) if eps[j] < eps[i] or (eps[j] == eps[i] and j < i))
            for i in range(N)]
    sel = [None] * K
    for i, r in enumerate(rank):
        if r < K:
            sel[r] = i
    return sel


def test_select_matches_brute_force(rng):
    for trial in range(20):
        N = int(rng.integers(1, 41))
        K = int(rng.integers(0, N + 1))
        eps = rng.choice([0.5, 1.0, 2.0, 3.5], size=N) if trial % 2 else rng.uniform(size=N)
        sel, is_local, st = select_layers(eps, K)
        assert st == 0
        assert list(sel) == _brute_select(list(eps), K)
        assert is_local.sum() == K and all(is_local[i] == 1 for i in sel)


def test_select_ties_lower_index_first():
    sel, _, _ = select_layers([2.0, 1.0, 1.0, 0.5, 1.0], 3)
    assert list(sel) == [3, 1, 2]


def test_select_nan_is_error():
    _, _, st = select_layers([0.1, float("nan"), 0.3], 1)
    assert st == 1


def test_select_permutation_equivariant(rng):
    eps = rng.uniform(size=30)
    p = rng.permutation(30)
    s1, _, _ = select_layers(eps, 15)
    s2, _, _ = select_layers(eps[p], 15)
    assert sorted(p[s2]) == sorted(s1)


def test_select_picks_planted_linear_layers(rng):
    # layers whose residual is exactly linear in A_loc have eps ~ ridge bias
    D, n, N = 8, 120, 10
    planted = {2, 5, 7}
    eps = []
    for layer in range(N):
        a = rng.normal(size=(n, D))
        w = rng.normal(size=(D, D)) / math.sqrt(D)
        if layer in planted:
            delta = a @ (0.1 * rng.normal(size=(D, D))) @ np.linalg.inv(w)
        else:
            delta = rng.normal(size=(n, D))
        G, C, r2 = accumulate_stats(a, delta, w)
        dW, _ = solve_dw(G, C, ridge_lambda(G, 0.0, 1e-3))
        eps.append(epsilon_from_stats(G, C, r2, dW))
    sel, _, _ = select_layers(eps, 3)
    assert set(sel.tolist()) == planted


def test_stream_groups_partition():
    T = 7
    for c in range(6):
        loc, hist = stream_groups(c, T)
        idx = [i for a, b in loc + hist for i in range(a, b)]
        assert sorted(idx) == list(range((c + 1) * T))  # disjoint, cover all keys
        assert loc[0] == (0, T)  # sink always local
        if c >= 1:
            assert loc[1] == (c * T, (c + 1) * T)
        assert (hist == []) == (c <= 1)


def test_stream_groups_kept_reduces_to_full_history():
    """A layer that never dropped history (first_kept = 1) has the groups of
    the plain stream."""
    T = 5
    for c in range(8):
        assert stream_groups_kept(c, T, 1) == stream_groups(c, T)


def test_stream_groups_kept_against_held_chunk_sets():
    """Brute force on chunk sets: a layer is full through chunk s - 1, becomes
    an L-Layer at the switch (it then holds the sink and its current chunk
    only), and re-enters warmup at chunk r (holding the sink and chunk r - 1).
    From then on every arriving chunk is kept.  At each warmup chunk c >= r the
    local group must be {sink, c} and the history every other held chunk below
    c; the oracle's ranges must name exactly those chunks."""
    T = 3

    def chunks(ranges):
        out = set()
        for a, b in ranges:
            assert a % T == 0 and b % T == 0
            out |= set(range(a // T, b // T))
        return out

    for s in range(2, 6):
        for r in range(s + 1, s + 5):
            held = set(range(s))            # full through the warmup
            for c in range(s, r):           # post-switch L-Layer: sink + current
                held = {0, c}
            for c in range(r, r + 5):       # re-entered warmup
                held.add(c)
                loc, hist = stream_groups_kept(c, T, r - 1)
                assert chunks(loc) == {0, c}
                assert chunks(hist) == held - {0, c}
                assert not (chunks(loc) & chunks(hist))


def test_table2_remaining_kv_identity():
    """Table 2 (EN review, Main Results and Ablation Study) prints the
    remaining-KV percentages in tests/golden/table2_remaining_kv.txt.  With
    r = local keys / full keys per layer, 1 - x (1 - r) reproduces each
    printed value to its one decimal."""
    rows = []
    with open(os.path.join(GOLDEN, "table2_remaining_kv.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, x, pct, r_num, r_den = line.split()[:5]
                rows.append((name, float(x), float(pct), int(r_num) / int(r_den)))
    assert len(rows) == 5
    for name, x, pct, r in rows:
        assert round(100 * remaining_kv_fraction(x, r), 1) == pct, name
    # a wrong reading (x as a memory fraction) does not reproduce the table
    assert any(round(100 * (1 - x), 1) != pct for _, x, pct, _ in rows)


@pytest.mark.parametrize("n_layers,K,c,expect", [(30, 15, 19, 0.55), (40, 20, 39, 0.525)])
def test_kv_accounting_streams(n_layers, K, c, expect):
    T, D = 4680, 1536
    loc, hist = stream_groups(c, T)
    n_loc = sum(b - a for a, b in loc)
    n_full = n_loc + sum(b - a for a, b in hist)
    kept = kv_bytes_retained([n_loc] * K + [n_full] * (n_layers - K), D)
    full = kv_bytes_retained([n_full] * n_layers, D)
    assert kept / full == pytest.approx(expect, rel=1e-12)
    assert kept / full == pytest.approx(remaining_kv_fraction(K / n_layers, n_loc / n_full))
    assert full == n_layers * 4 * n_full * D


def test_local_attn_proj_composition(rng):
    q, k, v = rng.normal(size=(5, 2, 4)), rng.normal(size=(9, 2, 4)), rng.normal(size=(9, 2, 4))
    w = rng.normal(size=(8, 8))
    y = local_attn_proj(q, k, v, w, 0.5)
    o, _ = group_attention(q, k, v, 0.5)
    for i in range(5):
        row = o[i].reshape(-1)
        np.testing.assert_allclose(y[i], [sum(row[t] * w[t, j] for t in range(8)) for j in range(8)],
                                   rtol=1e-12)
    # F-layer on all keys equals the merged dual-stream output projected by W
    r = dual_stream_attention(q, k[:3], v[:3], k[3:], v[3:], 0.5)
    np.testing.assert_allclose(y, r["a_full"].reshape(5, -1) @ w, rtol=1e-12, atol=1e-13)
