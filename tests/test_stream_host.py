"""Host logic of the chunked stream (no GPU): cache slots, eviction and the
key accounting against the oracle's grouping."""
import pytest
import torch

import oracle as O
from kv_cache_absorption_amd.stream import LayerKV, keys_retained, kv_bytes


def _fill(kv, c, T, H, d):
    val = torch.full((T, H, d), float(c))
    kv.write(c, val, -val)


def test_layer_cache_groups_follow_oracle():
    T, H, d = 3, 2, 4
    kv = LayerKV(2, T, H, d, torch.float32, "cpu")  # grows past two slots
    for c in range(7):
        _fill(kv, c, T, H, d)
        loc, hist = kv.warmup_groups(c)
        oloc, ohist = O.stream_groups(c, T)
        for got, want in ((loc, oloc), (hist, ohist)):
            assert [k.shape[0] for k, _ in got] == [b - a for a, b in want]
            for (k, v), (a, b) in zip(got, want):
                # row r of the key sequence holds chunk r // T
                assert torch.equal(k[:, 0, 0], torch.arange(a, b).div(T, rounding_mode="floor").float())
                assert torch.equal(v, -k)
        assert kv.keys_held(c) == (c + 1) * T
        (k_all, _), = kv.attend_all(c)
        assert k_all.shape[0] == (c + 1) * T
    assert kv.capacity >= 7


def test_eviction_keeps_sink_and_current():
    T, H, d = 2, 1, 4
    kv = LayerKV(6, T, H, d, torch.float32, "cpu")
    for c in range(6):
        _fill(kv, c, T, H, d)
    kv.evict_history()
    assert kv.capacity == 2 and kv.local_only
    assert kv.bytes_allocated() == 2 * 2 * T * H * d * 4
    for c in range(6, 9):
        _fill(kv, c, T, H, d)
        (k, v), = kv.attend_all(c)
        # the local group of chunk c: sink rows then the current chunk's rows
        assert k[:, 0, 0].tolist() == [0.0] * T + [float(c)] * T
        oloc, _ = O.stream_groups(c, T)
        assert kv.keys_held(c) == sum(b - a for a, b in oloc)


def test_keys_retained_matches_oracle_bytes():
    T, D = 4680, 1536
    flags = [1, 0] * 15
    for c in (0, 1, 5, 19):
        n = keys_retained(c, T, flags)
        oloc, ohist = O.stream_groups(c, T)
        n_loc = sum(b - a for a, b in oloc)
        n_full = n_loc + sum(b - a for a, b in ohist)
        assert n == [n_loc if f else n_full for f in flags]
        assert kv_bytes(n, D) == O.kv_bytes_retained(n, D)


def _check_groups(kv, c, T, oloc, ohist):
    loc, hist = kv.warmup_groups(c)
    for got, want in ((loc, oloc), (hist, ohist)):
        got_chunks = [int(x) for k, _ in got for x in k[:, 0, 0].tolist()]
        want_chunks = [r // T for a, b in want for r in range(a, b)]
        assert got_chunks == want_chunks


def test_reentered_warmup_groups_follow_oracle():
    """An L-Layer that re-enters warmup holds its sink and last chunk, then
    keeps every arriving chunk; its groups are the oracle's for that
    first-kept chunk.  A layer that stayed full keeps the plain groups."""
    T, H, d = 2, 1, 4
    for post_chunks in (1, 3):
        kv_l = LayerKV(6, T, H, d, torch.float32, "cpu")
        kv_f = LayerKV(6, T, H, d, torch.float32, "cpu")
        for c in range(5):                      # warmup 0..4
            _fill(kv_l, c, T, H, d)
            _fill(kv_f, c, T, H, d)
        kv_l.evict_history()                    # switch: kv_l is an L-Layer
        r = 5 + post_chunks
        for c in range(5, r):                   # post-switch chunks
            _fill(kv_l, c, T, H, d)
            _fill(kv_f, c, T, H, d)
        for kv in (kv_l, kv_f):
            kv.keep_from(r)                     # re-enter warmup at chunk r
        assert not kv_l.local_only
        for c in range(r, r + 4):
            _fill(kv_l, c, T, H, d)
            _fill(kv_f, c, T, H, d)
            _check_groups(kv_l, c, T, *O.stream_groups_kept(c, T, r - 1))
            _check_groups(kv_f, c, T, *O.stream_groups(c, T))
            assert kv_l.keys_held(c) == T * (2 + c - (r - 1))
            assert kv_f.keys_held(c) == T * (c + 1)


def test_reentry_right_after_eviction_holds_sink_only():
    """With no chunk written since the eviction, re-entering at chunk r keeps
    only the sink: history starts at r."""
    T, H, d = 2, 1, 4
    kv = LayerKV(4, T, H, d, torch.float32, "cpu")
    for c in range(4):
        _fill(kv, c, T, H, d)
    kv.evict_history()
    kv.keep_from(4)
    for c in range(4, 7):
        _fill(kv, c, T, H, d)
        _check_groups(kv, c, T, *O.stream_groups_kept(c, T, 4))


def test_stream_rejects_bad_statistics_options():
    """The statistics grouping options are checked before anything is
    allocated (no GPU needed): an unknown form, or fewer than one chunk per
    rank-k update."""
    from kv_cache_absorption_amd.stream import IspaStream
    with pytest.raises(ValueError):
        IspaStream(1, 2, 128, 64, 2, "cpu", stats="other")
    with pytest.raises(ValueError):
        IspaStream(1, 2, 128, 64, 2, "cpu", stats_chunks=0)
