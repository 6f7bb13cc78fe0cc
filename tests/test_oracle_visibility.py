"""Pins for the oracle's visibility / mask predicate (CPU only).

The pages state the geometry as key ranges: causal keeps keys up to the query's
offset position, and the window keeps keys closer than `window` to it, with or
without causal (ferrotensor-backend flash_attention_v2_backward.wgsl,
fab2_visible and fab2_key_range).  These tests check the predicate against
closed-form per-row ranges and counts derived from that statement, not by
re-evaluating the predicate.
"""
import numpy as np
import pytest

import oracle


def _rows(sq, sk, spec):
    return oracle.visible(np.arange(sq), np.arange(sk), sq, sk, spec)


@pytest.mark.parametrize("s", [1, 7, 64, 300])
def test_causal_count_closed_form(s):
    vis = _rows(s, s, oracle.Spec(scale=1.0, causal=True))
    assert vis.sum() == s * (s + 1) // 2
    for i in range(s):  # row i sees exactly keys 0..i, contiguous
        assert vis[i].sum() == i + 1 and vis[i, : i + 1].all()


def test_causal_window_geometry_of_the_extras_workload():
    # causal, offset 0, window 512, S = 2048: row i sees keys (i-512, i], i.e. min(i+1, 512) keys
    s, w = 2048, 512
    vis = _rows(s, s, oracle.Spec(scale=1.0, causal=True, window=w))
    per_row = vis.sum(axis=1)
    assert np.array_equal(per_row, np.minimum(np.arange(s) + 1, w))
    assert vis.sum() == 917760
    i = 1000
    assert vis[i, i - w + 1:i + 1].all() and not vis[i, i - w] and not vis[i, i + 1]


@pytest.mark.parametrize("sq,sk,off,w", [(5, 9, 4, 3), (16, 40, 24, 5), (33, 33, 0, 1), (10, 12, 2, 100)])
def test_offset_and_symmetric_window_ranges(sq, sk, off, w):
    # causal with offset: row i sees keys 0..i+off (bottom-right aligned when sk = sq + off)
    vis = _rows(sq, sk, oracle.Spec(scale=1.0, causal=True, causal_offset=off))
    assert np.array_equal(vis.sum(1), np.minimum(np.arange(sq) + off + 1, sk))
    # non-causal window: keys in (i+off-w, i+off+w) clipped to [0, sk)
    vis = _rows(sq, sk, oracle.Spec(scale=1.0, causal=False, causal_offset=off, window=w))
    qa = np.arange(sq) + off
    lo = np.maximum(0, qa - w + 1)
    hi = np.minimum(sk, qa + w)
    assert np.array_equal(vis.sum(1), np.maximum(hi - lo, 0))
    # causal window: keys in (i+off-w, i+off]
    vis = _rows(sq, sk, oracle.Spec(scale=1.0, causal=True, causal_offset=off, window=w))
    hi = np.minimum(sk, qa + 1)
    assert np.array_equal(vis.sum(1), np.maximum(hi - lo, 0))


def test_window_one_is_the_diagonal():
    vis = _rows(20, 20, oracle.Spec(scale=1.0, causal=False, window=1))
    assert np.array_equal(vis, np.eye(20, dtype=bool))


def test_large_window_is_no_window():
    for causal in (False, True):
        a = _rows(13, 17, oracle.Spec(scale=1.0, causal=causal, causal_offset=3))
        b = _rows(13, 17, oracle.Spec(scale=1.0, causal=causal, causal_offset=3, window=17 + 3))
        assert np.array_equal(a, b)


def test_out_of_range_is_invisible():
    vis = oracle.visible(np.arange(12), np.arange(12), 10, 9, oracle.Spec(scale=1.0))
    assert not vis[10:].any() and not vis[:, 9:].any() and vis[:10, :9].all()


def test_mask_exclusion_uses_the_sentinel_in_fp32():
    vis = np.ones((1, 6), dtype=bool)
    m = np.array([[0.0, -1e30, -2e30, -5e29, np.float32(-1e30) * np.float32(0.999999), 3.0]], np.float32)
    cnt = oracle.counted(vis, m)
    assert cnt.tolist() == [[True, False, False, True, True, True]]
