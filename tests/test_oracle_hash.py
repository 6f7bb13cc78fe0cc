"""Pins for the oracle's dropout hash (CPU only).

fmix32 is pinned to published MurmurHash3_x86_32 vectors (tests/golden); the
keep-mask composition built on it -- our own specification, since the pages
call a dropout helper whose definition is not on them -- is pinned by its
statistical properties (keep rate, no lag-1 correlation along i or j, a
bijection in j within a row, independence across seeds and heads) and by its
structure: a row's draws depend only on its flat index (b*H + h)*Sq + i, and
the oracle backward drops exactly the pairs of each query row's own index
(recovered from dV with one-hot dO rows, GQA with Sq != Sk).
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "murmur3_x86_32.txt")


def _rotl(x, r):
    return ((x << r) | (x >> (32 - r))) & 0xFFFFFFFF


def _murmur3_x86_32(data: bytes, seed: int) -> int:
    # Body of MurmurHash3_x86_32; the finaliser is the oracle's fmix32 under test.
    c1, c2 = 0xCC9E2D51, 0x1B873593
    h = seed & 0xFFFFFFFF
    n = len(data) // 4
    for b in range(n):
        k = int.from_bytes(data[4 * b:4 * b + 4], "little")
        k = (k * c1) & 0xFFFFFFFF
        k = _rotl(k, 15)
        k = (k * c2) & 0xFFFFFFFF
        h ^= k
        h = _rotl(h, 13)
        h = (h * 5 + 0xE6546B64) & 0xFFFFFFFF
    tail = data[4 * n:]
    k = 0
    for t in range(len(tail) - 1, -1, -1):
        k ^= tail[t] << (8 * t)
    if tail:
        k = (k * c1) & 0xFFFFFFFF
        k = _rotl(k, 15)
        k = (k * c2) & 0xFFFFFFFF
        h ^= k
    h ^= len(data)
    return int(oracle.fmix32(np.uint64(h)))


def _vectors():
    out = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, seed, want = line.split()
            data = b"" if key == "-" else bytes.fromhex(key)
            out.append((data, int(seed, 16), int(want, 16)))
    return out


@pytest.mark.parametrize("data,seed,want", _vectors())
def test_murmur3_published_vectors(data, seed, want):
    assert _murmur3_x86_32(data, seed) == want


def test_fmix32_is_bijective_on_a_block():
    x = np.arange(1 << 20, dtype=np.uint64)
    y = oracle.fmix32(x)
    assert np.unique(y).size == x.size


def test_threshold_exact():
    assert oracle.dropout_threshold(0.0) == 0
    assert oracle.dropout_threshold(0.1) == 429496736  # 0.1f = 13421773 * 2^-27
    assert oracle.dropout_threshold(0.5) == 1 << 31


def test_keep_rate_and_independence():
    p = 0.1
    B, H, S = 2, 4, 256
    keeps = np.stack([np.stack([oracle.dropout_keep(7, b, h, H, S, np.arange(S), np.arange(S), p)
                                for h in range(H)]) for b in range(B)])
    n = keeps.size
    rate = keeps.mean()
    sigma = np.sqrt(p * (1 - p) / n)
    assert abs(rate - (1 - p)) < 5 * sigma
    x = keeps.astype(np.float64)
    for axis in (-1, -2):
        a = np.moveaxis(x, axis, -1)
        c = np.corrcoef(a[..., :-1].ravel(), a[..., 1:].ravel())[0, 1]
        assert abs(c) < 5 / np.sqrt(a[..., 1:].size), (axis, c)
    # different heads / batches / seeds give different patterns
    assert (keeps[0, 0] != keeps[0, 1]).mean() > 0.1
    assert (keeps[0, 0] != keeps[1, 0]).mean() > 0.1
    other = oracle.dropout_keep(8, 0, 0, H, S, np.arange(S), np.arange(S), p)
    assert (keeps[0, 0] != other).mean() > 0.1


def test_row_hash_is_bijection_in_j():
    # u = fmix32(r ^ j*odd) is injective in j, so no two keys of a row share a draw.
    j = np.arange(1 << 20)
    u = oracle.dropout_draw(3, 0, 5, 8, 100, [42], j)[0]
    assert np.unique(u).size == j.size
    # and rows of one head differ (the row key enters before the column mix)
    u2 = oracle.dropout_draw(3, 0, 5, 8, 100, [43], j[:4096])[0]
    assert (u[:4096] != u2).mean() > 0.99


def test_p_zero_keeps_everything_and_multiplier():
    spec = oracle.Spec(scale=1.0, dropout_p=0.0, seed=9)
    m = oracle.dropout_multiplier(spec, 0, 0, 2, 16, np.arange(16), np.arange(16))
    assert np.all(m == 1.0)
    spec = oracle.Spec(scale=1.0, dropout_p=0.25, seed=9)
    m = oracle.dropout_multiplier(spec, 0, 0, 2, 16, np.arange(16), np.arange(16))
    assert set(np.unique(m)) <= {0.0, 1.0 / 0.75}


def test_draw_depends_only_on_the_flat_row_index():
    """The reading keys each row by its flat index (b*H + h)*Sq + i: row (b, h, i) of
    a B x H x Sq problem draws what row (b*H + h)*Sq + i of a one-head problem with
    B*H*Sq rows draws.  A slip in the flattening (Sk for Sq, b and h swapped, a
    dropped term) moves rows and fails this."""
    seed, B, H, Sq = 11, 3, 5, 37
    cols = np.arange(70)
    flat = oracle.dropout_draw(seed, 0, 0, 1, B * H * Sq, np.arange(B * H * Sq), cols)
    for b in range(B):
        for h in range(H):
            rows = np.arange(Sq)
            got = oracle.dropout_draw(seed, b, h, H, Sq, rows, cols)
            np.testing.assert_array_equal(got, flat[(b * H + h) * Sq + rows])
    # and the key enters on its own: column j of a row does not depend on the other columns asked for
    one = oracle.dropout_draw(seed, 1, 2, H, Sq, [4], [9])
    np.testing.assert_array_equal(one[0, 0], oracle.dropout_draw(seed, 1, 2, H, Sq, [4], cols)[0, 9])


def test_backward_drops_the_pairs_of_its_own_rows():
    """The oracle backward applies the keep bits of each query row's own flat index
    (query head, not KV head; Sq, not Sk): with one-hot dO rows and no other
    exclusion, dV[b, kvh, j, g*Sq + i] = P_ij M_ij of query head kvh*group + g, so
    its nonzero pattern is the keep pattern.  GQA with Sq != Sk catches a hash fed
    the KV head or the key length."""
    B, Hq, Hkv, Sq, Sk = 2, 4, 2, 6, 9
    group = Hq // Hkv
    D = group * Sq
    p, seed = 0.4, 23
    rng = np.random.default_rng(5)
    q = rng.standard_normal((B, Hq, Sq, D)) * 0.3
    k = rng.standard_normal((B, Hkv, Sk, D)) * 0.3
    v = rng.standard_normal((B, Hkv, Sk, D))
    do = np.zeros((B, Hq, Sq, D))
    for h in range(Hq):
        for i in range(Sq):
            do[:, h, i, (h % group) * Sq + i] = 1.0
    spec = oracle.Spec(scale=0.5, dropout_p=p, seed=seed)
    o, lse = oracle.forward(q, k, v, spec)
    _, _, _, dv = oracle.backward(q, k, v, o, do, lse, spec)
    flat = oracle.dropout_keep(seed, 0, 0, 1, B * Hq * Sq, np.arange(B * Hq * Sq), np.arange(Sk), p)
    for b in range(B):
        for h in range(Hq):
            kvh, g = h // group, h % group
            got = dv[b, kvh, :, g * Sq:(g + 1) * Sq].T != 0.0  # [i, j]
            want = flat[(b * Hq + h) * Sq:(b * Hq + h + 1) * Sq]
            np.testing.assert_array_equal(got, want)
    assert 0 < flat.mean() < 1
