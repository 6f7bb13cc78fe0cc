"""Pins for the oracle's forward and backward (CPU only).

* finite differences of the fp64 forward loss sum(dO * O), every feature;
* a brute-force softmax Jacobian per row;
* the invariants sum_j dS_ij = 0 and sum_j dK_j = 0;
* torch fp64 autograd and scaled_dot_product_attention as library cross-checks;
* closed forms (single counted key, V = 0, Q = 0 / uniform attention);
* GQA == MHA with repeated K/V; the sampled-row/key helpers == the full backward.
"""
import math

import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(1234)


def _problem(B, Hq, Hkv, Sq, Sk, D, rng=RNG, mask_kind=None):
    q = rng.standard_normal((B, Hq, Sq, D))
    k = rng.standard_normal((B, Hkv, Sk, D))
    v = rng.standard_normal((B, Hkv, Sk, D))
    do = rng.standard_normal((B, Hq, Sq, D))
    mask = None
    if mask_kind == "mixed":
        # finite additive entries plus sentinel exclusions, shared across heads ([B,1,Sq,Sk])
        mask = (0.5 * rng.standard_normal((B, 1, Sq, Sk))).astype(np.float32)
        mask[rng.random((B, 1, Sq, Sk)) < 0.2] = np.float32(-1e30)
    return q, k, v, do, mask


FEATURES = [
    dict(spec=oracle.Spec(scale=0.5), shape=(1, 2, 2, 5, 5, 4), mask=None),
    dict(spec=oracle.Spec(scale=0.7, causal=True), shape=(1, 2, 1, 6, 6, 4), mask=None),
    dict(spec=oracle.Spec(scale=0.6, causal=True, causal_offset=2, window=3), shape=(1, 4, 2, 5, 7, 4), mask=None),
    dict(spec=oracle.Spec(scale=0.6, causal=False, causal_offset=1, window=2), shape=(1, 2, 1, 7, 9, 3), mask=None),
    dict(spec=oracle.Spec(scale=0.4, causal=True, dropout_p=0.3, seed=77), shape=(2, 2, 1, 6, 6, 4), mask=None),
    dict(spec=oracle.Spec(scale=0.5, causal=True, causal_offset=1, window=4, dropout_p=0.25, seed=5),
         shape=(1, 4, 2, 7, 8, 4), mask="mixed"),
]


def _loss(q, k, v, do, spec, mask):
    o, _ = oracle.forward(q, k, v, spec, mask)
    return float((do * o).sum())


@pytest.mark.parametrize("case", range(len(FEATURES)))
def test_finite_differences(case):
    f = FEATURES[case]
    spec = f["spec"]
    rng = np.random.default_rng(100 + case)
    q, k, v, do, mask = _problem(*f["shape"], rng=rng, mask_kind=f["mask"])
    o, lse = oracle.forward(q, k, v, spec, mask)
    delta, dq, dk, dv = oracle.backward(q, k, v, o, do, lse, spec, mask)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            orig = x[idx]
            x[idx] = orig + eps
            lp = _loss(q, k, v, do, spec, mask)
            x[idx] = orig - eps
            lm = _loss(q, k, v, do, spec, mask)
            x[idx] = orig
            num[idx] = (lp - lm) / (2 * eps)
        scale = max(1.0, np.abs(num).max())
        assert np.abs(num - g).max() < 1e-7 * scale, name


def test_softmax_jacobian_per_row():
    spec = oracle.Spec(scale=0.5, causal=True, causal_offset=1, window=5, dropout_p=0.2, seed=3)
    q, k, v, do, mask = _problem(1, 2, 1, 8, 9, 6, rng=np.random.default_rng(7), mask_kind="mixed")
    o, lse = oracle.forward(q, k, v, spec, mask)
    delta = np.einsum("bhsd,bhsd->bhs", do, o)
    for h in range(2):
        rows = np.arange(8)
        cols = np.arange(9)
        p, mm, ds = oracle.backward_block(q, k, v, do, lse, delta, spec, mask, 0, h, rows, cols)
        dp = mm * (do[0, h] @ v[0, 0].T)
        for i in rows:
            pi = p[i]
            J = np.diag(pi) - np.outer(pi, pi)  # d softmax / d scores over the row
            np.testing.assert_allclose(J @ dp[i], ds[i], rtol=0, atol=1e-12)


def test_invariants_row_and_key_sums():
    spec = oracle.Spec(scale=0.3, causal=True, window=6, dropout_p=0.15, seed=11)
    q, k, v, do, mask = _problem(2, 4, 2, 12, 12, 8, rng=np.random.default_rng(8), mask_kind="mixed")
    o, lse = oracle.forward(q, k, v, spec, mask)
    delta, dq, dk, dv = oracle.backward(q, k, v, o, do, lse, spec, mask)
    for b in range(2):
        for h in range(4):
            _, _, ds = oracle.backward_block(q, k, v, do, lse, delta, spec, mask, b, h, np.arange(12), np.arange(12))
            assert np.abs(ds.sum(axis=1)).max() < 1e-12
    # shifting every key of a KV head by one vector leaves softmax unchanged => sum_j dK_j = 0
    assert np.abs(dk.sum(axis=2)).max() < 1e-12


def _torch_reference(q, k, v, do, spec, mask):
    """Masked softmax attention in torch fp64 with the oracle's visibility and dropout multiplier."""
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    g = Hq // Hkv
    add = np.zeros((B, Hq, Sq, Sk))
    mul = np.ones((B, Hq, Sq, Sk))
    for b in range(B):
        for h in range(Hq):
            vis = oracle.visible(np.arange(Sq), np.arange(Sk), Sq, Sk, spec)
            mv = None if mask is None else np.broadcast_to(mask, (B, Hq, Sq, Sk))[b, h].astype(np.float64)
            cnt = oracle.counted(vis, mv)
            add[b, h] = np.where(cnt, 0.0 if mv is None else mv, -np.inf)
            mul[b, h] = oracle.dropout_multiplier(spec, b, h, Hq, Sq, np.arange(Sq), np.arange(Sk))
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    kk = tk.repeat_interleave(g, dim=1)
    vv = tv.repeat_interleave(g, dim=1)
    s = spec.scale * torch.matmul(tq, kk.transpose(-1, -2).contiguous()) + torch.tensor(add)
    p = torch.softmax(s, dim=-1)
    o = torch.matmul(p * torch.tensor(mul), vv)
    (o * torch.tensor(do)).sum().backward()
    return o.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("case", [0, 2, 3, 4, 5])
def test_torch_autograd_cross_check(case):
    f = FEATURES[case]
    spec = f["spec"]
    B, Hq, Hkv, Sq, Sk, D = f["shape"]
    q, k, v, do, mask = _problem(B, Hq, Hkv, 3 * Sq, 3 * Sk, 8, rng=np.random.default_rng(200 + case),
                                 mask_kind=f["mask"])
    if mask is not None:  # keep each row's own position counted (torch softmax of all -inf is NaN)
        i = np.arange(3 * Sq)
        j = i + spec.causal_offset
        ok = j < 3 * Sk
        mask[:, :, i[ok], j[ok]] = 0.0
    o, lse = oracle.forward(q, k, v, spec, mask)
    _, dq, dk, dv = oracle.backward(q, k, v, o, do, lse, spec, mask)
    to, tdq, tdk, tdv = _torch_reference(q, k, v, do, spec, mask)
    for a, b in ((o, to), (dq, tdq), (dk, tdk), (dv, tdv)):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("causal,off,window", [(False, 0, 0), (True, 0, 0), (True, 3, 4), (False, 2, 3)])
def test_forward_matches_torch_sdpa(causal, off, window):
    rng = np.random.default_rng(9)
    B, Hq, Hkv, Sq, Sk, D = 2, 4, 2, 10, 13, 16
    q, k, v, do, _ = _problem(B, Hq, Hkv, Sq, Sk, D, rng=rng)
    mask = (0.3 * rng.standard_normal((B, 1, Sq, Sk))).astype(np.float32)
    spec = oracle.Spec(scale=1 / math.sqrt(D), causal=causal, causal_offset=off, window=window)
    o, lse = oracle.forward(q, k, v, spec, mask)
    vis = oracle.visible(np.arange(Sq), np.arange(Sk), Sq, Sk, spec)
    add = np.where(vis[None, None], mask.astype(np.float64), -np.inf)
    tout = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q), torch.tensor(k), torch.tensor(v), attn_mask=torch.tensor(add),
        scale=spec.scale, enable_gqa=True)
    np.testing.assert_allclose(o, tout.numpy(), rtol=1e-11, atol=1e-11)
    # log-sum-exp against scipy's routine on the same counted scores
    from scipy.special import logsumexp
    kk = np.repeat(k, Hq // Hkv, axis=1)
    s = spec.scale * np.einsum("bhid,bhjd->bhij", q, kk) + add
    np.testing.assert_allclose(lse, logsumexp(s, axis=-1), rtol=1e-12, atol=1e-12)


def test_single_counted_key_gives_zero_dq_row():
    # causal row 0 sees only key 0: P = 1, so dS = 0 and dQ_0 = 0, with or without dropout.
    for p in (0.0, 0.5):
        spec = oracle.Spec(scale=0.9, causal=True, dropout_p=p, seed=1)
        q, k, v, do, _ = _problem(1, 2, 2, 9, 9, 4)
        o, lse = oracle.forward(q, k, v, spec)
        _, dq, _, _ = oracle.backward(q, k, v, o, do, lse, spec)
        assert np.abs(dq[:, :, 0]).max() < 1e-14


def test_zero_values_closed_form():
    spec = oracle.Spec(scale=0.8, causal=True, dropout_p=0.2, seed=4)
    q, k, v, do, _ = _problem(1, 2, 1, 7, 7, 4)
    v[:] = 0.0
    o, lse = oracle.forward(q, k, v, spec)
    assert np.all(o == 0.0)
    _, dq, dk, dv = oracle.backward(q, k, v, o, do, lse, spec)
    assert np.all(dq == 0.0) and np.all(dk == 0.0)
    # dV_j = sum_h sum_i P_ij M_ij dO_i, the plain definition with P from the forward scores
    want = np.zeros_like(dv)
    for h in range(2):
        p, mm, _ = oracle.backward_block(q, k, v, do, lse, np.zeros((1, 2, 7)), spec, None, 0, h,
                                         np.arange(7), np.arange(7))
        want[0, 0] += (p * mm).T @ do[0, h]
    np.testing.assert_allclose(dv, want, atol=1e-13)


def test_zero_queries_uniform_attention_closed_form():
    # Q = 0: every counted key gets P = 1/n_i, L_i = ln n_i and dS_ij = (dP_ij - mean_j dP_ij) / n_i.
    spec = oracle.Spec(scale=0.5, causal=True, causal_offset=2, window=4)
    Sq, Sk = 6, 8
    q, k, v, do, _ = _problem(1, 1, 1, Sq, Sk, 5)
    q[:] = 0.0
    o, lse = oracle.forward(q, k, v, spec)
    vis = oracle.visible(np.arange(Sq), np.arange(Sk), Sq, Sk, spec)
    n = vis.sum(1)
    np.testing.assert_allclose(lse[0, 0], np.log(n), atol=1e-14)
    delta = np.einsum("bhsd,bhsd->bhs", do, o)
    p, _, ds = oracle.backward_block(q, k, v, do, lse, delta, spec, None, 0, 0, np.arange(Sq), np.arange(Sk))
    dp = do[0, 0] @ v[0, 0].T
    for i in range(Sq):
        sel = vis[i]
        want = np.zeros(Sk)
        want[sel] = (dp[i, sel] - dp[i, sel].mean()) / n[i]
        np.testing.assert_allclose(ds[i], want, atol=1e-13)


def test_fully_masked_row():
    spec = oracle.Spec(scale=0.5, causal=True)
    q, k, v, do, _ = _problem(1, 2, 1, 6, 6, 4)
    mask = np.zeros((1, 1, 6, 6), np.float32)
    mask[0, 0, 0, 0] = np.float32(-1e30)  # row 0's only visible key is excluded
    o, lse = oracle.forward(q, k, v, spec, mask)
    assert np.isinf(lse[0, :, 0]).all() and np.all(o[0, :, 0] == 0)
    delta, dq, dk, dv = oracle.backward(q, k, v, o, do, lse, spec, mask)
    assert np.all(dq[0, :, 0] == 0)
    assert np.isfinite(dq).all() and np.isfinite(dk).all() and np.isfinite(dv).all()


def test_gqa_equals_repeated_kv():
    spec = oracle.Spec(scale=0.4, causal=True, window=5, dropout_p=0.1, seed=21)
    q, k, v, do, mask = _problem(1, 6, 2, 9, 9, 4, rng=np.random.default_rng(31), mask_kind="mixed")
    o, lse = oracle.forward(q, k, v, spec, mask)
    _, dq, dk, dv = oracle.backward(q, k, v, o, do, lse, spec, mask)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    o2, lse2 = oracle.forward(q, kr, vr, spec, mask)
    _, dq2, dk2, dv2 = oracle.backward(q, kr, vr, o2, do, lse2, spec, mask)
    np.testing.assert_allclose(o, o2, atol=1e-13)
    np.testing.assert_allclose(dq, dq2, atol=1e-13)
    np.testing.assert_allclose(dk, dk2.reshape(1, 2, 3, 9, 4).sum(2), atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(1, 2, 3, 9, 4).sum(2), atol=1e-13)


def test_equivalences_no_dropout_window_mask():
    q, k, v, do, _ = _problem(1, 2, 1, 8, 10, 4)
    base = oracle.Spec(scale=0.5, causal=True, causal_offset=2)
    o, lse = oracle.forward(q, k, v, base)
    ref = oracle.backward(q, k, v, o, do, lse, base)
    for spec, mask in ((oracle.Spec(scale=0.5, causal=True, causal_offset=2, window=12), None),
                       (base, np.zeros((1, 1, 8, 10), np.float32)),
                       (oracle.Spec(scale=0.5, causal=True, causal_offset=2, dropout_p=0.0, seed=99), None)):
        got = oracle.backward(q, k, v, o, do, lse, spec, mask)
        for a, b in zip(ref, got):
            assert np.array_equal(a, b)


def test_sampled_helpers_match_full_backward():
    spec = oracle.Spec(scale=0.35, causal=True, causal_offset=1, window=6, dropout_p=0.2, seed=8)
    q, k, v, do, mask = _problem(2, 4, 2, 11, 12, 8, rng=np.random.default_rng(5), mask_kind="mixed")
    o, lse = oracle.forward(q, k, v, spec, mask)
    _, dq, dk, dv = oracle.backward(q, k, v, o, do, lse, spec, mask, chunk=4)
    rows = np.array([0, 3, 10])
    np.testing.assert_allclose(oracle.backward_dq_rows(q, k, v, o, do, lse, spec, mask, 1, 2, rows),
                               dq[1, 2, rows], atol=1e-13)
    keys = np.array([1, 7, 11])
    sk, sv = oracle.backward_dkdv_keys(q, k, v, o, do, lse, spec, mask, 1, 1, keys, chunk=5)
    np.testing.assert_allclose(sk, dk[1, 1, keys], atol=1e-13)
    np.testing.assert_allclose(sv, dv[1, 1, keys], atol=1e-13)
    o2, lse2 = oracle.forward_rows(q, k, v, spec, mask, 1, 3, rows)
    np.testing.assert_allclose(o2, o[1, 3, rows], atol=1e-14)
    np.testing.assert_allclose(lse2, lse[1, 3, rows], atol=1e-14)
