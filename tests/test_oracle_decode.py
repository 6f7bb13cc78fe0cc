"""Pins for the oracle's decode-step backward (CPU only).

* decode == the general backward with Sq = 1, scale 1, non-causal, L = log-sum-exp
  and O = probs V, with d_scores equal to dS;
* sum_j d_scores_hj = 0 (probs sum to 1);
* a brute-force softmax Jacobian over the history;
* GQA head mapping: heads h and h' of one KV head see the same history;
* pass 2 (history dK, dV): equal to the general backward's dK, dV with one
  query per head, and to central finite differences of the decode forward
  loss sum_h d_out_h . out_h in K and V.
"""
import numpy as np

import oracle


def _decode_problem(rng, N=2, H=8, Hkv=2, D=16, L=40):
    q = rng.standard_normal((N, H, D))
    d_out = rng.standard_normal((N, H, D))
    k_hist = rng.standard_normal((N, L, Hkv, D)) / 4
    v_hist = rng.standard_normal((N, L, Hkv, D)) / 4
    return q, d_out, k_hist, v_hist


def test_decode_equals_general_backward_with_one_query():
    rng = np.random.default_rng(3)
    N, H, Hkv, D, L = 2, 8, 2, 16, 40
    q, d_out, k_hist, v_hist = _decode_problem(rng, N, H, Hkv, D, L)
    probs = oracle.decode_probs(q, k_hist, H // Hkv)
    d_scores, d_q = oracle.decode_backward(k_hist, v_hist, probs, d_out, H // Hkv)
    spec = oracle.Spec(scale=1.0)
    for n in range(N):
        qq = q[n][None, :, None, :]                     # [1, H, 1, D]
        kk = np.transpose(k_hist[n], (1, 0, 2))[None]    # [1, Hkv, L, D]
        vv = np.transpose(v_hist[n], (1, 0, 2))[None]
        do = d_out[n][None, :, None, :]
        o, lse = oracle.forward(qq, kk, vv, spec)
        delta, dq, dk, dv = oracle.backward(qq, kk, vv, o, do, lse, spec)
        np.testing.assert_allclose(d_q[n], dq[0, :, 0], atol=1e-13)
        dkh, dvh = oracle.decode_dkdv(q[n:n + 1], probs[n:n + 1], d_scores[n:n + 1], d_out[n:n + 1], H // Hkv)
        np.testing.assert_allclose(dkh[0], np.transpose(dk[0], (1, 0, 2)), atol=1e-13)
        np.testing.assert_allclose(dvh[0], np.transpose(dv[0], (1, 0, 2)), atol=1e-13)
        for h in range(H):
            p, _, ds = oracle.backward_block(qq, kk, vv, do, lse, delta, spec, None, 0, h, [0], np.arange(L))
            np.testing.assert_allclose(p[0], probs[n, h], atol=1e-14)
            np.testing.assert_allclose(ds[0], d_scores[n, h], atol=1e-14)


def test_decode_score_grads_sum_to_zero_and_jacobian():
    rng = np.random.default_rng(4)
    q, d_out, k_hist, v_hist = _decode_problem(rng, N=1, H=4, Hkv=1, D=8, L=64)
    probs = oracle.decode_probs(q, k_hist, 4)
    d_scores, _ = oracle.decode_backward(k_hist, v_hist, probs, d_out, 4)
    assert np.abs(d_scores.sum(-1)).max() < 1e-14
    for h in range(4):
        p = probs[0, h]
        J = np.diag(p) - np.outer(p, p)
        dp = v_hist[0, :, 0, :] @ d_out[0, h]
        np.testing.assert_allclose(J @ dp, d_scores[0, h], atol=1e-14)


def test_decode_gqa_mapping_contiguous_groups():
    rng = np.random.default_rng(5)
    q, d_out, k_hist, v_hist = _decode_problem(rng, N=1, H=8, Hkv=2, D=8, L=16)
    probs = oracle.decode_probs(q, k_hist, 4)
    # make heads 0 and 3 identical queries: same KV head (0) => same probs; head 4 uses KV head 1
    q[0, 3] = q[0, 0]
    q[0, 4] = q[0, 0]
    probs = oracle.decode_probs(q, k_hist, 4)
    np.testing.assert_allclose(probs[0, 3], probs[0, 0], atol=1e-15)
    assert np.abs(probs[0, 4] - probs[0, 0]).max() > 1e-3


def _decode_loss(q, k_hist, v_hist, d_out, g):
    probs = oracle.decode_probs(q, k_hist, g)
    N, H, _ = probs.shape
    loss = 0.0
    for n in range(N):
        for h in range(H):
            loss += d_out[n, h] @ (probs[n, h] @ v_hist[n, :, h // g, :])
    return loss


def test_decode_history_grads_match_finite_differences():
    rng = np.random.default_rng(7)
    N, H, Hkv, D, L = 1, 4, 2, 6, 9
    g = H // Hkv
    q, d_out, k_hist, v_hist = _decode_problem(rng, N, H, Hkv, D, L)
    probs = oracle.decode_probs(q, k_hist, g)
    d_scores, _ = oracle.decode_backward(k_hist, v_hist, probs, d_out, g)
    dk, dv = oracle.decode_dkdv(q, probs, d_scores, d_out, g)
    eps = 1e-6
    for arr, grad in ((k_hist, dk), (v_hist, dv)):
        for idx in [(0, 0, 0, 0), (0, 3, 1, 2), (0, 8, 0, 5), (0, 5, 1, 1)]:
            a = arr.copy(); a[idx] += eps
            lp = _decode_loss(q, a if arr is k_hist else k_hist, a if arr is v_hist else v_hist, d_out, g)
            a[idx] -= 2 * eps
            lm = _decode_loss(q, a if arr is k_hist else k_hist, a if arr is v_hist else v_hist, d_out, g)
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(fd)), (idx, fd, grad[idx])
