"""Plain fp64 definitions of attention forward/backward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module.  The product (the HIP library and its binding)
never imports it and must fail loudly rather than fall back to it.

Everything is evaluated as dense numpy float64 matrices per (batch, head), in
the order the pages state the formulas.  Rows are processed in chunks only to
bound memory; every sum is complete over its index.

Logical tensor layout used throughout (the tests repack for the GPU):
  q, o, do, dq : [B, Hq, Sq, D]
  k, v, dk, dv : [B, Hkv, Sk, D]
  lse, delta   : [B, Hq, Sq]
  mask         : None, or an array broadcastable to [B, Hq, Sq, Sk]
"""

from __future__ import annotations

import dataclasses

import numpy as np

# Mask sentinel of ferrotensor-backend flash_attention_v2_backward.wgsl
# (constant FAB_MASKED): an additive mask entry at or below it removes the
# element from the softmax.  Compared in fp32, as the mask is an fp32 tensor.
MASKED = np.float64(np.float32(-1.0e30))

_U32 = np.uint64(0xFFFFFFFF)


@dataclasses.dataclass(frozen=True)
class Spec:
    """Scalar parameters of one attention problem.

    Field meanings follow the parameter struct of ferrotensor-backend
    flash_attention_v2_backward.wgsl (FlashBwdParams): softmax scale, causal
    flag with a query-position offset, sliding window (0 = off), dropout
    probability and seed.
    """

    scale: float
    causal: bool = False
    causal_offset: int = 0
    window: int = 0
    dropout_p: float = 0.0
    seed: int = 0


# --------------------------------------------------------------------------
# Dropout hash.
#
# ferrotensor-backend flash_attention_v2_backward.wgsl calls a dropout
# multiplier keyed by (p, seed, b*Hq+h, i, j) -- the *query* head -- but the
# helper that defines it lives in a file that is not on the page.  The
# composition below is therefore our own specification; its only published
# ingredient is fmix32, the 32-bit finaliser of Austin Appleby's MurmurHash3
# (public domain), which is pinned by published MurmurHash3_x86_32 vectors.
#
#   row  = ((b*Hq + h)*Sq + i)                       mod 2^32
#   r    = fmix32((row + fmix32(seed))               mod 2^32)
#   u    = fmix32(r XOR (j * 0x9E3779B9              mod 2^32))
#   keep = u >= floor(p_f32 * 2^32)
#   M    = keep / (1 - p)          (inverted dropout; M == 1 when p == 0)
# --------------------------------------------------------------------------

def fmix32(x):
    """MurmurHash3 32-bit finaliser on uint32 values (mod 2^32 arithmetic)."""
    x = np.asarray(x, dtype=np.uint64) & _U32
    x ^= x >> np.uint64(16)
    x = (x * np.uint64(0x85EBCA6B)) & _U32
    x ^= x >> np.uint64(13)
    x = (x * np.uint64(0xC2B2AE35)) & _U32
    x ^= x >> np.uint64(16)
    return x.astype(np.uint32)


def dropout_threshold(p: float) -> int:
    """floor(p * 2^32) for the fp32 value of p (exact: fp32 * 2^32 is exact)."""
    pf = float(np.float32(p))
    thr = int(np.floor(pf * 4294967296.0))
    return min(thr, 0xFFFFFFFF)


def dropout_draw(seed: int, b: int, h: int, num_heads: int, seq_q: int, rows, cols):
    """The uint32 draw u for query rows ``rows`` x key columns ``cols`` of head (b, h)."""
    rows = np.asarray(rows, dtype=np.uint64).reshape(-1, 1)
    cols = np.asarray(cols, dtype=np.uint64).reshape(1, -1)
    bh = np.uint64(b * num_heads + h)
    row_id = (bh * np.uint64(seq_q) + rows) & _U32
    seed_mix = fmix32(np.uint64(seed)).astype(np.uint64)
    r = fmix32((row_id + seed_mix) & _U32).astype(np.uint64)
    col_mix = (cols * np.uint64(0x9E3779B9)) & _U32
    return fmix32(r ^ col_mix)


def dropout_keep(seed: int, b: int, h: int, num_heads: int, seq_q: int, rows, cols, p: float):
    """Keep bits: u >= floor(p * 2^32)."""
    u = dropout_draw(seed, b, h, num_heads, seq_q, rows, cols)
    return u.astype(np.uint64) >= np.uint64(dropout_threshold(p))


def dropout_multiplier(spec: Spec, b: int, h: int, num_heads: int, seq_q: int, rows, cols):
    """M_ij = keep_ij / (1 - p) (ferrotensor-backend header: M is the dropout multiplier)."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    if spec.dropout_p == 0.0:
        return np.ones((rows.size, cols.size), dtype=np.float64)
    keep = dropout_keep(spec.seed, b, h, num_heads, seq_q, rows, cols, spec.dropout_p)
    inv = 1.0 / (1.0 - float(np.float32(spec.dropout_p)))
    return np.where(keep, inv, 0.0)


# --------------------------------------------------------------------------
# Visibility (ferrotensor-backend fab2_visible and fab2_mask_at).
# --------------------------------------------------------------------------

def visible(rows, cols, seq_q: int, seq_k: int, spec: Spec):
    """Geometric visibility of key j to query i.

    In range, causal (j <= i + offset) and, when window > 0, |j - (i+offset)| < window
    -- the window applies with or without causal.
    """
    i = np.asarray(rows, dtype=np.int64).reshape(-1, 1)
    j = np.asarray(cols, dtype=np.int64).reshape(1, -1)
    qa = i + spec.causal_offset
    vis = (i < seq_q) & (j < seq_k) & (i >= 0) & (j >= 0)
    if spec.causal:
        vis = vis & (j <= qa)
    if spec.window > 0:
        vis = vis & (np.abs(j - qa) < spec.window)
    return vis


def counted(vis, mask_vals):
    """An element enters the softmax iff visible and its mask entry is above the sentinel."""
    if mask_vals is None:
        return vis
    return vis & ~(np.asarray(mask_vals, dtype=np.float64) <= MASKED)


def _mask_block(mask, shape4, b, h, rows, cols):
    """Additive fp32 mask entries (ferrotensor-backend fab2_mask_at), broadcast to [B, Hq, Sq, Sk]."""
    if mask is None:
        return None
    m = np.broadcast_to(np.asarray(mask), shape4)
    return m[b, h][np.ix_(np.asarray(rows), np.asarray(cols))].astype(np.float64)


def _scores(q, k, spec, mask, b, h, kvh, rows, cols):
    """S = scale * Q K^T + mask, and the counted-element predicate."""
    s = spec.scale * (q[b, h, rows].astype(np.float64) @ k[b, kvh, cols].astype(np.float64).T)
    shape4 = (q.shape[0], q.shape[1], q.shape[2], k.shape[2])
    mv = _mask_block(mask, shape4, b, h, rows, cols)
    if mv is not None:
        s = s + mv
    cnt = counted(visible(rows, cols, q.shape[2], k.shape[2], spec), mv)
    return s, cnt


def _group(q, k):
    hq, hkv = q.shape[1], k.shape[1]
    if hq % hkv:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    return hq // hkv


# --------------------------------------------------------------------------
# Forward: O and the natural-log log-sum-exp L.
# --------------------------------------------------------------------------

def forward_rows(q, k, v, spec: Spec, mask, b: int, h: int, rows):
    """O and L for query rows ``rows`` of head (b, h).

    L_i = log sum_{counted j} exp(S_ij); L_i = +inf when no key is counted
    (the page's 3e38 sentinel, read as +inf: every P_ij of such a row is 0).
    P_ij = exp(S_ij - L_i) on counted elements, 0 elsewhere;
    O_i = sum_j P_ij M_ij V_j (dropout applied to P, not to L).
    """
    g = _group(q, k)
    kvh = h // g
    rows = np.asarray(rows)
    cols = np.arange(k.shape[2])
    s, cnt = _scores(q, k, spec, mask, b, h, kvh, rows, cols)
    has = cnt.any(axis=1)
    s_c = np.where(cnt, s, -np.inf)
    m = np.where(has, s_c.max(axis=1, initial=-np.inf), 0.0)
    with np.errstate(under="ignore"):
        l = np.exp(s_c - m[:, None]).sum(axis=1)
    lse = np.where(has, m + np.log(np.where(has, l, 1.0)), np.inf)
    with np.errstate(under="ignore", invalid="ignore"):
        p = np.where(cnt, np.exp(s_c - lse[:, None]), 0.0)
    mm = dropout_multiplier(spec, b, h, q.shape[1], q.shape[2], rows, cols)
    o = (p * mm) @ v[b, kvh].astype(np.float64)
    return o, lse


def forward(q, k, v, spec: Spec, mask=None, chunk: int = 1024):
    """Full forward over every (b, h) and row chunk."""
    B, Hq, Sq, D = q.shape
    o = np.zeros((B, Hq, Sq, v.shape[3]), dtype=np.float64)
    lse = np.zeros((B, Hq, Sq), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            for r0 in range(0, Sq, chunk):
                rows = np.arange(r0, min(Sq, r0 + chunk))
                o[b, h, rows], lse[b, h, rows] = forward_rows(q, k, v, spec, mask, b, h, rows)
    return o, lse


# --------------------------------------------------------------------------
# Backward given the provided Q, K, V, O, dO and L.
# Formulas: rustytorch dQ kernel header (dQ = scale * dS K, dS = P (dO V^T - D),
# D = rowsum(dO * O)); ferrotensor-backend header (dV_j = sum_i P_ij M_ij dO_i,
# dK_j = scale * sum_i dS_ij Q_i summed over the query heads of a KV head,
# dS_ij = P_ij (M_ij dO_i.V_j - Delta_i)).
# --------------------------------------------------------------------------

def backward_block(q, k, v, do, lse, delta, spec: Spec, mask, b: int, h: int, rows, cols):
    """P, M and dS on the sub-matrix rows x cols of head (b, h).

    Uses the provided L (no recomputation): P_ij = exp(S_ij - L_i) on counted
    elements; dP_ij = M_ij (dO_i . V_j); dS_ij = P_ij (dP_ij - Delta_i).
    """
    g = _group(q, k)
    kvh = h // g
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    s, cnt = _scores(q, k, spec, mask, b, h, kvh, rows, cols)
    L = lse[b, h, rows].astype(np.float64)
    with np.errstate(under="ignore", invalid="ignore", over="ignore"):
        p = np.where(cnt, np.exp(np.where(cnt, s, -np.inf) - L[:, None]), 0.0)
    mm = dropout_multiplier(spec, b, h, q.shape[1], q.shape[2], rows, cols)
    dp = mm * (do[b, h, rows].astype(np.float64) @ v[b, kvh, cols].astype(np.float64).T)
    ds = p * (dp - delta[b, h, rows].astype(np.float64)[:, None])
    return p, mm, ds


def _delta(o, do):
    """Delta_i = dO_i . O_i (rustytorch dQ kernel, D = rowsum(dO * O))."""
    return np.einsum("bhsd,bhsd->bhs", do.astype(np.float64), o.astype(np.float64))


def backward(q, k, v, o, do, lse, spec: Spec, mask=None, chunk: int = 1024):
    """Delta, dQ, dK, dV for every element."""
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    g = _group(q, k)
    delta = _delta(o, do)
    dq = np.zeros((B, Hq, Sq, D), dtype=np.float64)
    dk = np.zeros((B, Hkv, Sk, D), dtype=np.float64)
    dv = np.zeros((B, Hkv, Sk, v.shape[3]), dtype=np.float64)
    cols = np.arange(Sk)
    for b in range(B):
        for h in range(Hq):
            kvh = h // g
            for r0 in range(0, Sq, chunk):
                rows = np.arange(r0, min(Sq, r0 + chunk))
                p, mm, ds = backward_block(q, k, v, do, lse, delta, spec, mask, b, h, rows, cols)
                dq[b, h, rows] = spec.scale * (ds @ k[b, kvh].astype(np.float64))
                dk[b, kvh] += spec.scale * (ds.T @ q[b, h, rows].astype(np.float64))
                dv[b, kvh] += (p * mm).T @ do[b, h, rows].astype(np.float64)
    return delta, dq, dk, dv


def backward_dq_rows(q, k, v, o, do, lse, spec: Spec, mask, b: int, h: int, rows):
    """dQ for a subset of query rows of head (b, h); each row is a complete sum over keys."""
    g = _group(q, k)
    rows = np.asarray(rows)
    delta = np.zeros(lse.shape, dtype=np.float64)
    delta[b, h, rows] = _delta(o[b:b + 1, h:h + 1, rows], do[b:b + 1, h:h + 1, rows])[0, 0]
    cols = np.arange(k.shape[2])
    _, _, ds = backward_block(q, k, v, do, lse, delta, spec, mask, b, h, rows, cols)
    return spec.scale * (ds @ k[b, h // g].astype(np.float64))


def backward_dkdv_keys(q, k, v, o, do, lse, spec: Spec, mask, b: int, kvh: int, keys, chunk: int = 4096):
    """dK, dV for a subset of keys of KV head (b, kvh), summed over its query heads and all rows."""
    g = _group(q, k)
    keys = np.asarray(keys)
    Sq = q.shape[2]
    dk = np.zeros((keys.size, k.shape[3]), dtype=np.float64)
    dv = np.zeros((keys.size, v.shape[3]), dtype=np.float64)
    for h in range(kvh * g, (kvh + 1) * g):
        delta = np.zeros(lse.shape, dtype=np.float64)
        delta[b, h] = _delta(o[b:b + 1, h:h + 1], do[b:b + 1, h:h + 1])[0, 0]
        for r0 in range(0, Sq, chunk):
            rows = np.arange(r0, min(Sq, r0 + chunk))
            p, mm, ds = backward_block(q, k, v, do, lse, delta, spec, mask, b, h, rows, keys)
            dk += spec.scale * (ds.T @ q[b, h, rows].astype(np.float64))
            dv += (p * mm).T @ do[b, h, rows].astype(np.float64)
    return dk, dv


# --------------------------------------------------------------------------
# Decode-step backward (rullama attention_backward_dq.wgsl, pass 1).
# Scores are unscaled; probs is an input; outputs d_scores and d_q only.
#   k_hist, v_hist : [N, len, Hkv, D]
#   probs, d_scores: [N, H, len]
#   d_out, d_q     : [N, H, D]
# --------------------------------------------------------------------------

def decode_probs(q, k_hist, heads_per_kv: int):
    """probs = softmax_j(q_h . K_j) over the whole history (unscaled), fp64."""
    N, H, D = q.shape
    L = k_hist.shape[1]
    out = np.zeros((N, H, L), dtype=np.float64)
    for n in range(N):
        for h in range(H):
            kv = h // heads_per_kv
            s = k_hist[n, :, kv, :].astype(np.float64) @ q[n, h].astype(np.float64)
            e = np.exp(s - s.max())
            out[n, h] = e / e.sum()
    return out


def decode_backward(k_hist, v_hist, probs, d_out, heads_per_kv: int):
    """Phase A: dp_j = d_out_h . V_j; sum_pd = sum_j probs_j dp_j;
    Phase B: d_scores_j = probs_j (dp_j - sum_pd);
    Phase C: d_q_h = sum_j d_scores_j K_j."""
    N, H, L = probs.shape
    D = d_out.shape[2]
    d_scores = np.zeros((N, H, L), dtype=np.float64)
    d_q = np.zeros((N, H, D), dtype=np.float64)
    for n in range(N):
        for h in range(H):
            kv = h // heads_per_kv
            dp = v_hist[n, :, kv, :].astype(np.float64) @ d_out[n, h].astype(np.float64)
            pr = probs[n, h].astype(np.float64)
            sum_pd = pr @ dp
            ds = pr * (dp - sum_pd)
            d_scores[n, h] = ds
            d_q[n, h] = ds @ k_hist[n, :, kv, :].astype(np.float64)
    return d_scores, d_q


def decode_dkdv(q, probs, d_scores, d_out, heads_per_kv: int):
    """Decode-step backward, pass 2 (named after pass 1 on the rullama page;
    its code is not shown there): the history gradients, summed over the
    query heads sharing a KV head.  With scores s_hj = q_h . K_j (unscaled) and
    out_h = sum_j probs_hj V_j:
      dK_j = sum_h d_scores_hj q_h,   dV_j = sum_h probs_hj d_out_h.
    Returns dk_hist, dv_hist [N, L, Hkv, D], fp64."""
    N, H, L = probs.shape
    D = q.shape[2]
    Hkv = H // heads_per_kv
    dk = np.zeros((N, L, Hkv, D), dtype=np.float64)
    dv = np.zeros((N, L, Hkv, D), dtype=np.float64)
    for n in range(N):
        for h in range(H):
            kv = h // heads_per_kv
            dk[n, :, kv, :] += np.outer(d_scores[n, h].astype(np.float64), q[n, h].astype(np.float64))
            dv[n, :, kv, :] += np.outer(probs[n, h].astype(np.float64), d_out[n, h].astype(np.float64))
    return dk, dv
