"""Seeded synthetic inputs for the attention-backward workloads.

This module only draws random numbers and rounds them to the storage dtype; it
holds none of the attention arithmetic, so both the HIP path's tests and the
CPU oracle can consume its arrays.  All draws use numpy's PCG64 with a fixed
per-workload seed, in a fixed order (Q, K, V, dO, then the mask), as fp32
standard normals; bf16 workloads round them to nearest-even bf16 values
(returned as float32 arrays holding exactly representable bf16 values).

Arrays are returned in the logical layout [B, H, S, D] (decode: [N, len, Hkv, D]
for the history and [N, H, D] / [N, H, len] for the rest); callers repack them
into whatever strided device layout they exercise.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class PrefillWorkload:
    """One prefill-backward problem: sizes, layout, scalar parameters and its seed."""

    name: str
    dtype: str  # "f32" or "bf16"
    batch: int
    num_heads: int
    num_kv_heads: int
    seq_q: int
    seq_k: int
    head_dim: int
    layout: str  # "bhsd" or "bshd" (device layout of Q/K/V/O/dO and the grads)
    scale: float
    causal: bool = False
    causal_offset: int = 0
    window: int = 0
    mask_density: float = 0.0  # fraction of -1e30 entries in a [B,1,Sq,Sk] mask; 0 = no mask
    dropout_p: float = 0.0
    dropout_seed: int = 0
    seed: int = 0
    qk_std: float = 1.0  # standard deviation of the Q and K draws (scores then have std ~ qk_std^2 at scale 1/sqrt(D))

    def resized(self, **kw) -> "PrefillWorkload":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """Single-query decode-step backward problem (unscaled scores)."""

    name: str
    num_seqs: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    history_len: int
    kv_std: float = 1.0 / 16.0
    seed: int = 0

    def resized(self, **kw) -> "DecodeWorkload":
        return dataclasses.replace(self, **kw)


# The five workloads, named by what they are.
TINY_F32 = PrefillWorkload(
    name="f32_mha_b1_h2_s64_d64", dtype="f32", batch=1, num_heads=2, num_kv_heads=2,
    seq_q=64, seq_k=64, head_dim=64, layout="bhsd", scale=1.0 / 8.0, seed=101)
CAUSAL_F32 = PrefillWorkload(
    name="f32_causal_mha_b2_h8_s1024_d64", dtype="f32", batch=2, num_heads=8, num_kv_heads=8,
    seq_q=1024, seq_k=1024, head_dim=64, layout="bhsd", scale=1.0 / 8.0, causal=True, seed=202)
DECODE_F32 = DecodeWorkload(
    name="f32_decode_n64_h32_kv8_d256_len4096", num_seqs=64, n_heads=32, n_kv_heads=8,
    head_dim=256, history_len=4096, seed=303)
EXTRAS_BF16 = PrefillWorkload(
    name="bf16_gqa_causal_window512_mask5pct_dropout0.1_b4_hq32_hkv8_s2048_d128", dtype="bf16",
    batch=4, num_heads=32, num_kv_heads=8, seq_q=2048, seq_k=2048, head_dim=128, layout="bshd",
    scale=1.0 / math.sqrt(128.0), causal=True, window=512, mask_density=0.05, dropout_p=0.1,
    dropout_seed=0x5EED1234, seed=404)
LONG_BF16 = PrefillWorkload(
    name="bf16_gqa_causal_b1_hq32_hkv8_s16384_d128", dtype="bf16", batch=1, num_heads=32,
    num_kv_heads=8, seq_q=16384, seq_k=16384, head_dim=128, layout="bshd",
    scale=1.0 / math.sqrt(128.0), causal=True, seed=505)

PREFILL_WORKLOADS = (TINY_F32, CAUSAL_F32, EXTRAS_BF16, LONG_BF16)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns float32 storage."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
    return r.view(np.float32).reshape(x.shape)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_to_bf16(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def prefill_inputs(w: PrefillWorkload):
    """Q, K, V, dO ([B,H,S,D] float32, bf16-representable for bf16) and the mask.

    Q and K are N(0, qk_std^2) draws (the fp32 standard normal times qk_std, then
    rounded to the storage dtype); V and dO are N(0, 1)."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    B, Hq, Hkv, Sq, Sk, D = w.batch, w.num_heads, w.num_kv_heads, w.seq_q, w.seq_k, w.head_dim
    sd = np.float32(w.qk_std)
    q = _store(rng.standard_normal((B, Hq, Sq, D), dtype=np.float32) * sd, w.dtype)
    k = _store(rng.standard_normal((B, Hkv, Sk, D), dtype=np.float32) * sd, w.dtype)
    v = _store(rng.standard_normal((B, Hkv, Sk, D), dtype=np.float32), w.dtype)
    do = _store(rng.standard_normal((B, Hq, Sq, D), dtype=np.float32), w.dtype)
    mask = None
    if w.mask_density > 0.0:
        hit = rng.random((B, 1, Sq, Sk), dtype=np.float32) < np.float32(w.mask_density)
        mask = np.where(hit, np.float32(-1.0e30), np.float32(0.0)).astype(np.float32)
    return {"q": q, "k": k, "v": v, "do": do, "mask": mask}


def decode_inputs(w: DecodeWorkload, seqs=None):
    """Per-sequence draws (each sequence has its own PCG64 stream, so any subset is cheap).

    Returns q, d_out [n,H,D] ~ N(0,1) and k_hist, v_hist [n,len,Hkv,D] ~ N(0,1)*kv_std.
    """
    if seqs is None:
        seqs = range(w.num_seqs)
    seqs = list(seqs)
    n = len(seqs)
    H, Hkv, D, L = w.n_heads, w.n_kv_heads, w.head_dim, w.history_len
    q = np.empty((n, H, D), np.float32)
    d_out = np.empty((n, H, D), np.float32)
    k_hist = np.empty((n, L, Hkv, D), np.float32)
    v_hist = np.empty((n, L, Hkv, D), np.float32)
    for t, s in enumerate(seqs):
        rng = np.random.Generator(np.random.PCG64([w.seed, s]))
        q[t] = rng.standard_normal((H, D), dtype=np.float32)
        d_out[t] = rng.standard_normal((H, D), dtype=np.float32)
        k_hist[t] = rng.standard_normal((L, Hkv, D), dtype=np.float32) * np.float32(w.kv_std)
        v_hist[t] = rng.standard_normal((L, Hkv, D), dtype=np.float32) * np.float32(w.kv_std)
    return {"q": q, "d_out": d_out, "k_hist": k_hist, "v_hist": v_hist}
