"""GPU parity of the forward pass (O, L) against the fp64 oracle forward.

O to its dtype's bar (bf16: relative Frobenius error 2e-2; fp32: max |err| <=
2e-4 * max |ref|).  L is fp32 computed from fp32 MFMA sums (of exact bf16
products, or of fp32 products) and the hardware exp2/log2, so it must agree to
1e-4 * max(1, |L|) (bf16 inputs) or 1e-5 * max(1, |L|) (fp32) on every finite
row, and be +inf exactly on the rows where no element counts.  Every case of
the backward parity tests, plus rows with every key masked.  fa_bwd_lse (L
alone) must give the oracle's L at the same bar, and the forward's L.
"""
import numpy as np
import pytest
import torch

import oracle
from flashattention_backward_pass_bwd_amd import api, synth

from fa_testlib import assert_close, dev, logical, say, spec_of
from test_gpu_parity import CASES, DEGENERATE

pytestmark = pytest.mark.gpu

FWD_CASES = dict(CASES)


def _l_tol(w):
    return 1e-4 if w.dtype == "bf16" else 1e-5


def _check(w, inp, mask_dev=None):
    spec = spec_of(w)
    ref_o, ref_l = oracle.forward(inp["q"], inp["k"], inp["v"], spec, inp["mask"])
    q, k, v = (dev(inp[n], w.layout, w.dtype) for n in ("q", "k", "v"))
    mask = mask_dev if mask_dev is not None else (
        torch.from_numpy(inp["mask"]).cuda() if inp["mask"] is not None else None)
    p = api.make_params(q, k, scale=w.scale, causal=w.causal, causal_offset=w.causal_offset, window=w.window,
                        dropout_p=w.dropout_p, seed=w.dropout_seed, mask=mask)
    o, lse = api.forward(p, q, k, v)
    torch.cuda.synchronize()
    got_l = lse.cpu().numpy().astype(np.float64)
    inf = np.isinf(ref_l)
    assert np.array_equal(np.isinf(got_l), inf) and np.all(got_l[inf] > 0), "rows with nothing counted"
    err = np.abs(got_l[~inf] - ref_l[~inf]) / np.maximum(1.0, np.abs(ref_l[~inf]))
    say(f"  L: max err {err.max() if err.size else 0.0:.2e} (tol {_l_tol(w):g})")
    assert err.size == 0 or err.max() <= _l_tol(w)
    assert_close(logical(o), ref_o, w.dtype, "o")
    # the L-only sweep against the oracle's L, at the same bar, and against the forward's L
    lonly = api.lse(p, q, k).cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isinf(lonly), inf) and np.all(lonly[inf] > 0), "L-only sweep: rows with nothing counted"
    lerr = np.abs(lonly[~inf] - ref_l[~inf]) / np.maximum(1.0, np.abs(ref_l[~inf]))
    say(f"  L-only sweep: max err {lerr.max() if lerr.size else 0.0:.2e} (tol {_l_tol(w):g})")
    assert lerr.size == 0 or lerr.max() <= _l_tol(w)
    assert np.abs(lonly[~inf] - got_l[~inf]).max(initial=0.0) <= 1e-5 * max(1.0, np.abs(got_l[~inf]).max(initial=1.0))
    return logical(o), got_l


@pytest.mark.parametrize("name", sorted(FWD_CASES))
def test_forward_parity(name):
    w = FWD_CASES[name]
    say(f"[forward] {name}: {w}")
    _check(w, synth.prefill_inputs(w))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("sq,sk,causal", DEGENERATE)
def test_forward_degenerate_sizes(dtype, sq, sk, causal):
    """One query or one key, two of each, one past a tile edge (the backward's
    degenerate cases), for O, L and the L-only sweep."""
    base = synth.CAUSAL_F32 if dtype == "f32" else synth.LONG_BF16
    w = base.resized(batch=1, num_heads=2, num_kv_heads=1, seq_q=sq, seq_k=sk, causal=causal, causal_offset=0,
                     seed=60 + sq + 7 * sk)
    if sq > 2 and sk > 2:
        w = w.resized(dropout_p=0.2, dropout_seed=5)
    say(f"[forward degenerate] {w}")
    _check(w, synth.prefill_inputs(w))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_fully_masked_rows(dtype):
    w = synth.EXTRAS_BF16.resized(dtype=dtype, batch=2, num_heads=4, num_kv_heads=2, seq_q=96, seq_k=96, window=8,
                                  mask_density=0.05, seed=41)
    inp = synth.prefill_inputs(w)
    inp["mask"][1, 0, 0, 0] = np.float32(-1e30)  # row 0 of batch 1 sees only key 0, now excluded
    inp["mask"][0, 0, 5, :] = np.float32(-1e30)  # row 5 of batch 0: every key excluded
    o, lse = _check(w, inp)
    assert np.isinf(lse[1, :, 0]).all() and np.isinf(lse[0, :, 5]).all()
    assert np.all(o[1, :, 0] == 0.0) and np.all(o[0, :, 5] == 0.0)


@pytest.mark.parametrize("which", ["extras", "long"])
def test_forward_full_size_sampled(which):
    """The full-size bf16 workloads: sampled rows of a few heads against the oracle's rows."""
    w = synth.EXTRAS_BF16 if which == "extras" else synth.LONG_BF16
    inp = synth.prefill_inputs(w)
    spec = spec_of(w)
    q, k, v = (dev(inp[n], w.layout, w.dtype) for n in ("q", "k", "v"))
    mask = torch.from_numpy(inp["mask"]).cuda() if inp["mask"] is not None else None
    p = api.make_params(q, k, scale=w.scale, causal=w.causal, causal_offset=w.causal_offset, window=w.window,
                        dropout_p=w.dropout_p, seed=w.dropout_seed, mask=mask)
    o, lse = api.forward(p, q, k, v)
    torch.cuda.synchronize()
    go, gl = logical(o), lse.cpu().numpy().astype(np.float64)
    S = w.seq_q
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, S // 2, S - 2, S - 1], rng.integers(0, S, 41)]))
    for (b, h) in [(0, 0), (w.batch - 1, w.num_heads - 1), (w.batch // 2, w.num_heads // 2 + 1)]:
        ro, rl = oracle.forward_rows(inp["q"], inp["k"], inp["v"], spec, inp["mask"], b, h, rows)
        assert_close(go[b, h, rows], ro, "bf16", f"o rows (b={b}, h={h})")
        err = np.abs(gl[b, h, rows] - rl) / np.maximum(1.0, np.abs(rl))
        assert err.max() <= 1e-4, err.max()


@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("layout", ["per_head", "key_major", "key_padding", "padded_rows"])
def test_forward_mask_layouts(layout, head_dim):
    """The mask layouts of the backward's tests (one mask per head with finite
    values, a key-major copy, a key-padding row broadcast over queries) with a
    window, dropout and a key count that is not a multiple of 4."""
    w = synth.EXTRAS_BF16.resized(batch=2, num_heads=4, num_kv_heads=2, head_dim=head_dim, seq_q=197,
                                  seq_k=230, window=90, causal_offset=40, seed=61 + head_dim)
    inp = synth.prefill_inputs(w)
    rng = np.random.default_rng(200 + head_dim)
    B, H, Sq, Sk = w.batch, w.num_heads, w.seq_q, w.seq_k
    if layout == "per_head":
        m = np.where(rng.random((B, H, Sq, Sk)) < 0.1, -1e30, rng.normal(0.0, 0.5, (B, H, Sq, Sk)))
        inp["mask"] = m.astype(np.float32)
        mask_dev = torch.from_numpy(inp["mask"]).cuda()
    elif layout == "key_major":
        m = np.where(rng.random((B, 1, Sq, Sk)) < 0.1, -1e30, 0.0).astype(np.float32)
        inp["mask"] = m
        mask_dev = torch.from_numpy(np.ascontiguousarray(m.transpose(0, 1, 3, 2))).cuda().transpose(2, 3)
    elif layout == "key_padding":
        m = np.where(rng.random((B, 1, 1, Sk)) < 0.15, -1e30, 0.0).astype(np.float32)
        inp["mask"] = m
        mask_dev = torch.from_numpy(m).cuda()
    else:
        # [B, 1, Sq, Sk] stored in rows padded to a multiple of 4 keys: 16-byte aligned rows (the
        # vector mask paths) with a ragged last group of keys
        m = np.where(rng.random((B, 1, Sq, Sk)) < 0.1, -1e30, 0.0).astype(np.float32)
        inp["mask"] = m
        full = torch.zeros((B, 1, Sq, (Sk + 3) // 4 * 4), dtype=torch.float32)
        full[..., :Sk] = torch.from_numpy(m)
        mask_dev = full.cuda()[..., :Sk]
        assert mask_dev.stride(2) % 4 == 0 and Sk % 4 != 0
    say(f"[forward mask layout] {layout} D={head_dim}")
    _check(w, inp, mask_dev)
