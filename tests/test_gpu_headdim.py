"""GPU parity at head dimensions other than 64 and 128 (any multiple of 8 up
to 128; the kernels pad the tail of their 64- or 128-wide tiles).

Backward (both bf16 paths and fp32) and forward against the fp64 oracle, every
output element, at each dtype's bar; the GQA window + mask + dropout feature
set and plain causal attention (the 64-row dQ kernel for D > 64), ragged
lengths, BSHD and BHSD layouts.
"""
import numpy as np
import pytest
import torch

import oracle
from flashattention_backward_pass_bwd_amd import api, synth

from fa_testlib import assert_close, dev, forward_inputs, gpu_backward, logical, say, spec_of

pytestmark = pytest.mark.gpu

HEAD_DIMS = [8, 32, 80, 96, 120]


def _cases(d):
    return {
        "extras_bf16": synth.EXTRAS_BF16.resized(head_dim=d, batch=2, num_heads=4, num_kv_heads=2, seq_q=230,
                                                 seq_k=230, window=90, scale=1.0 / np.sqrt(d), seed=700 + d),
        "causal_bf16": synth.LONG_BF16.resized(head_dim=d, num_heads=4, num_kv_heads=2, seq_q=300, seq_k=300,
                                               causal_offset=7, scale=1.0 / np.sqrt(d), seed=800 + d),
        "extras_f32": synth.EXTRAS_BF16.resized(dtype="f32", head_dim=d, batch=1, num_heads=4, num_kv_heads=2,
                                                seq_q=200, seq_k=200, window=60, scale=1.0 / np.sqrt(d),
                                                seed=900 + d),
        "causal_f32_bhsd": synth.CAUSAL_F32.resized(head_dim=d, batch=1, num_heads=2, num_kv_heads=2, seq_q=260,
                                                    seq_k=260, scale=1.0 / np.sqrt(d), seed=950 + d),
    }


CASES = [(d, n) for d in HEAD_DIMS for n in sorted(_cases(d))]


@pytest.mark.parametrize("d,name", CASES)
def test_backward_general_head_dim(d, name):
    w = _cases(d)[name]
    say(f"[head_dim {d}] {name}: {w}")
    inp = synth.prefill_inputs(w)
    o, lse = forward_inputs(w, inp)
    delta, rq, rk, rv = oracle.backward(inp["q"], inp["k"], inp["v"], o, inp["do"], lse, spec_of(w), inp["mask"])
    for share in ((False, True) if w.dtype == "bf16" else (False,)):
        got = gpu_backward(w, inp, o, lse, share_ds=share)
        assert_close(got["delta"], delta, "f32", "delta")
        assert_close(got["dq"], rq, w.dtype, f"dq (shared dS: {share})")
        assert_close(got["dk"], rk, w.dtype, f"dk (shared dS: {share})")
        assert_close(got["dv"], rv, w.dtype, f"dv (shared dS: {share})")


@pytest.mark.parametrize("d,name", CASES)
def test_forward_general_head_dim(d, name):
    w = _cases(d)[name]
    inp = synth.prefill_inputs(w)
    ref_o, ref_l = oracle.forward(inp["q"], inp["k"], inp["v"], spec_of(w), inp["mask"])
    q, k, v = (dev(inp[n], w.layout, w.dtype) for n in ("q", "k", "v"))
    mask = torch.from_numpy(inp["mask"]).cuda() if inp["mask"] is not None else None
    p = api.make_params(q, k, scale=w.scale, causal=w.causal, causal_offset=w.causal_offset, window=w.window,
                        dropout_p=w.dropout_p, seed=w.dropout_seed, mask=mask)
    o, lse = api.forward(p, q, k, v)
    lonly = api.lse(p, q, k)
    torch.cuda.synchronize()
    assert_close(logical(o), ref_o, w.dtype, "o")
    tol = 1e-4 if w.dtype == "bf16" else 1e-5
    for what, got in (("L", lse), ("L alone", lonly)):
        g = got.cpu().numpy().astype(np.float64)
        inf = np.isinf(ref_l)
        assert np.array_equal(np.isinf(g), inf), what
        err = np.abs(g[~inf] - ref_l[~inf]) / np.maximum(1.0, np.abs(ref_l[~inf]))
        say(f"  {what}: max err {err.max():.2e} (tol {tol:g})")
        assert err.max() <= tol, what


def test_outputs_past_the_head_dimension_are_untouched():
    """The kernels write dQ, dK, dV and O only up to head_dim: in tensors whose
    rows are wider than head_dim (a strided view), the columns past it keep what
    the caller put there."""
    d, wide = 40, 64
    w = synth.EXTRAS_BF16.resized(head_dim=d, batch=1, num_heads=4, num_kv_heads=2, seq_q=150, seq_k=150,
                                  window=50, scale=1.0 / np.sqrt(d), seed=990)
    inp = synth.prefill_inputs(w)
    o_ref, lse = forward_inputs(w, inp)

    def padded(x):  # logical [B,H,S,d] -> device [B,S,H,wide] bf16 filled with a sentinel, viewed [..., :d]
        B, H, S, _ = x.shape
        t = torch.full((B, S, H, wide), 7.0, dtype=torch.bfloat16)
        t[..., :d] = torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3))).to(torch.bfloat16)
        return t.cuda()[..., :d]

    q, k, v, do = (padded(inp[n]) for n in ("q", "k", "v", "do"))
    od = padded(o_ref)
    L = torch.from_numpy(lse).cuda()
    mask = torch.from_numpy(inp["mask"]).cuda()
    dq, dk, dv = (padded(np.zeros_like(x)) for x in (inp["q"], inp["k"], inp["v"]))
    o_out = padded(np.zeros_like(inp["q"]))
    p = api.make_params(q, k, scale=w.scale, causal=w.causal, window=w.window, dropout_p=w.dropout_p,
                        seed=w.dropout_seed, mask=mask)
    delta = api.preprocess(p, od, do)
    for share in (False, True):
        if share:
            ws = api.ds_workspace(p, q.device)
            api.dkdv_ds(p, q, k, v, do, L, delta, ws, dk, dv)
            api.dq_ds(p, q, k, ws, dq)
        else:
            api.dkdv(p, q, k, v, do, L, delta, dk, dv)
            api.dq(p, q, k, v, do, L, delta, dq)
        api.forward(p, q, k, v, o_out, torch.empty_like(L))
        torch.cuda.synchronize()
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv), ("o", o_out)):
            base = t.as_strided(t.shape[:3] + (wide,), t.stride())  # the full rows
            assert torch.all(base[..., d:].float() == 7.0), name
        _, rq, rk, rv = oracle.backward(inp["q"], inp["k"], inp["v"], o_ref, inp["do"], lse, spec_of(w), inp["mask"])
        for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            assert_close(logical(got), ref, "bf16", f"{name} (shared dS: {share})")
