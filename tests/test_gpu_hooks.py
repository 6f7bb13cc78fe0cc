"""Bitwise checks of the device visibility predicate and dropout hash (GPU).

The hooks run the very device functions the backward kernels evaluate; the
oracle's numpy predicate and hash must agree on every (b, h, i, j).  A
black-box check recovers the keep mask from dV (dO = one-hot rows) so the
kernels' own use of the hash is checked too.
"""
import numpy as np
import pytest
import torch

import oracle
from flashattention_backward_pass_bwd_amd import api, synth

from fa_testlib import dev, forward_inputs, gpu_backward, say, spec_of

pytestmark = pytest.mark.gpu

GEOMS = [
    dict(B=2, Hq=4, Hkv=2, Sq=70, Sk=90, causal=True, off=20, window=0, density=0.0),
    dict(B=1, Hq=3, Hkv=1, Sq=64, Sk=64, causal=False, off=3, window=7, density=0.2),
    dict(B=2, Hq=2, Hkv=2, Sq=129, Sk=129, causal=True, off=0, window=16, density=0.05),
    # the geometry of the bf16 GQA window workload (one batch, two heads)
    dict(B=1, Hq=2, Hkv=1, Sq=2048, Sk=2048, causal=True, off=0, window=512, density=0.05),
]


def _setup(g, dropout_p=0.1, seed=7):
    rng = np.random.default_rng(5)
    q = torch.zeros((g["B"], g["Sq"], g["Hq"], 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((g["B"], g["Sk"], g["Hkv"], 64), dtype=torch.bfloat16, device="cuda")
    mask = None
    if g["density"] > 0:
        mask = np.where(rng.random((g["B"], 1, g["Sq"], g["Sk"])) < g["density"], -1e30, 0.0).astype(np.float32)
    mdev = None if mask is None else torch.from_numpy(mask).cuda()
    p = api.make_params(q, k, scale=0.125, causal=g["causal"], causal_offset=g["off"], window=g["window"],
                        dropout_p=dropout_p, seed=seed, mask=mdev)
    spec = oracle.Spec(scale=0.125, causal=g["causal"], causal_offset=g["off"], window=g["window"],
                       dropout_p=dropout_p, seed=seed)
    return p, spec, mask, mdev


@pytest.mark.parametrize("gi", range(len(GEOMS)))
def test_visibility_bitwise(gi):
    g = GEOMS[gi]
    p, spec, mask, _mdev = _setup(g)
    got = api.debug_visibility(p, "cuda").cpu().numpy()
    vis = oracle.visible(np.arange(g["Sq"]), np.arange(g["Sk"]), g["Sq"], g["Sk"], spec)
    for b in range(g["B"]):
        for h in range(g["Hq"]):
            mv = None if mask is None else mask[b, 0]
            want = oracle.counted(vis, mv)
            assert np.array_equal(got[b, h].astype(bool), want), (b, h)
    if gi == 3:
        assert vis.sum() == 917760


@pytest.mark.parametrize("gi", range(len(GEOMS)))
def test_dropout_keep_bitwise(gi):
    g = GEOMS[gi]
    for p_drop, seed in ((0.1, 7), (0.5, 0xDEADBEEF), (0.0, 3)):
        p, spec, _m, _d = _setup(g, dropout_p=p_drop, seed=seed)
        got = api.debug_dropout_keep(p, "cuda").cpu().numpy().astype(bool)
        for b in range(g["B"]):
            for h in range(g["Hq"]):
                if p_drop == 0.0:
                    want = np.ones((g["Sq"], g["Sk"]), bool)
                else:
                    want = oracle.dropout_keep(seed, b, h, g["Hq"], g["Sq"], np.arange(g["Sq"]),
                                               np.arange(g["Sk"]), p_drop)
                assert np.array_equal(got[b, h], want), (b, h, p_drop)


def test_keep_mask_recovered_from_dv():
    # dO_i = e_i (one-hot, Sq <= D): dV_j[i] = sum_h P_ij M_ij, so with one query head per KV head
    # the nonzero pattern of dV^T equals the keep mask on visible elements.
    S, D = 48, 64
    w = synth.PrefillWorkload(name="keep_recovery", dtype="f32", batch=1, num_heads=2, num_kv_heads=2,
                              seq_q=S, seq_k=S, head_dim=D, layout="bshd", scale=0.3, causal=True,
                              dropout_p=0.4, dropout_seed=4242, seed=31)
    inp = synth.prefill_inputs(w)
    inp["do"][:] = 0.0
    for h in range(2):
        inp["do"][0, h, np.arange(S), np.arange(S)] = 1.0
    o, lse = forward_inputs(w, inp)
    got = gpu_backward(w, inp, o, lse)
    spec = spec_of(w)
    for h in range(2):
        keep = oracle.dropout_keep(w.dropout_seed, 0, h, 2, S, np.arange(S), np.arange(S), w.dropout_p)
        vis = oracle.visible(np.arange(S), np.arange(S), S, S, spec)
        nz = got["dv"][0, h][:, :S].T != 0.0  # [i, j]
        assert np.array_equal(nz, keep & vis), h
        say(f"  head {h}: {int((keep & vis).sum())} kept of {int(vis.sum())} visible")


def test_mfma_calibration_kernel_sums():
    """The MFMA calibration kernel does the products it claims.

    With one iteration, the sum of every accumulator element of a wave equals
    sum over its 32 MFMAs of sum_k (sum_m A[m,k]) (sum_n B[k,n]), where lane l
    holds A[l%32][8(l/32) .. +7] and B[8(l/32) .. +7][l%32]; MFMA j uses A block
    (j/4)%4 and B block (j/2)%4.  Checked per wave against fp64 on the host.
    """
    g = torch.Generator(device="cpu").manual_seed(3)
    ops = torch.randn(2048 * 8, generator=g).to(torch.bfloat16)
    blocks = 2
    sink = torch.zeros(blocks * 256, dtype=torch.float32, device="cuda")
    api.calib_mfma_bf16(ops.cuda(), sink, blocks, 1)
    torch.cuda.synchronize()
    got = sink.cpu().double().view(blocks, 4, 64).sum(dim=2)  # per (block, wave)
    v = ops.double().view(2048, 8)
    for w in range(4):
        t = 64 * w + torch.arange(64)
        kblk = (torch.arange(64) // 32)  # lane's 8-wide k block
        want, mag = 0.0, 0.0
        for j in range(32):
            a = v[t + 256 * ((j >> 2) & 3)]          # [64 lanes, 8]
            b = v[1024 + t + 256 * ((j >> 1) & 3)]
            for kb in range(2):
                sel = kblk == kb
                terms = a[sel].sum(dim=0) * b[sel].sum(dim=0)
                want += float(terms.sum())
                mag += float(terms.abs().sum())
        for blk in range(blocks):
            assert abs(float(got[blk, w]) - want) <= 1e-4 * mag + 1e-3, (blk, w, float(got[blk, w]), want, mag)
