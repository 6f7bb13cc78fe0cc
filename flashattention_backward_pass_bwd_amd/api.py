"""torch-facing wrappers over the C ABI (marshalling only).

Tensor convention: query-side tensors (q, o, do, dq) are indexed [B, Sq, Hq, D]
and key-side tensors (k, v, dk, dv) [B, Sk, Hkv, D]; any strides are accepted
as long as D is unit-stride, rows are 16-byte aligned, the tensors of one side
share one stride set (so [B,H,S,D] storage is passed as ``x.transpose(1, 2)``)
and that set maps distinct elements to distinct memory (the outputs are
written through it: no broadcast, stride-0 batch or sequence dimensions).
lse and delta are fp32 contiguous [B, Hq, Sq].  All calls enqueue on torch's
current HIP stream and return without synchronising.
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib


def _vp(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _lib.FA_DTYPE_BF16
    if t.dtype == torch.float32:
        return _lib.FA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16 or float32")


def make_params(q: torch.Tensor, k: torch.Tensor, *, scale: float, causal: bool = False,
                causal_offset: int = 0, window: int = 0, dropout_p: float = 0.0, seed: int = 0,
                mask: torch.Tensor | None = None) -> _lib.FaBwdParams:
    """Fill ``fa_bwd_params`` from a query-side and a key-side tensor.

    ``mask``: fp32 tensor broadcastable to [B, Hq, Sq, Sk] (e.g. [B, 1, Sq, Sk]);
    broadcast dimensions become stride-0.
    """
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be 4-d [B, S, H, D] views")
    B, Sq, Hq, D = q.shape
    Bk, Sk, Hkv, Dk = k.shape
    if Bk != B or Dk != D:
        raise ValueError("q and k disagree on batch or head_dim")
    if q.dtype != k.dtype:
        raise TypeError("q and k must share a dtype")
    p = _lib.FaBwdParams()
    p.dtype = _dtype_code(q)
    p.batch, p.num_heads, p.num_kv_heads, p.seq_q, p.seq_k, p.head_dim = B, Hq, Hkv, Sq, Sk, D
    p.q_stride_b, p.q_stride_s, p.q_stride_h = (int(s) for s in q.stride()[:3])
    p.kv_stride_b, p.kv_stride_s, p.kv_stride_h = (int(s) for s in k.stride()[:3])
    if q.stride(3) != 1 or k.stride(3) != 1:
        raise ValueError("head_dim must be unit-stride")
    p.scale = float(scale)
    p.causal = 1 if causal else 0
    p.causal_offset = int(causal_offset)
    p.window = int(window)
    p.dropout_p = float(dropout_p)
    p.seed = int(seed) & 0xFFFFFFFF
    if mask is not None:
        if mask.dtype != torch.float32:
            raise TypeError("mask must be float32")
        m = mask.expand(B, Hq, Sq, Sk)
        p.mask = m.data_ptr()
        p.mask_stride_b, p.mask_stride_h, p.mask_stride_q, p.mask_stride_k = (int(s) for s in m.stride())
    return p


def _same_layout(ref: torch.Tensor, *others: torch.Tensor) -> None:
    for t in others:
        if t.shape != ref.shape or t.stride() != ref.stride() or t.dtype != ref.dtype:
            raise ValueError("tensors of one side must share shape, strides and dtype")


def _like(t: torch.Tensor) -> torch.Tensor:
    return torch.empty_strided(t.shape, t.stride(), dtype=t.dtype, device=t.device)


def forward(p: _lib.FaBwdParams, q, k, v, o=None, lse=None):
    """Forward pass (bf16): O (q's shape and layout) and L fp32 [B, Hq, Sq]."""
    _same_layout(k, v)
    o = _like(q) if o is None else o
    _same_layout(q, o)
    if lse is None:
        lse = torch.empty((p.batch, p.num_heads, p.seq_q), dtype=torch.float32, device=q.device)
    _lib.check("fa_fwd", _lib.lib().fa_fwd(ctypes.byref(p), _vp(q), _vp(k), _vp(v), _vp(o), _vp(lse), _stream()))
    return o, lse


def lse(p: _lib.FaBwdParams, q, k, out=None):
    """L fp32 [B, Hq, Sq] alone (bf16), for a caller whose forward did not keep it."""
    if out is None:
        out = torch.empty((p.batch, p.num_heads, p.seq_q), dtype=torch.float32, device=q.device)
    _lib.check("fa_bwd_lse", _lib.lib().fa_bwd_lse(ctypes.byref(p), _vp(q), _vp(k), _vp(out), _stream()))
    return out


def preprocess(p: _lib.FaBwdParams, o: torch.Tensor, do: torch.Tensor, delta: torch.Tensor | None = None):
    _same_layout(o, do)
    if delta is None:
        delta = torch.empty((p.batch, p.num_heads, p.seq_q), dtype=torch.float32, device=o.device)
    _lib.check("fa_bwd_preprocess", _lib.lib().fa_bwd_preprocess(
        ctypes.byref(p), _vp(o), _vp(do), _vp(delta), _stream()))
    return delta


def dkdv(p: _lib.FaBwdParams, q, k, v, do, lse, delta, dk=None, dv=None):
    _same_layout(q, do)
    _same_layout(k, v)
    dk = _like(k) if dk is None else dk
    dv = _like(v) if dv is None else dv
    _same_layout(k, dk, dv)
    _lib.check("fa_bwd_dkdv", _lib.lib().fa_bwd_dkdv(
        ctypes.byref(p), _vp(q), _vp(k), _vp(v), _vp(do), _vp(lse), _vp(delta), _vp(dk), _vp(dv),
        _stream()))
    return dk, dv


def dq(p: _lib.FaBwdParams, q, k, v, do, lse, delta, dq_out=None):
    _same_layout(q, do)
    _same_layout(k, v)
    dq_out = _like(q) if dq_out is None else dq_out
    _same_layout(q, dq_out)
    _lib.check("fa_bwd_dq", _lib.lib().fa_bwd_dq(
        ctypes.byref(p), _vp(q), _vp(k), _vp(v), _vp(do), _vp(lse), _vp(delta), _vp(dq_out),
        _stream()))
    return dq_out


def ds_workspace_bytes(p: _lib.FaBwdParams) -> int:
    """Bytes of dS workspace fa_bwd_dkdv_ds / fa_bwd_dq_ds need for these parameters."""
    n = ctypes.c_uint64(0)
    _lib.check("fa_bwd_ds_workspace_size", _lib.lib().fa_bwd_ds_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return int(n.value)


def ds_workspace(p: _lib.FaBwdParams, device) -> torch.Tensor:
    """A workspace tensor of the size the dS entry points need (at least 16 bytes)."""
    return torch.empty(max(ds_workspace_bytes(p), 16), dtype=torch.uint8, device=device)


def dkdv_ds(p: _lib.FaBwdParams, q, k, v, do, lse, delta, ws, dk=None, dv=None):
    """dK/dV pass that also stores dS into the workspace ws (uint8 device tensor)."""
    _same_layout(q, do)
    _same_layout(k, v)
    dk = _like(k) if dk is None else dk
    dv = _like(v) if dv is None else dv
    _same_layout(k, dk, dv)
    _lib.check("fa_bwd_dkdv_ds", _lib.lib().fa_bwd_dkdv_ds(
        ctypes.byref(p), _vp(q), _vp(k), _vp(v), _vp(do), _vp(lse), _vp(delta), _vp(dk), _vp(dv),
        _vp(ws), ws.numel() * ws.element_size(), _stream()))
    return dk, dv


def dq_ds(p: _lib.FaBwdParams, q, k, ws, dq_out=None):
    """dQ from the dS that dkdv_ds stored in ws (q gives dQ's shape and layout only)."""
    dq_out = _like(q) if dq_out is None else dq_out
    _same_layout(q, dq_out)
    _lib.check("fa_bwd_dq_ds", _lib.lib().fa_bwd_dq_ds(
        ctypes.byref(p), _vp(k), _vp(ws), ws.numel() * ws.element_size(), _vp(dq_out), _stream()))
    return dq_out


def dkdv_dq_noalloc(p: _lib.FaBwdParams, q, k, v, do, lse, delta, dq_out=None, dk=None, dv=None):
    """Both passes of the shared-dS pair with the library-owned dS workspace
    (fa_bwd_dkdv_dq_noalloc: no device allocation in the library); returns (dq, dk, dv)."""
    _same_layout(q, do)
    _same_layout(k, v)
    dq_out = _like(q) if dq_out is None else dq_out
    dk = _like(k) if dk is None else dk
    dv = _like(v) if dv is None else dv
    _same_layout(q, dq_out)
    _same_layout(k, dk, dv)
    _lib.check("fa_bwd_dkdv_dq_noalloc", _lib.lib().fa_bwd_dkdv_dq_noalloc(
        ctypes.byref(p), _vp(q), _vp(k), _vp(v), _vp(do), _vp(lse), _vp(delta), _vp(dq_out), _vp(dk), _vp(dv),
        _stream()))
    return dq_out, dk, dv


# The shared-dS path's workspace grows as B * Hq * Sq * Sk * 2 bytes (8.7 GB for
# one 16k x 16k sequence of 32 heads): it is used only while it fits in this
# share of the device memory that is free at the call.
DS_WORKSPACE_FRACTION = 0.5


def use_shared_ds(dtype_code: int, ws_bytes: int, free_bytes: int, fraction: float = DS_WORKSPACE_FRACTION) -> bool:
    """Path choice of backward(): share dS through a workspace (bf16 only) when
    the workspace takes at most `fraction` of the free device memory, else
    recompute dS in the dQ pass (no workspace)."""
    return dtype_code == _lib.FA_DTYPE_BF16 and 0 < ws_bytes <= fraction * free_bytes


def backward(q, k, v, o, do, lse, *, scale, causal=False, causal_offset=0, window=0, dropout_p=0.0,
             seed=0, mask=None, share_ds=None):
    """Delta preprocess, then the dK/dV and dQ passes; returns (dq, dk, dv, delta).

    share_ds: None or True -- bf16 shares dS: the dK/dV pass stores it in a
    workspace and the dQ pass reads it (fa_bwd_dkdv_ds, fa_bwd_dq_ds) instead of
    recomputing it, as long as the workspace fits in DS_WORKSPACE_FRACTION of
    the free device memory (use_shared_ds); otherwise, for fp32, or with
    share_ds=False, both passes recompute (fa_bwd_dkdv, fa_bwd_dq)."""
    p = make_params(q, k, scale=scale, causal=causal, causal_offset=causal_offset, window=window,
                    dropout_p=dropout_p, seed=seed, mask=mask)
    _same_layout(q, o, do)
    delta = preprocess(p, o, do)
    if share_ds is None or share_ds:
        share_ds = p.dtype == _lib.FA_DTYPE_BF16 and use_shared_ds(
            p.dtype, ds_workspace_bytes(p), torch.cuda.mem_get_info(q.device)[0])
    if share_ds:
        ws = ds_workspace(p, q.device)
        dk_, dv_ = dkdv_ds(p, q, k, v, do, lse, delta, ws)
        dq_ = dq_ds(p, q, k, ws)
    else:
        dk_, dv_ = dkdv(p, q, k, v, do, lse, delta)
        dq_ = dq(p, q, k, v, do, lse, delta)
    return dq_, dk_, dv_, delta


def decode_params(k_hist: torch.Tensor, probs: torch.Tensor) -> _lib.FaDecodeParams:
    N, L, Hkv, D = k_hist.shape
    p = _lib.FaDecodeParams()
    p.num_seqs, p.n_heads, p.n_kv_heads, p.head_dim, p.history_len = N, probs.shape[1], Hkv, D, L
    return p


def decode_backward(k_hist, v_hist, probs, d_out, d_scores=None, d_q=None):
    """Decode-step backward: returns (d_scores [N,H,len], d_q [N,H,D]); fp32 contiguous tensors."""
    for t in (k_hist, v_hist, probs, d_out):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("decode tensors must be contiguous float32")
    p = decode_params(k_hist, probs)
    d_scores = torch.empty_like(probs) if d_scores is None else d_scores
    d_q = torch.empty_like(d_out) if d_q is None else d_q
    _lib.check("fa_bwd_decode", _lib.lib().fa_bwd_decode(
        ctypes.byref(p), _vp(k_hist), _vp(v_hist), _vp(probs), _vp(d_out), _vp(d_scores), _vp(d_q),
        _stream()))
    return d_scores, d_q


def decode_dkdv(q, d_out, probs, d_scores, n_kv_heads: int, dk_hist=None, dv_hist=None):
    """Decode-step backward pass 2: history dK, dV [N, len, Hkv, D] from q, d_out
    [N, H, D] and probs, d_scores [N, H, len]; fp32 contiguous tensors."""
    for t in (q, d_out, probs, d_scores):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("decode tensors must be contiguous float32")
    N, H, D = q.shape
    L = probs.shape[2]
    p = _lib.FaDecodeParams(num_seqs=N, n_heads=H, n_kv_heads=n_kv_heads, head_dim=D, history_len=L)
    shape = (N, L, n_kv_heads, D)
    dk_hist = torch.empty(shape, dtype=torch.float32, device=q.device) if dk_hist is None else dk_hist
    dv_hist = torch.empty(shape, dtype=torch.float32, device=q.device) if dv_hist is None else dv_hist
    _lib.check("fa_bwd_decode_dkdv", _lib.lib().fa_bwd_decode_dkdv(
        ctypes.byref(p), _vp(q), _vp(d_out), _vp(probs), _vp(d_scores), _vp(dk_hist), _vp(dv_hist), _stream()))
    return dk_hist, dv_hist


def debug_visibility(p: _lib.FaBwdParams, device) -> torch.Tensor:
    out = torch.empty((p.batch, p.num_heads, p.seq_q, p.seq_k), dtype=torch.uint8, device=device)
    _lib.check("fa_bwd_debug_visibility", _lib.lib().fa_bwd_debug_visibility(ctypes.byref(p), _vp(out), _stream()))
    return out


def debug_dropout_keep(p: _lib.FaBwdParams, device) -> torch.Tensor:
    out = torch.empty((p.batch, p.num_heads, p.seq_q, p.seq_k), dtype=torch.uint8, device=device)
    _lib.check("fa_bwd_debug_dropout_keep", _lib.lib().fa_bwd_debug_dropout_keep(ctypes.byref(p), _vp(out), _stream()))
    return out


def calib_mfma_bf16(operands: torch.Tensor, sink: torch.Tensor, blocks: int, iters: int) -> None:
    """Enqueue the MFMA calibration kernel (see include/fa_bwd.h) on the current stream.

    operands: bf16 device tensor of at least 2048 * 8 elements; sink: fp32 device
    tensor of at least blocks * 256 elements.  Work: blocks * 4 * iters * 32 * 32768 FLOP.
    """
    if operands.dtype != torch.bfloat16 or operands.numel() < 2048 * 8 or not operands.is_contiguous():
        raise ValueError("operands: contiguous bf16 tensor of at least 16384 elements")
    if sink.dtype != torch.float32 or sink.numel() < blocks * 256:
        raise ValueError("sink: fp32 tensor of at least blocks*256 elements")
    _lib.check("fa_bwd_calib_mfma_bf16",
               _lib.lib().fa_bwd_calib_mfma_bf16(_vp(operands), _vp(sink), blocks, iters, _stream()))
