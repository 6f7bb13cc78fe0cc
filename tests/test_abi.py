"""C ABI checks that need no GPU (CPU only).

* libfa_bwd.so loads and exports every function include/fa_bwd.h declares;
* the ctypes mirrors of the parameter structs match the C layout (gcc probe);
* every invalid argument is rejected with its status code before any HIP call.
"""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from flashattention_backward_pass_bwd_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_bwd.h")
CALIB_HEADER = os.path.join(ROOT, "include", "fa_bwd_calib.h")  # the measurement hook, apart from the method

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libfa_bwd.so not built")


def _declared_functions(headers=(HEADER, CALIB_HEADER)):
    text = "".join(open(h).read() for h in headers)
    return sorted(set(re.findall(r"^\s*(?:fa_status|int32_t|const char\*)\s+(fa_\w+)\s*\(", text, re.M)))


def test_method_header_holds_only_the_method():
    assert "fa_bwd_calib_mfma_bf16" not in _declared_functions((HEADER,))
    assert _declared_functions((CALIB_HEADER,)) == ["fa_bwd_calib_mfma_bf16"]


def test_header_declares_the_binding_surface():
    assert _declared_functions() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    for name in _declared_functions():
        assert re.search(rf"\bT {name}\b", out), name


def test_struct_layouts_match_c():
    src = r"""
    #include <stdio.h>
    #include <stddef.h>
    #include "fa_bwd.h"
    #define F(s, m) printf(#m " %zu\n", offsetof(s, m));
    int main(void) {
      printf("size_bwd %zu\nsize_dec %zu\n", sizeof(fa_bwd_params), sizeof(fa_decode_params));
      F(fa_bwd_params, q_stride_b) F(fa_bwd_params, kv_stride_h) F(fa_bwd_params, scale)
      F(fa_bwd_params, dropout_p) F(fa_bwd_params, seed) F(fa_bwd_params, mask) F(fa_bwd_params, mask_stride_k)
      F(fa_decode_params, history_len)
      return 0;
    }
    """
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "probe.c")
        exe = os.path.join(d, "probe")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        lines = dict(l.split() for l in subprocess.run([exe], capture_output=True, text=True).stdout.splitlines())
    assert int(lines["size_bwd"]) == ctypes.sizeof(_lib.FaBwdParams)
    assert int(lines["size_dec"]) == ctypes.sizeof(_lib.FaDecodeParams)
    for name in ("q_stride_b", "kv_stride_h", "scale", "dropout_p", "seed", "mask", "mask_stride_k"):
        assert int(lines[name]) == getattr(_lib.FaBwdParams, name).offset, name
    assert int(lines["history_len"]) == _lib.FaDecodeParams.history_len.offset


def _valid():
    p = _lib.FaBwdParams()
    p.dtype = _lib.FA_DTYPE_BF16
    p.batch, p.num_heads, p.num_kv_heads, p.seq_q, p.seq_k, p.head_dim = 2, 8, 2, 100, 120, 128
    p.q_stride_b, p.q_stride_s, p.q_stride_h = 100 * 8 * 128, 8 * 128, 128
    p.kv_stride_b, p.kv_stride_s, p.kv_stride_h = 120 * 2 * 128, 2 * 128, 128
    p.scale = 0.088
    return p


FAKE = ctypes.c_void_p(4096)  # never dereferenced: every case below fails validation first

BAD = [
    ("head_dim", 0, _lib.FA_ERR_SHAPE),
    ("dtype", 7, _lib.FA_ERR_UNSUPPORTED),
    ("batch", 0, _lib.FA_ERR_SHAPE),
    ("seq_q", -1, _lib.FA_ERR_SHAPE),
    ("seq_k", 0, _lib.FA_ERR_SHAPE),
    ("num_kv_heads", 3, _lib.FA_ERR_SHAPE),
    ("dropout_p", 1.0, _lib.FA_ERR_ARG),
    ("dropout_p", -0.1, _lib.FA_ERR_ARG),
    ("dropout_p", float("nan"), _lib.FA_ERR_ARG),
    ("causal_offset", -1, _lib.FA_ERR_ARG),
    ("window", -5, _lib.FA_ERR_ARG),
    ("causal", 2, _lib.FA_ERR_ARG),
    ("q_stride_s", 8 * 128 + 4, _lib.FA_ERR_ALIGN),
    ("kv_stride_h", 130, _lib.FA_ERR_ALIGN),
    ("q_stride_b", -1, _lib.FA_ERR_ARG),
    # outputs are written through the same strides: layouts whose rows overlap are rejected
    ("q_stride_b", 0, _lib.FA_ERR_ARG),        # two batches on one row set
    ("kv_stride_s", 0, _lib.FA_ERR_ARG),       # every key on one row
    ("q_stride_h", 64, _lib.FA_ERR_ARG),       # heads 64 elements apart, rows of 128
    ("kv_stride_b", 2 * 128, _lib.FA_ERR_ARG),  # batch 1 starts inside batch 0's keys
    # block counts fit 32 bits: batch * num_heads * ceil(seq / 32) < 2^31
    ("batch", 1 << 26, _lib.FA_ERR_UNSUPPORTED),
    # head_dim: any multiple of 8 up to 128
    ("head_dim", 0, _lib.FA_ERR_SHAPE),
    ("head_dim", 100, _lib.FA_ERR_UNSUPPORTED),
    ("head_dim", 136, _lib.FA_ERR_UNSUPPORTED),
    ("head_dim", 4, _lib.FA_ERR_UNSUPPORTED),
    # the score chains start from -L / scale: a zero, infinite, NaN or subnormal scale is rejected
    ("scale", 0.0, _lib.FA_ERR_ARG),
    ("scale", float("inf"), _lib.FA_ERR_ARG),
    ("scale", float("nan"), _lib.FA_ERR_ARG),
    ("scale", 1e-39, _lib.FA_ERR_ARG),
]


@pytest.mark.parametrize("field,value,code", BAD)
def test_invalid_prefill_arguments(field, value, code):
    L = _lib.lib()
    p = _valid()
    setattr(p, field, value)
    P = ctypes.byref(p)
    assert L.fa_bwd_preprocess(P, FAKE, FAKE, FAKE, None) == code
    assert L.fa_fwd(P, FAKE, FAKE, FAKE, FAKE, FAKE, None) == code
    assert L.fa_bwd_lse(P, FAKE, FAKE, FAKE, None) == code
    assert L.fa_bwd_dkdv(P, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == code
    assert L.fa_bwd_dq(P, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == code
    assert L.fa_bwd_debug_visibility(P, FAKE, None) == code
    assert L.fa_bwd_debug_dropout_keep(P, FAKE, None) == code
    assert L.fa_bwd_dkdv_ds(P, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == code
    assert L.fa_bwd_dq_ds(P, FAKE, FAKE, 1 << 40, FAKE, None) == code
    assert L.fa_bwd_dkdv_dq_noalloc(P, *([FAKE] * 9), None) == code


def test_null_and_misaligned_pointers():
    L = _lib.lib()
    p = _valid()
    P = ctypes.byref(p)
    assert L.fa_bwd_preprocess(None, FAKE, FAKE, FAKE, None) == _lib.FA_ERR_NULL
    assert L.fa_bwd_preprocess(P, None, FAKE, FAKE, None) == _lib.FA_ERR_NULL
    assert L.fa_bwd_dkdv(P, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == _lib.FA_ERR_NULL
    assert L.fa_bwd_dq(P, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == _lib.FA_ERR_NULL
    odd = ctypes.c_void_p(4096 + 8)
    assert L.fa_bwd_preprocess(P, odd, FAKE, FAKE, None) == _lib.FA_ERR_ALIGN
    assert L.fa_bwd_dkdv(P, FAKE, odd, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == _lib.FA_ERR_ALIGN
    assert L.fa_bwd_dq(P, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, odd, None) == _lib.FA_ERR_ALIGN
    p.mask = 4096 + 2
    assert L.fa_bwd_dq(P, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == _lib.FA_ERR_ALIGN
    p.mask = 4096
    p.mask_stride_q = -2
    assert L.fa_bwd_dq(P, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == _lib.FA_ERR_ARG


def test_invalid_decode_arguments():
    L = _lib.lib()

    def dp(**kw):
        p = _lib.FaDecodeParams()
        p.num_seqs, p.n_heads, p.n_kv_heads, p.head_dim, p.history_len = 4, 32, 8, 256, 4096
        for k, v in kw.items():
            setattr(p, k, v)
        return p

    def call(p, *ptrs):
        ptrs = ptrs or (FAKE,) * 6
        return L.fa_bwd_decode(ctypes.byref(p), *ptrs, None)

    assert call(dp(n_kv_heads=5)) == _lib.FA_ERR_SHAPE
    assert call(dp(num_seqs=0)) == _lib.FA_ERR_SHAPE
    assert call(dp(n_heads=48, n_kv_heads=4)) == _lib.FA_ERR_UNSUPPORTED  # 12 heads per KV head
    assert call(dp(head_dim=96)) == _lib.FA_ERR_UNSUPPORTED
    maxlen = L.fa_bwd_decode_max_history(ctypes.byref(dp()))
    assert maxlen >= 8192
    assert call(dp(history_len=maxlen + 1)) == _lib.FA_ERR_UNSUPPORTED
    assert call(dp(), None, FAKE, FAKE, FAKE, FAKE, FAKE) == _lib.FA_ERR_NULL
    assert call(dp(), FAKE, ctypes.c_void_p(4100), FAKE, FAKE, FAKE, FAKE) == _lib.FA_ERR_ALIGN
    assert L.fa_bwd_decode_max_history(ctypes.byref(dp(n_heads=30))) == 0


def _ws_bytes(L, p):
    n = ctypes.c_uint64(0)
    assert L.fa_bwd_ds_workspace_size(ctypes.byref(p), ctypes.byref(n)) == _lib.FA_OK
    return n.value


def test_invalid_workspace_arguments():
    L = _lib.lib()
    p = _valid()
    P = ctypes.byref(p)
    need = _ws_bytes(L, p)
    assert need > 0
    odd = ctypes.c_void_p(4096 + 8)
    assert L.fa_bwd_ds_workspace_size(None, None) == _lib.FA_ERR_NULL
    assert L.fa_bwd_ds_workspace_size(P, None) == _lib.FA_ERR_NULL
    dkdv = lambda ws, nb: L.fa_bwd_dkdv_ds(P, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, nb, None)
    assert dkdv(None, need) == _lib.FA_ERR_NULL
    assert dkdv(FAKE, need - 1) == _lib.FA_ERR_ARG
    assert dkdv(odd, need) == _lib.FA_ERR_ALIGN
    assert L.fa_bwd_dq_ds(P, FAKE, None, need, FAKE, None) == _lib.FA_ERR_NULL
    assert L.fa_bwd_dq_ds(P, FAKE, FAKE, need, None, None) == _lib.FA_ERR_NULL
    assert L.fa_bwd_dq_ds(P, FAKE, FAKE, need - 1, FAKE, None) == _lib.FA_ERR_ARG
    assert L.fa_bwd_dq_ds(P, FAKE, odd, need, FAKE, None) == _lib.FA_ERR_ALIGN
    assert L.fa_bwd_dq_ds(P, odd, FAKE, need, FAKE, None) == _lib.FA_ERR_ALIGN
    p.dtype = _lib.FA_DTYPE_F32  # the shared-dS passes are bf16 only
    n = ctypes.c_uint64(0)
    assert L.fa_bwd_ds_workspace_size(P, ctypes.byref(n)) == _lib.FA_ERR_UNSUPPORTED
    assert dkdv(FAKE, 1 << 40) == _lib.FA_ERR_UNSUPPORTED
    assert L.fa_bwd_dq_ds(P, FAKE, FAKE, 1 << 40, FAKE, None) == _lib.FA_ERR_UNSUPPORTED


# (seq_q, seq_k, causal, causal_offset, window): full, causal, offsets that
# leave key blocks' first rows off the 64-row grid, windows with and without
# causal, rows or keys nobody sees, and the extras workload's geometry.
WS_GEOMS = [
    (100, 120, 0, 0, 0),
    (1100, 1100, 1, 0, 0),
    (300, 520, 1, 220, 130),
    (260, 400, 1, 157, 0),
    (300, 150, 0, 0, 20),
    (200, 190, 0, 5, 33),
    (80, 300, 1, 0, 0),
    (70, 70, 1, 0, 1),
    (2048, 2048, 1, 0, 512),
]


@pytest.mark.parametrize("geom", WS_GEOMS)
def test_ds_workspace_counts_visible_tiles(geom):
    """The workspace holds one 16 KB tile per (b, h) and 64-row x 128-key block
    with at least one visible element: checked against the oracle's own
    visibility rule, counted by brute force."""
    import numpy as np
    import oracle
    from oracle.attention import visible
    sq, sk, causal, off, win = geom
    L = _lib.lib()
    p = _valid()
    p.seq_q, p.seq_k, p.causal, p.causal_offset, p.window = sq, sk, causal, off, win
    p.q_stride_b, p.kv_stride_b = sq * 8 * 128, sk * 2 * 128
    vis = visible(np.arange(sq), np.arange(sk), sq, sk,
                  oracle.Spec(scale=0.1, causal=bool(causal), causal_offset=off, window=win))
    nt, nk = -(-sq // 64), -(-sk // 128)
    pad = np.zeros((nt * 64, nk * 128), dtype=bool)
    pad[:sq, :sk] = vis
    tiles = int(pad.reshape(nt, 64, nk, 128).any(axis=(1, 3)).sum())
    assert _ws_bytes(L, p) == p.batch * p.num_heads * tiles * 16384


def test_invalid_forward_arguments():
    L = _lib.lib()
    p = _valid()
    P = ctypes.byref(p)
    odd = ctypes.c_void_p(4096 + 8)
    assert L.fa_fwd(P, None, FAKE, FAKE, FAKE, FAKE, None) == _lib.FA_ERR_NULL
    assert L.fa_fwd(P, FAKE, FAKE, FAKE, FAKE, None, None) == _lib.FA_ERR_NULL
    assert L.fa_fwd(P, FAKE, FAKE, FAKE, odd, FAKE, None) == _lib.FA_ERR_ALIGN
    assert L.fa_fwd(P, FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(4096 + 2), None) == _lib.FA_ERR_ALIGN
    assert L.fa_bwd_lse(P, FAKE, None, FAKE, None) == _lib.FA_ERR_NULL
    assert L.fa_bwd_lse(P, FAKE, odd, FAKE, None) == _lib.FA_ERR_ALIGN
    p.dtype = _lib.FA_DTYPE_F32
    assert L.fa_fwd(P, None, FAKE, FAKE, FAKE, FAKE, None) == _lib.FA_ERR_NULL
    assert L.fa_bwd_lse(P, FAKE, odd, FAKE, None) == _lib.FA_ERR_ALIGN
    p.head_dim = 100  # not a multiple of 8
    assert L.fa_fwd(P, FAKE, FAKE, FAKE, FAKE, FAKE, None) == _lib.FA_ERR_UNSUPPORTED


def test_invalid_decode_pass2_arguments():
    L = _lib.lib()
    def dp(**kw):
        p = _lib.FaDecodeParams(num_seqs=2, n_heads=8, n_kv_heads=2, head_dim=128, history_len=100)
        for k, v in kw.items():
            setattr(p, k, v)
        return ctypes.byref(p)
    f = L.fa_bwd_decode_dkdv
    odd = ctypes.c_void_p(4096 + 8)
    assert f(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == _lib.FA_ERR_NULL
    assert f(dp(), FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == _lib.FA_ERR_NULL
    assert f(dp(history_len=0), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == _lib.FA_ERR_SHAPE
    assert f(dp(n_kv_heads=3), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == _lib.FA_ERR_SHAPE
    assert f(dp(n_heads=24, n_kv_heads=2), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == _lib.FA_ERR_UNSUPPORTED
    assert f(dp(head_dim=96), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == _lib.FA_ERR_UNSUPPORTED
    assert f(dp(), odd, FAKE, FAKE, FAKE, FAKE, FAKE, None) == _lib.FA_ERR_ALIGN
    assert f(dp(), FAKE, FAKE, FAKE, FAKE, FAKE, odd, None) == _lib.FA_ERR_ALIGN
    assert f(dp(), FAKE, FAKE, ctypes.c_void_p(4096 + 2), FAKE, FAKE, FAKE, None) == _lib.FA_ERR_ALIGN


def test_invalid_calibration_arguments():
    L = _lib.lib()
    f = L.fa_bwd_calib_mfma_bf16
    assert f(None, FAKE, 4, 1, None) == _lib.FA_ERR_NULL
    assert f(FAKE, None, 4, 1, None) == _lib.FA_ERR_NULL
    assert f(FAKE, FAKE, 0, 1, None) == _lib.FA_ERR_ARG
    assert f(FAKE, FAKE, 4, -1, None) == _lib.FA_ERR_ARG
    assert f(ctypes.c_void_p(4096 + 4), FAKE, 4, 1, None) == _lib.FA_ERR_ALIGN


def test_invalid_noalloc_arguments():
    L = _lib.lib()
    p = _valid()
    P = ctypes.byref(p)
    f = lambda *ptrs: L.fa_bwd_dkdv_dq_noalloc(P, *ptrs, None)
    ten = [FAKE] * 9
    odd = ctypes.c_void_p(4096 + 8)
    assert L.fa_bwd_dkdv_dq_noalloc(None, *ten, None) == _lib.FA_ERR_NULL
    for i in range(9):
        assert f(*ten[:i], None, *ten[i + 1:]) == _lib.FA_ERR_NULL, i
    assert f(odd, *ten[1:]) == _lib.FA_ERR_ALIGN
    assert f(*ten[:6], odd, *ten[7:]) == _lib.FA_ERR_ALIGN
    # a problem whose dS workspace exceeds the library-owned buffer: rejected before any HIP call
    p.seq_q = p.seq_k = 8192
    p.q_stride_b, p.kv_stride_b = 8192 * 8 * 128, 8192 * 2 * 128
    assert _ws_bytes(L, p) > _lib.NOALLOC_SCRATCH_BYTES
    assert f(*ten) == _lib.FA_ERR_SCRATCH
    p.dtype = _lib.FA_DTYPE_F32
    assert f(*ten) == _lib.FA_ERR_UNSUPPORTED


def test_noalloc_buffer_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define FA_BWD_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.NOALLOC_SCRATCH_BYTES


def test_status_strings():
    for code in range(-7, 1):
        s = _lib.status_string(code)
        assert s.startswith("FA_")
    assert "unknown" in _lib.status_string(-99)


@pytest.mark.parametrize("head_dim", [8, 16, 40, 72, 96, 120, 128])
def test_general_head_dims_pass_validation(head_dim):
    """Every multiple of 8 up to 128 passes the checks: a call with NULL data
    pointers then stops at FA_ERR_NULL, never at FA_ERR_UNSUPPORTED."""
    L = _lib.lib()
    for dtype in (_lib.FA_DTYPE_BF16, _lib.FA_DTYPE_F32):
        p = _valid()
        p.dtype, p.head_dim = dtype, head_dim
        p.q_stride_b, p.q_stride_s, p.q_stride_h = 100 * 8 * head_dim, 8 * head_dim, head_dim
        p.kv_stride_b, p.kv_stride_s, p.kv_stride_h = 120 * 2 * head_dim, 2 * head_dim, head_dim
        P = ctypes.byref(p)
        assert L.fa_bwd_dkdv(P, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == _lib.FA_ERR_NULL
        assert L.fa_bwd_dq(P, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == _lib.FA_ERR_NULL
        assert L.fa_fwd(P, FAKE, FAKE, FAKE, None, FAKE, None) == _lib.FA_ERR_NULL
        if dtype == _lib.FA_DTYPE_BF16:
            assert _ws_bytes(L, p) > 0


@pytest.mark.parametrize("layout", ["bshd", "bhsd", "padded_rows", "size_one_dims_any_stride"])
def test_non_overlapping_layouts_are_accepted(layout):
    """[B,S,H,D], [B,H,S,D], rows padded past head_dim, and dimensions of extent 1
    with any stride pass the layout check (workspace sizing validates the
    parameters without launching anything)."""
    p = _valid()
    if layout == "bhsd":
        p.q_stride_b, p.q_stride_h, p.q_stride_s = 8 * 100 * 128, 100 * 128, 128
        p.kv_stride_b, p.kv_stride_h, p.kv_stride_s = 2 * 120 * 128, 120 * 128, 128
    elif layout == "padded_rows":
        p.head_dim = 40
        p.q_stride_b, p.q_stride_s, p.q_stride_h = 100 * 8 * 64, 8 * 64, 64
        p.kv_stride_b, p.kv_stride_s, p.kv_stride_h = 120 * 2 * 64, 2 * 64, 64
    elif layout == "size_one_dims_any_stride":
        p.batch, p.num_kv_heads = 1, 1
        p.q_stride_b, p.kv_stride_b, p.kv_stride_h = 0, 8, 0
    size = ctypes.c_uint64(0)
    assert _lib.lib().fa_bwd_ds_workspace_size(ctypes.byref(p), ctypes.byref(size)) == _lib.FA_OK
    assert size.value > 0
