"""ctypes binding of libfa_bwd.so (include/fa_bwd.h).

Argument marshalling only: every step of the backward pass runs in the HIP
kernels behind the C ABI.  torch tensors supply device pointers, strides and
the current HIP stream; nothing here computes attention.  The library is
loaded on first use and a missing build raises -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa_bwd.so")

FA_OK = 0
FA_ERR_NULL = -1
FA_ERR_SHAPE = -2
FA_ERR_UNSUPPORTED = -3
FA_ERR_ALIGN = -4
FA_ERR_ARG = -5
FA_ERR_HIP = -6
FA_ERR_SCRATCH = -7

# Size of the library-owned dS workspace of fa_bwd_dkdv_dq_noalloc (FA_BWD_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 128 << 20

FA_DTYPE_F32 = 0
FA_DTYPE_BF16 = 1

# Every function include/fa_bwd.h declares.
EXPORTED = (
    "fa_fwd",
    "fa_bwd_lse",
    "fa_bwd_preprocess",
    "fa_bwd_dkdv",
    "fa_bwd_dq",
    "fa_bwd_ds_workspace_size",
    "fa_bwd_dkdv_ds",
    "fa_bwd_dq_ds",
    "fa_bwd_dkdv_dq_noalloc",
    "fa_bwd_decode",
    "fa_bwd_decode_dkdv",
    "fa_bwd_decode_max_history",
    "fa_bwd_status_string",
    "fa_bwd_debug_visibility",
    "fa_bwd_debug_dropout_keep",
    "fa_bwd_calib_mfma_bf16",
)


class FaBwdParams(ctypes.Structure):
    """Mirror of ``fa_bwd_params``."""

    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("seq_q", ctypes.c_int32),
        ("seq_k", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("q_stride_b", ctypes.c_int64),
        ("q_stride_s", ctypes.c_int64),
        ("q_stride_h", ctypes.c_int64),
        ("kv_stride_b", ctypes.c_int64),
        ("kv_stride_s", ctypes.c_int64),
        ("kv_stride_h", ctypes.c_int64),
        ("scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("causal_offset", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("dropout_p", ctypes.c_float),
        ("seed", ctypes.c_uint32),
        ("mask", ctypes.c_void_p),
        ("mask_stride_b", ctypes.c_int64),
        ("mask_stride_h", ctypes.c_int64),
        ("mask_stride_q", ctypes.c_int64),
        ("mask_stride_k", ctypes.c_int64),
    ]


class FaDecodeParams(ctypes.Structure):
    """Mirror of ``fa_decode_params``."""

    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("history_len", ctypes.c_int32),
    ]


class FaError(RuntimeError):
    def __init__(self, fn: str, code: int, text: str):
        super().__init__(f"{fn} failed: {text} ({code})")
        self.code = code


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libfa_bwd.so (once); raise if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m flashattention_backward_pass_bwd_amd.build` "
            "(or __graft_entry__.build()). There is no non-HIP fallback.")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(FaBwdParams)
    DP = ctypes.POINTER(FaDecodeParams)
    vp = ctypes.c_void_p
    L.fa_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp]
    L.fa_bwd_lse.argtypes = [P, vp, vp, vp, vp]
    L.fa_bwd_preprocess.argtypes = [P, vp, vp, vp, vp]
    L.fa_bwd_dkdv.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.fa_bwd_dq.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    u64 = ctypes.c_uint64
    L.fa_bwd_ds_workspace_size.argtypes = [P, ctypes.POINTER(u64)]
    L.fa_bwd_dkdv_ds.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, u64, vp]
    L.fa_bwd_dq_ds.argtypes = [P, vp, vp, u64, vp, vp]
    L.fa_bwd_dkdv_dq_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.fa_bwd_decode.argtypes = [DP, vp, vp, vp, vp, vp, vp, vp]
    L.fa_bwd_decode_dkdv.argtypes = [DP, vp, vp, vp, vp, vp, vp, vp]
    L.fa_bwd_decode_max_history.argtypes = [DP]
    L.fa_bwd_decode_max_history.restype = ctypes.c_int32
    L.fa_bwd_status_string.argtypes = [ctypes.c_int]
    L.fa_bwd_status_string.restype = ctypes.c_char_p
    L.fa_bwd_debug_visibility.argtypes = [P, vp, vp]
    L.fa_bwd_debug_dropout_keep.argtypes = [P, vp, vp]
    L.fa_bwd_calib_mfma_bf16.argtypes = [vp, vp, ctypes.c_int32, ctypes.c_int32, vp]
    for name in ("fa_fwd", "fa_bwd_lse", "fa_bwd_preprocess", "fa_bwd_dkdv", "fa_bwd_dq", "fa_bwd_ds_workspace_size",
                 "fa_bwd_dkdv_ds", "fa_bwd_dq_ds", "fa_bwd_dkdv_dq_noalloc", "fa_bwd_decode", "fa_bwd_decode_dkdv",
                 "fa_bwd_debug_visibility", "fa_bwd_debug_dropout_keep", "fa_bwd_calib_mfma_bf16"):
        getattr(L, name).restype = ctypes.c_int
    _LIB = L
    return L


def status_string(code: int) -> str:
    return lib().fa_bwd_status_string(code).decode()


def check(fn: str, code: int) -> None:
    if code != FA_OK:
        raise FaError(fn, code, status_string(code))
