"""FlashAttention backward pass for AMD MI355X (gfx950).

The compute lives in ``libfa_bwd.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/fa_bwd.h``); this package is a thin ctypes binding that
marshals torch tensors (device memory and streams only) into those calls.
Importing the package does not load the library; the first call does, and it
raises if the library has not been built -- there is no fallback path.
"""
