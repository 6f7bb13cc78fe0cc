"""CPU fp64 oracle for the FlashAttention backward pass -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct definition that the HIP
kernels are checked against.  It is not part of the product: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It imports nothing from the HIP package and the HIP package never
imports it; the two share only the seeded input generators, which hold none of
the method's arithmetic.

Pages the definitions come from (cited by page title and section):

* rustytorch, ``flash_attention_backward_dq.metal`` -- Metal dQ kernel
  (header comment and kernel body).
* ferrotensor-backend 0.2.0, ``flash_attention_v2_backward.wgsl`` -- WebGPU
  two-pass FA-v2 backward (header comment, ``fab2_visible``,
  ``fab2_mask_at``, ``flash_bwd_dq``, ``flash_bwd_dk_dv``).
* rullama 0.2.0, ``attention_backward_dq.wgsl`` -- WebGPU decode-step
  backward, pass 1 (header comment, phases A-C).

Parity status: every function here is pinned by a ``-m "not gpu"`` test
(finite differences, brute-force softmax Jacobians, invariants, a torch fp64
autograd cross-check, closed forms, published MurmurHash3 vectors).  Nothing is
"parity unpinned" except the choice of dropout hash composition itself, which
the pages leave undefined (see ``attention.dropout_keep``); its fmix32 core is
pinned against published vectors and its output statistics are tested.
"""

from .attention import (  # noqa: F401
    MASKED,
    Spec,
    fmix32,
    dropout_threshold,
    dropout_draw,
    dropout_keep,
    dropout_multiplier,
    visible,
    counted,
    forward,
    forward_rows,
    backward,
    backward_block,
    backward_dq_rows,
    backward_dkdv_keys,
    decode_probs,
    decode_backward,
    decode_dkdv,
)
