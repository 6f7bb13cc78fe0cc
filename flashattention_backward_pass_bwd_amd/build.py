"""Build libfa_bwd.so in-tree with hipcc for gfx950.

Usage: ``python -m flashattention_backward_pass_bwd_amd.build`` (or call
``build()``).  Every call recompiles: one object per source file in parallel
under ``_build/``, then one shared library next to this file.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libfa_bwd.so")

SOURCES = [
    "fa_preprocess.hip",
    "fa_dkdv.hip",
    "fa_dkdv_bf16.hip",
    "fa_dq.hip",
    "fa_dq_bf16.hip",
    "fa_dq2_bf16.hip",
    "fa_dqs_bf16.hip",
    "fa_fwd_bf16.hip",
    "fa_fwd.hip",
    "fa_decode.hip",
    "fa_decode_kv.hip",
    "fa_debug.hip",
    "fa_noalloc.hip",
    "fa_api.cpp",
]

ARCH = "gfx950"

# Per-file extra flags.  The bf16 tile kernels fix their own instruction order
# with scheduling fences and issue their MFMAs as inline assembly, so the
# compiler's scheduling strategy and MFMA register form do not shape them; but
# every slot loop must unroll completely (register arrays indexed by a runtime
# slot number become select chains and spills).  The 64-row dQ kernel's slot
# loop is larger than the default size limit of a requested full unroll.
EXTRA_FLAGS: dict = {
    "fa_dq2_bf16.hip": ["-mllvm", "-pragma-unroll-threshold=100000"],
}

COMMON_FLAGS = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    f"--offload-arch={ARCH}",
    # Packed fp32 VALU instructions are kept out of generated code on purpose.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; a ROCm toolchain is required to build libfa_bwd.so")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [_hipcc(), *COMMON_FLAGS, *EXTRA_FLAGS.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source and link ``libfa_bwd.so``; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
