"""The tile kernels' global->LDS copies write M0 without saving it (fa_tiles.h).

That is only sound while the compiler itself never reads or writes M0 in those
kernels.  This CPU test compiles each source that issues the copies to gfx950
assembly with the library's own flags and checks that M0 appears only inside
inline-assembly blocks.
"""
import concurrent.futures
import os
import re
import subprocess
import tempfile

import pytest

from flashattention_backward_pass_bwd_amd import build

SOURCES = [s for s in build.SOURCES if s.endswith(".hip") and "dma16(" in open(os.path.join(build.CSRC, s)).read()]


def _have_hipcc() -> bool:
    try:
        build._hipcc()
        return True
    except RuntimeError:
        return False


pytestmark = pytest.mark.skipif(not _have_hipcc(), reason="hipcc not available")


def _asm(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, src + ".s")
    cmd = [build._hipcc(), *build.COMMON_FLAGS, *build.EXTRA_FLAGS.get(src, []), "--cuda-device-only", "-x", "hip", "-S", os.path.join(build.CSRC, src), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return open(out).read()


def _m0_outside_inline_asm(text: str):
    bad, inside = [], False
    for line in text.splitlines():
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            inside = True
        elif s.startswith(";;#ASMEND"):
            inside = False
        elif not inside and re.search(r"\bm0\b", s.split(";")[0]):
            bad.append(s.split(";")[0].strip())
    return bad


def test_copy_sources_found():
    assert {"fa_dkdv_bf16.hip", "fa_dq_bf16.hip"} <= set(SOURCES)


def test_compiler_leaves_m0_to_the_copies():
    with tempfile.TemporaryDirectory() as d:
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            texts = dict(zip(SOURCES, ex.map(lambda s: _asm(s, d), SOURCES)))
    for src, text in texts.items():
        assert "global_load_lds_dwordx4" in text, src
        assert _m0_outside_inline_asm(text) == [], src


def test_detector_flags_compiler_m0_use():
    text = "\n".join([
        ";;#ASMSTART", "\ts_mov_b32 m0, s4", ";;#ASMEND",   # the copies' own write: allowed
        "\ts_mov_b32 m0, -1",                                  # a compiler write: flagged
        "\tv_movrels_b32 v0, v1 ; uses m0",                    # comment text is ignored
    ])
    assert _m0_outside_inline_asm(text) == ["s_mov_b32 m0, -1"]
