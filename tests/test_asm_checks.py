"""Checks on the generated gfx950 assembly of the tile kernels (CPU only).

* The global->LDS copies write M0 without saving it (fa_tiles.h).  That is
  only sound while the compiler itself never reads or writes M0 in those
  kernels: M0 may appear only inside inline-assembly blocks.
* The MFMAs are inline assembly, so the compiler's hazard tracking does not
  see them.  Two hazards it would otherwise resolve are checked here:
  a register written by an instruction outside the asm and read as an MFMA
  operand within the two instructions before it (two wait states are needed),
  and a register that an MFMA reads as its accumulator input (other than its
  own result) written within the ten instructions after it, while the MFMA
  may still read it.
  A third: a VGPR result of an MFMA read or written by any instruction other
  than the next MFMA of its own chain within the twelve wait states an XDL
  result needs (the count the compiler itself inserts for
  v_mfma_f32_32x32x16_bf16 on gfx950).
* A VMEM store of more than 8 bytes reads its data registers after issue;
  a write to them by the next instruction (one wait state is needed) would
  change the stored data.  Checked for the inline-assembly stores.
* The tile kernels use no scratch memory (no VGPR spills; SGPRs spill only
  into VGPR lanes): a spill in their software pipelines means a slot loop did
  not unroll or the register plan broke.
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


_TEXTS = {}


def _compiled():
    if not _TEXTS:
        with tempfile.TemporaryDirectory() as d:
            with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
                _TEXTS.update(zip(SOURCES, ex.map(lambda s: _asm(s, d), SOURCES)))
    return _TEXTS


def _regs(txt):
    out = set()
    for m in re.finditer(r"\b([va])(\d+)\b|\b([va])\[(\d+):(\d+)\]", txt):
        if m.group(1):
            out.add((m.group(1), int(m.group(2))))
        else:
            out.update((m.group(3), r) for r in range(int(m.group(4)), int(m.group(5)) + 1))
    return out


def _instructions(text):
    """(text, inside inline asm) for every instruction, per kernel."""
    seq, inside = [], False
    for line in text.splitlines():
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            inside = True
        elif s.startswith(";;#ASMEND"):
            inside = False
        elif s and not s.startswith((";", ".")) and not s.endswith(":"):
            seq.append((s.split(";")[0].strip(), inside))
        elif re.match(r"^_Z\w+:", line):
            seq.append(("<kernel>", False))
    return seq


def _writes(ins):
    op = ins.split()[0]
    if op.startswith(("s_", "global_load_lds", "buffer_", "global_store", "ds_write")):
        return set()
    return _regs(ins[len(op):].split(",")[0])


def _mfma_hazards(text):
    bad = []
    seq = _instructions(text)
    for i, (ins, inside) in enumerate(seq):
        op = ins.split()[0]
        if not (inside and op.startswith("v_mfma")):
            continue
        parts = [p.strip() for p in ins[len(op):].split(",")]
        srcs = _regs(",".join(parts[1:]))
        ws = 0
        for j in range(i - 1, -1, -1):  # writes just before
            pins, pin = seq[j]
            if pins == "<kernel>":
                break
            pop = pins.split()[0]
            if pop == "s_nop":
                ws += int(pins.split()[1], 0) + 1
            else:
                if not pin and _writes(pins) & srcs:
                    bad.append(f"{pins} -> {ins}")
                ws += 1
            if ws >= 2:
                break
        if len(parts) >= 4:  # accumulator input that is not the result
            vd, sc = _regs(parts[0]), _regs(parts[3])
            if sc and sc != vd:
                for nins, nin in seq[i + 1:i + 11]:
                    if nins == "<kernel>":
                        break
                    if not (nin and nins.startswith("v_mfma")) and _writes(nins) & sc:
                        bad.append(f"{ins} -> {nins}")
                        break
    return bad


def _result_reads(text, need=12):
    bad = []
    seq = _instructions(text)
    for i, (ins, inside) in enumerate(seq):
        op = ins.split()[0]
        if not (inside and op.startswith("v_mfma")):
            continue
        vd = _regs(ins[len(op):].split(",")[0])
        if not vd or next(iter(vd))[0] != "v":
            continue
        ws = 0
        for nins, _ in seq[i + 1:]:
            if nins == "<kernel>" or ws >= need:
                break
            nop = nins.split()[0]
            if nop == "s_nop":
                ws += int(nins.split()[1], 0) + 1
                continue
            if nop.startswith("v_mfma"):
                nparts = [p.strip() for p in nins[len(nop):].split(",")]
                if _regs(nparts[0]) == vd and len(nparts) >= 4 and _regs(nparts[3]) == vd:
                    break  # the chain's next MFMA (the hardware forwards the result)
            if _regs(nins[len(nop):]) & vd:
                bad.append(f"{ins} -> {nins} ({ws} wait states)")
                break
            ws += 1
    return bad


def test_sources_assemble():
    # The checks below read the compiler's assembly text (-S), which is emitted
    # even when an inline-asm operand is invalid; assembling catches that.
    def obj(src):
        with tempfile.TemporaryDirectory() as d:
            cmd = [build._hipcc(), *build.COMMON_FLAGS, *build.EXTRA_FLAGS.get(src, []), "--cuda-device-only", "-x", "hip",
                   "-c", os.path.join(build.CSRC, src), "-o", os.path.join(d, src + ".o")]
            return src, subprocess.run(cmd, capture_output=True, text=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        for src, res in ex.map(obj, SOURCES):
            assert res.returncode == 0, (src, res.stderr[-2000:])


def test_copy_sources_found():
    assert {"fa_dkdv_bf16.hip", "fa_dq_bf16.hip"} <= set(SOURCES)


def test_compiler_leaves_m0_to_the_copies():
    for src, text in _compiled().items():
        assert "global_load_lds_dwordx4" in text, src
        assert _m0_outside_inline_asm(text) == [], src


def test_detector_flags_compiler_m0_use():
    text = "\n".join([
        ";;#ASMSTART", "\ts_mov_b32 m0, s4", ";;#ASMEND",   # the copies' own write: allowed
        "\ts_mov_b32 m0, -1",                                  # a compiler write: flagged
        "\tv_movrels_b32 v0, v1 ; uses m0",                    # comment text is ignored
    ])
    assert _m0_outside_inline_asm(text) == ["s_mov_b32 m0, -1"]


_SREG = re.compile(r"^(s\[(\d+):(\d+)\]|s(\d+)|vcc)$")


def _sregs(op):
    m = _SREG.match(op.strip())
    if not m:
        return set()
    if m.group(1) == "vcc":
        return {"vcc"}
    if m.group(2):
        return {f"s{r}" for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    return {f"s{m.group(4)}"}


def _vmem_sgpr_hazards(text):
    """VMEM instructions (global_, buffer_, flat_, scratch_) reading an SGPR that a
    VALU instruction (v_readfirstlane, a compare or carry-out into SGPRs) wrote
    fewer than five wait states earlier.  gfx9 needs those five; the compiler
    inserts them for its own instructions, but not in front of an inline-asm
    statement whose SGPR input it just produced with VALU.  Straight-line code
    (a label does not reset the count, which only undercounts across loop
    back edges)."""
    bad, since = [], {}
    for line in text.splitlines():
        s = line.split(";")[0].strip()
        if re.match(r"^_Z\w*:", s):
            since = {}
            continue
        if not s or s.startswith(".") or s.endswith(":"):
            continue
        mn, _, rest = s.partition(" ")
        ops = [o.strip() for o in re.split(r",\s*", rest)] if rest else []
        if re.match(r"^(global|buffer|flat|scratch)_", mn):
            near = sorted(r for o in ops for r in _sregs(o.split(" ")[0]) if since.get(r, 99) < 5)
            if near:
                bad.append(f"{s}  ({', '.join(near)} written by VALU {min(since[r] for r in near)} wait states before)")
        m = re.match(r"^s_nop\s+(\d+)$", s)
        step = int(m.group(1)) + 1 if m else 1
        for r in since:
            since[r] += step
        if mn.startswith("v_") and ops:
            written = _sregs(ops[0])
            if len(ops) > 1 and re.search(r"_co_|div_scale|mad_u64_u32|mad_i64_i32", mn):
                written |= _sregs(ops[1])
            for r in written:
                since[r] = 0
    return bad


def test_vmem_sgpr_operands_after_valu_writes():
    for src, text in _compiled().items():
        assert _vmem_sgpr_hazards(text) == [], src


def test_vmem_sgpr_detector_flags_plain_cases():
    text = "\n".join([
        "_ZN2fa1kEv:",
        "\tv_readfirstlane_b32 s59, v151",
        "\tv_readfirstlane_b32 s58, v150",
        ";;#ASMSTART", "\tglobal_store_dwordx4 v160, v[4:7], s[58:59] nt", ";;#ASMEND",     # flagged
        "\tv_readfirstlane_b32 s4, v1",
        ";;#ASMSTART", "\ts_mov_b32 m0, s4", "\ts_nop 4", "\tglobal_load_lds_dwordx4 v3, s[4:5]", ";;#ASMEND",
        "\tv_cmp_gt_i32_e64 s[6:7], v1, v2",
        "\tbuffer_load_dword v1, v2, s[8:11], 0 offen",                                    # other SGPRs: fine
        "\tglobal_load_dword v1, v2, s[6:7]",                                             # flagged
    ])
    bad = _vmem_sgpr_hazards(text)
    assert len(bad) == 2 and "s[58:59]" in bad[0] and "s[6:7]" in bad[1], bad


def test_no_write_hazards_around_asm_mfmas():
    for src, text in _compiled().items():
        assert "v_mfma_f32_32x32x16_bf16" in text, src
        assert _mfma_hazards(text) == [], src


def test_hazard_detector_flags_plain_cases():
    text = "\n".join([
        "_ZN2fa1kEv:",
        "\tv_mov_b32_e32 v4, 0",                                    # writes an A operand register ...
        ";;#ASMSTART", "\tv_mfma_f32_32x32x16_bf16 v[16:31], v[4:7], a[0:3], v[32:47]", ";;#ASMEND",
        "\tv_add_u32_e32 v40, 1, v0",                              # ... and the accumulator input after
        ";;#ASMSTART", "\ts_nop 1", "\tv_mfma_f32_32x32x16_bf16 v[48:63], v[8:11], a[4:7], 0", ";;#ASMEND",
    ])
    assert len(_mfma_hazards(text)) == 2


def test_mfma_results_read_after_their_wait_states():
    for src, text in _compiled().items():
        assert _result_reads(text) == [], src


def test_result_read_detector_flags_plain_cases():
    text = "\n".join([
        "_ZN2fa1kEv:",
        ";;#ASMSTART", "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], a[0:3], 0", ";;#ASMEND",
        ";;#ASMSTART", "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], a[4:7], v[0:15]", ";;#ASMEND",  # chain: fine
        ";;#ASMSTART", "\ts_nop 7", ";;#ASMEND",
        "\tv_exp_f32_e32 v30, v3",                                                                  # 8 wait states: flagged
        ";;#ASMSTART", "\tv_mfma_f32_32x32x16_bf16 v[32:47], v[16:19], a[0:3], 0", ";;#ASMEND",
        ";;#ASMSTART", "\ts_nop 7", "\ts_nop 3", ";;#ASMEND",
        "\tv_exp_f32_e32 v50, v40",                                                                 # 13 wait states: fine
    ])
    bad = _result_reads(text)
    assert len(bad) == 1 and "v_exp_f32_e32 v30, v3" in bad[0]


def test_tile_kernels_use_no_scratch():
    for src, text in _compiled().items():
        spills = [int(m) for m in re.findall(r"\.vgpr_spill_count:\s+(\d+)", text)]
        scratch = [int(m) for m in re.findall(r"; ScratchSize:\s+(\d+)", text)]
        assert spills and max(spills) == 0, (src, "vgpr spills", spills)
        assert scratch and max(scratch) == 0, (src, "scratch bytes", scratch)


_WIDE_STORE = re.compile(r"^(global|flat|buffer|scratch)_store_dwordx[34]\b")


def _store_data_hazards(text):
    """Instructions that write a wide inline-asm store's data registers in the
    wait state right after it."""
    bad = []
    seq = _instructions(text)
    for i, (ins, inside) in enumerate(seq):
        op = ins.split()[0]
        if not (inside and _WIDE_STORE.match(op)):
            continue
        ops = [o.strip() for o in ins[len(op):].split(",")]
        data = _regs(ops[0] if op.startswith("buffer_") else ops[1])
        for nins, _ in seq[i + 1:i + 2]:
            if nins == "<kernel>" or nins.split()[0] == "s_nop":
                break
            w = _regs(nins[len(nins.split()[0]):].split(",")[0]) if not nins.startswith(("s_", "ds_write", "global_store", "buffer_store")) else set()
            if w & data:
                bad.append(f"{ins} -> {nins}")
    return bad


def test_wide_asm_stores_keep_their_data_for_a_wait_state():
    found = 0
    for src, text in _compiled().items():
        found += len([1 for ins, inside in _instructions(text) if inside and _WIDE_STORE.match(ins.split()[0])])
        assert _store_data_hazards(text) == [], src
    assert found > 0


def test_store_data_detector_flags_plain_cases():
    text = "\n".join([
        "_ZN2fa1kEv:",
        ";;#ASMSTART", "\tglobal_store_dwordx4 v160, v[4:7], s[58:59] nt", ";;#ASMEND",
        "\tv_cvt_pk_bf16_f32 v5, v1, v2",                          # flagged: writes store data at once
        ";;#ASMSTART", "\tglobal_store_dwordx4 v160, v[8:11], s[58:59] nt", "\ts_nop 1", ";;#ASMEND",
        "\tv_cvt_pk_bf16_f32 v9, v1, v2",                          # fine: wait states in between
        ";;#ASMSTART", "\tglobal_store_dwordx4 v160, v[12:15], s[58:59] nt", ";;#ASMEND",
        "\tv_cvt_pk_bf16_f32 v20, v1, v2",                         # fine: other registers
    ])
    bad = _store_data_hazards(text)
    assert len(bad) == 1 and "v5" in bad[0], bad
