"""Static check of the inline-asm direct-to-LDS tile loads.

The forward, the backward's dq pass and the decode partials issue their tile
loads (buffer_load_dwordx4 ... lds) as inline asm, so that the compiler does
not make the transposed LDS reads of the current tile wait for the next tile's
load.  The compiler therefore does not know those loads exist: nothing but the
kernel's own code makes a tile visible before it is read, and the M0 write
that sets each load's LDS address needs its wait state from the asm itself.
This compiles the sources to gfx950 assembly as the library build does and
checks, in every kernel that issues such loads:
  - each one is preceded inside its asm block by s_nop (M0 -> LDS-DMA hazard);
  - no VALU instruction writes one of its descriptor SGPRs fewer than 5 wait
    states before it (a vector memory instruction reads an SGPR correctly only
    5 wait states after a VALU write; under SGPR pressure the compiler reloads
    descriptors from VGPR lanes with v_readlane just before the statement, and
    a stale descriptor dword sends the load to a wrong address).  A branch
    target or the kernel start inside that window counts as a violation.  The
    check is asm_check's, which the build also runs on every kernel before it
    links the library;
  - each s_barrier follows an s_waitcnt with vmcnt(0), with no vector memory
    instruction and no branch target in between (the tile pipeline's publish
    step: all of the wave's loads have landed before the barrier)."""
import os
import shutil
import subprocess

import pytest

from depth_stream_attention_amd import build as B
from depth_stream_attention_amd.asm_check import functions, sgpr_hazards

pytestmark = pytest.mark.skipif(shutil.which(B._hipcc()) is None and not os.path.exists(B._hipcc()),
                                reason="needs hipcc")


def scan(lines):
    """(asm LDS loads found, violations) for one kernel's lines."""
    n, bad = 0, []
    in_asm, asm_block = False, []
    clear = False  # an s_waitcnt vmcnt(0) with no vector memory operation or label since
    for ln, line in enumerate(lines):
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm, asm_block = True, []
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        t = t.split(";")[0].strip()
        if t.endswith(":"):
            clear = False  # paths merge here
            continue
        if not t or t.startswith("."):
            continue
        op = t.split()[0]
        if in_asm:
            if op.startswith("buffer_load") and t.endswith(" lds"):
                n += 1
                if not any(x.startswith("s_nop") for x in asm_block):
                    bad.append("line %d: LDS load without a preceding s_nop in its asm block: %s" % (ln, t))
            asm_block.append(op)
        if op == "s_waitcnt" and "vmcnt(0)" in t:
            clear = True
        elif op.startswith(("buffer_", "global_", "flat_", "scratch_")):
            clear = False
        elif op == "s_barrier" and not clear:
            bad.append("line %d: s_barrier without a preceding s_waitcnt vmcnt(0)" % ln)
    return n, bad


def _compile(tmp_path, src):
    out = tmp_path / (src + ".s")
    cmd = ([B._hipcc()] + B.HIPCC_FLAGS + B.SOURCE_FLAGS.get(src, []) +
           ["--cuda-device-only", "-S", "-x", "hip", os.path.join(B.CSRC, src), "-o", str(out)])
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


@pytest.mark.parametrize("src,kernel", [("moda_fwd_bf16.hip", "moda_fwd_bf16_kernel"),
                                        ("moda_bwd.hip", "moda_bwd_dq_kernel"),
                                        ("moda_decode.hip", "moda_decode_partial_kernel")])
def test_asm_lds_loads_are_published(tmp_path, src, kernel):
    funcs = {k: v for k, v in functions(_compile(tmp_path, src)).items() if kernel in k}
    assert funcs, "no %s in %s" % (kernel, src)
    for name, lines in funcs.items():
        n, bad = scan(lines)
        assert n > 0, "%s: no inline-asm LDS loads found: the check is looking at the wrong code" % name
        bad += sgpr_hazards(lines)
        assert not bad, name + "\n" + "\n".join(bad[:10])


def test_scanner_flags_a_missing_nop():
    lines = [";;#ASMSTART", "buffer_load_dwordx4 v1, s[4:7], 0 offen lds", ";;#ASMEND",
             "s_waitcnt vmcnt(0)", "s_barrier"]
    n, bad = scan(lines)
    assert n == 1 and len(bad) == 1 and "s_nop" in bad[0]


def test_scanner_flags_a_barrier_without_the_wait():
    lines = [";;#ASMSTART", "s_nop 0", "buffer_load_dwordx4 v1, s[4:7], 0 offen lds", ";;#ASMEND",
             "s_waitcnt lgkmcnt(0)", "s_barrier"]
    n, bad = scan(lines)
    assert n == 1 and len(bad) == 1 and "vmcnt(0)" in bad[0]


def test_scanner_flags_a_load_between_the_wait_and_the_barrier():
    lines = [";;#ASMSTART", "s_nop 0", "buffer_load_dwordx4 v1, s[4:7], 0 offen lds", ";;#ASMEND",
             "s_waitcnt vmcnt(0)", "global_load_dword v2, v[4:5], off", "s_barrier"]
    n, bad = scan(lines)
    assert n == 1 and len(bad) == 1 and "vmcnt(0)" in bad[0]


def test_scanner_flags_a_label_between_the_wait_and_the_barrier():
    lines = ["s_waitcnt vmcnt(0)", ".LBB0_3:", "s_barrier"]
    n, bad = scan(lines)
    assert n == 0 and len(bad) == 1


def test_scanner_accepts_the_publish_pattern():
    lines = [";;#ASMSTART", "s_nop 0", "buffer_load_dwordx4 v1, s[4:7], 0 offen lds", ";;#ASMEND",
             "v_add_u32_e32 v2, v3, v4", "s_waitcnt vmcnt(0) lgkmcnt(0)", "; a comment",
             "v_writelane_b32 v159, s1, 43", "s_barrier"]
    n, bad = scan(lines)
    assert n == 1 and not bad


def test_functions_splits_kernels():
    text = "\n".join(["_Z1av:", "s_nop 0", "s_endpgm", "_Z1bv:  ; comment", "s_barrier", "s_endpgm"])
    f = functions(text)
    assert list(f) == ["_Z1av", "_Z1bv"] and f["_Z1bv"][0] == "s_barrier"


def test_hazard_check_flags_a_descriptor_read_too_soon():
    lines = ["v_readlane_b32 s27, v223, 41", "v_cndmask_b32_e32 v72, v69, v72, vcc", "s_mov_b32 m0, s50",
             ";;#ASMSTART", "s_nop 0", "buffer_load_dwordx4 v72, s[24:27], 0 offen lds", ";;#ASMEND"]
    bad = sgpr_hazards(lines)
    assert len(bad) == 1 and "v_readlane_b32 s27" in bad[0] and "3 wait states" in bad[0]


def test_hazard_check_accepts_five_wait_states():
    lines = ["v_readlane_b32 s27, v223, 41", "s_mov_b32 m0, s50",
             ";;#ASMSTART", "s_nop 4", "buffer_load_dwordx4 v72, s[24:27], 0 offen lds", ";;#ASMEND"]
    assert sgpr_hazards(lines) == []


def test_hazard_check_ignores_other_sgprs_and_flags_labels():
    ok = ["s_nop 4", "v_readlane_b32 s30, v1, 0", "s_nop 0", "buffer_load_dwordx4 v2, s[24:27], 0 offen lds"]
    assert sgpr_hazards(ok) == []
    assert len(sgpr_hazards([".LBB0_1:", "s_nop 0", "buffer_load_dwordx4 v2, s[4:7], 0 offen lds"])) == 1


def test_hazard_check_sees_scalar_carry_outputs():
    lines = ["v_add_co_u32_e64 v1, s[26:27], v2, v3", "s_nop 0",
             "buffer_load_dwordx4 v2, s[24:27], 0 offen lds"]
    bad = sgpr_hazards(lines)
    assert len(bad) == 1 and "v_add_co_u32_e64" in bad[0]
