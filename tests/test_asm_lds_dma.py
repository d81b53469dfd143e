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
  - each s_barrier follows an s_waitcnt with vmcnt(0), with no vector memory
    instruction and no branch target in between (the tile pipeline's publish
    step: all of the wave's loads have landed before the barrier)."""
import os
import re
import shutil
import subprocess

import pytest

from depth_stream_attention_amd import build as B

pytestmark = pytest.mark.skipif(shutil.which(B._hipcc()) is None and not os.path.exists(B._hipcc()),
                                reason="needs hipcc")

_FUNC = re.compile(r"^(_Z\S+):")


def functions(asm_text):
    """{name: [lines]} of the kernels in one assembly listing."""
    out, cur = {}, None
    for line in asm_text.split("\n"):
        m = _FUNC.match(line)
        if m:
            cur = m.group(1)
            out[cur] = []
        elif cur is not None:
            out[cur].append(line)
            if line.strip().startswith("s_endpgm"):
                cur = None
    return out


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
