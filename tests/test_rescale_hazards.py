"""Static check of the in-place output rescale's hand-placed wait states.

The rescale multiplies every element of the MFMA output accumulator by one
factor inside inline asm, so that each element keeps its register.  The
compiler's hazard recognizer cannot see into inline asm, so the asm itself
carries the waits: three s_nop 7 before the first multiply (an MFMA may have
written the accumulator just before; the factor comes from a v_exp), and
s_nop 3 after the last multiply (the next MFMA reads the accumulator as its
C operand).  Those waits are only enough when the rescale runs as one block:
an MFMA scheduled between the first and the last multiply could write an
element that a later multiply reads, or read one that an earlier multiply has
just written, with no wait in between; a branch or label inside the block
could enter or leave it past its waits.  This compiles the kernel sources to
gfx950 assembly exactly as the library build does (same flags, same
scheduler) and checks every rescale block for that."""
import os
import re
import shutil
import subprocess

import pytest

from depth_stream_attention_amd import build as B

pytestmark = pytest.mark.skipif(shutil.which(B._hipcc()) is None and not os.path.exists(B._hipcc()),
                                reason="needs hipcc")


def _asm_blocks(lines):
    """Yield (first line index, last line index, instruction lines) of each inline-asm block."""
    start = None
    for ln, line in enumerate(lines):
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            start, body = ln, []
        elif t.startswith(";;#ASMEND") and start is not None:
            yield start, ln, body
            start = None
        elif start is not None and t:
            body.append(t)


def scan(asm_text):
    """(list of (multiplies, accumulator elements) per rescale block, list of violations)."""
    lines = asm_text.split("\n")
    blocks = list(_asm_blocks(lines))
    regions, bad = [], []
    i = 0
    while i < len(blocks):
        s0, _, body = blocks[i]
        if body[:3] == ["s_nop 7"] * 3 and len(body) == 4 and body[3].startswith("v_mul_f32"):
            # find the block that closes the region
            j = i
            while j < len(blocks) and not (len(blocks[j][2]) == 2 and blocks[j][2][0].startswith("v_mul_f32")
                                           and blocks[j][2][1] == "s_nop 3"):
                j += 1
            if j == len(blocks):
                bad.append("line %d: rescale block opened and never closed" % s0)
                break
            e1 = blocks[j][1]
            muls, regs = 0, set()
            for ln in range(s0, e1 + 1):
                t = lines[ln].split(";")[0].strip()
                if not t:
                    continue
                op = t.split()[0]
                if op.startswith("v_mfma") or op.startswith("v_smfmac"):
                    bad.append("line %d: matrix instruction inside the rescale block of line %d: %s" % (ln, s0, t))
                if op.startswith("s_branch") or op.startswith("s_cbranch") or op.startswith("s_setpc"):
                    bad.append("line %d: branch inside the rescale block of line %d: %s" % (ln, s0, t))
                if t.endswith(":"):
                    bad.append("line %d: label inside the rescale block of line %d: %s" % (ln, s0, t))
            for k in range(i, j + 1):
                for ins in blocks[k][2]:
                    m = re.match(r"v_mul_f32 (v\d+), (v\d+), (v\d+)$", ins)
                    if m:
                        muls += 1
                        regs.add(m.group(1))
                        if m.group(1) != m.group(2):
                            bad.append("line %d: rescale multiply not in place: %s" % (blocks[k][0], ins))
            regions.append((muls, len(regs)))
            i = j + 1
        else:
            i += 1
    return regions, bad


def _compile(tmp_path, src):
    out = tmp_path / (src + ".s")
    cmd = ([B._hipcc()] + B.HIPCC_FLAGS + B.SOURCE_FLAGS.get(src, []) +
           ["--cuda-device-only", "-S", "-x", "hip", os.path.join(B.CSRC, src), "-o", str(out)])
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


@pytest.mark.parametrize("src", ["moda_fwd_bf16.hip", "moda_decode.hip"])
def test_rescale_blocks_hold_no_matrix_op_or_branch(tmp_path, src):
    regions, bad = scan(_compile(tmp_path, src))
    assert regions, "no rescale blocks found: the check is looking at the wrong code"
    # one multiply per accumulator element, on distinct registers: 16 * d/32 for d = 64 or 128
    assert all(m == r and m in (32, 64) for m, r in regions), sorted(set(regions))
    assert not bad, "\n".join(bad[:10])


def _region(middle):
    return "\n".join(["kern:", ";;#ASMSTART", "s_nop 7", "s_nop 7", "s_nop 7", "v_mul_f32 v0, v0, v9", ";;#ASMEND"]
                     + middle + [";;#ASMSTART", "v_mul_f32 v1, v1, v9", "s_nop 3", ";;#ASMEND"])


def test_scanner_accepts_a_clean_block():
    regions, bad = scan(_region([";;#ASMSTART", "v_mul_f32 v2, v2, v9", ";;#ASMEND", "v_mul_f32_e32 v20, v9, v20"]))
    assert regions == [(3, 3)] and not bad


def test_scanner_flags_a_matrix_op_inside():
    regions, bad = scan(_region(["v_mfma_f32_32x32x16_bf16 v[0:15], v[40:43], v[44:47], v[0:15]"]))
    assert len(bad) == 1 and "matrix" in bad[0]


def test_scanner_flags_a_branch_or_label_inside():
    regions, bad = scan(_region(["s_cbranch_vccnz .LBB0_3", ".LBB0_3:"]))
    assert len(bad) == 2 and "branch" in bad[0] and "label" in bad[1]
