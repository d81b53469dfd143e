"""Static check of the backward's inline-asm transposed LDS reads.

Those reads (ds_read_b64_tr_b16 issued from inline asm, so that they need not
wait for the direct-to-LDS loads filling the other buffer) are invisible to the
compiler's wait-count pass.  Their destination registers are only valid after
an explicit lgkmcnt(0) wait; any instruction that reads or overwrites such a
register earlier would see stale data.  This compiles the kernel source to
gfx950 assembly exactly as the library build does and scans it for that."""
import os
import re
import shutil
import subprocess

import pytest

from depth_stream_attention_amd import build as B

pytestmark = pytest.mark.skipif(shutil.which(B._hipcc()) is None and not os.path.exists(B._hipcc()),
                                reason="needs hipcc")


def _regs(op):
    m = re.match(r"([va])\[(\d+):(\d+)\]", op)
    if m:
        return ["%s%d" % (m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)]
    return [op] if re.match(r"[va]\d+$", op) else []


def scan(asm_text):
    """(number of async reads, list of violations) for one assembly listing."""
    pending, bad, n, in_asm = {}, [], 0, False
    for ln, line in enumerate(asm_text.split("\n")):
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not t or t.startswith(";") or (t.startswith(".") and not t.endswith(":")):
            continue
        if t.endswith(":"):
            # A label: control may arrive from elsewhere.  Every async read must
            # have been waited for within its own basic block.
            if pending and t.startswith("."):
                bad.append("line %d: label %s reached with async reads pending (%s)" % (ln, t, sorted(pending)[:4]))
            pending.clear()
            continue
        parts = t.replace(",", " ").split()
        if parts[0].startswith("s_branch") or parts[0].startswith("s_cbranch"):
            if pending:
                bad.append("line %d: branch with async reads pending (%s)" % (ln, sorted(pending)[:4]))
            pending.clear()
            continue
        if in_asm and parts[0] == "ds_read_b64_tr_b16":
            n += 1
            for r in _regs(parts[1]):
                pending[r] = ln
            continue
        if parts[0] == "s_waitcnt" and "lgkmcnt(0)" in t:
            pending.clear()
            continue
        if parts[0] in ("s_endpgm", "s_setpc_b64"):
            pending.clear()
            continue
        for opnd in parts[1:]:
            for r in _regs(opnd):
                if r in pending:
                    bad.append("line %d uses %s before its read (line %d) returned: %s" % (ln, r, pending[r], t))
    return n, bad


def test_no_use_before_wait(tmp_path):
    out = tmp_path / "moda_bwd.s"
    cmd = ([B._hipcc()] + B.HIPCC_FLAGS + B.SOURCE_FLAGS.get("moda_bwd.hip", []) +
           ["--cuda-device-only", "-S", "-x", "hip", os.path.join(B.CSRC, "moda_bwd.hip"), "-o", str(out)])
    subprocess.run(cmd, check=True, capture_output=True)
    n, bad = scan(out.read_text())
    assert n > 0, "no inline-asm transposed reads found: the check is looking at the wrong code"
    assert not bad, "\n".join(bad[:10])


def test_scanner_flags_pending_reads_across_control_flow():
    text = "\n".join(["kern:", ";;#ASMSTART", "ds_read_b64_tr_b16 v[4:5], v1", ";;#ASMEND",
                      "s_cbranch_scc1 .LBB0_2", "s_waitcnt lgkmcnt(0)", ".LBB0_2:", "v_mov_b32 v10, v4"])
    n, bad = scan(text)
    assert n == 1 and len(bad) == 1 and "branch" in bad[0]


def test_scanner_flags_an_early_use():
    text = "\n".join([
        "kern:", ";;#ASMSTART", "ds_read_b64_tr_b16 v[4:5], v1", ";;#ASMEND",
        "v_mov_b32 v9, v5",
        "s_waitcnt lgkmcnt(0)",
        "v_mov_b32 v10, v4"])
    n, bad = scan(text)
    assert n == 1 and len(bad) == 1 and "v5" in bad[0]
