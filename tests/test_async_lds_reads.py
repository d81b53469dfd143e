"""Static check of the inline-asm transposed LDS reads.

Those reads (ds_read_b64_tr_b16 issued from inline asm, so that they need not
wait for the direct-to-LDS loads filling the other buffer) are invisible to the
compiler's wait-count pass.  Their destination registers are only valid after
an explicit lgkmcnt wait that covers them; any instruction that reads or
overwrites such a register earlier would see stale data.  This compiles the kernel source to
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


def _lgkm(t):
    m = re.search(r"lgkmcnt\((\d+)\)", t)
    return int(m.group(1)) if m else None


def scan(asm_text):
    """(number of async reads, list of violations) for one assembly listing.

    The state is the wave's queue of outstanding LDS operations in issue order
    (async reads carry their destination registers; every other ds_*
    instruction is an anonymous entry).  LDS operations complete in order, so
    s_waitcnt lgkmcnt(N) leaves only the N most recent ones outstanding.  A
    forward branch hands its state to its target label, where the states of
    all incoming paths are kept side by side; a backward branch (a loop edge)
    must not carry an async read."""
    labels = {}
    lines = asm_text.split("\n")
    for ln, line in enumerate(lines):
        t = line.strip()
        if t.endswith(":") and not t.startswith(";"):
            labels[t[:-1]] = ln
    saved = {}         # label -> list of alternative states
    alts = [()]        # alternative states reaching this point (tuples of entries)
    bad, n, in_asm = [], 0, False

    def pending(states):
        return {r: e[1] for st in states for e in st if e[0] for r in e[2]}

    for ln, line in enumerate(lines):
        t = line.split(";")[0].strip() if not line.strip().startswith(";;#ASM") else line.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not t or (t.startswith(".") and not t.endswith(":")):
            continue
        if t.endswith(":"):
            alts = list(dict.fromkeys(list(alts) + saved.pop(t[:-1], [])))
            continue
        parts = t.replace(",", " ").split()
        op = parts[0]
        if op.startswith("s_branch") or op.startswith("s_cbranch"):
            target = parts[1] if len(parts) > 1 else ""
            if target in labels and labels[target] > ln:
                saved.setdefault(target, [])
                saved[target] = list(dict.fromkeys(saved[target] + list(alts)))
            elif pending(alts):
                bad.append("line %d: backward branch with async reads pending (%s)"
                           % (ln, sorted(pending(alts))[:4]))
            if op.startswith("s_branch"):
                alts = []  # no fall-through
            continue
        if op in ("s_endpgm", "s_setpc_b64"):
            alts = [()]
            continue
        if op == "s_waitcnt":
            k = _lgkm(t)
            if k is not None:
                alts = list(dict.fromkeys(st[len(st) - k:] if k > 0 else () for st in alts))
                alts = [st if k > 0 else () for st in alts]
            continue
        pend = pending(alts)
        operands = parts[1:]
        if op.startswith("ds_") and in_asm and op == "ds_read_b64_tr_b16":
            regs = tuple(_regs(operands[0]))
            for r in _regs(operands[1]) if len(operands) > 1 else []:
                if r in pend:
                    bad.append("line %d uses %s before its read (line %d) returned: %s" % (ln, r, pend[r], t))
            n += 1
            alts = [st + ((True, ln, regs),) for st in alts]
            continue
        for opnd in operands:
            for r in _regs(opnd):
                if r in pend:
                    bad.append("line %d uses %s before its read (line %d) returned: %s" % (ln, r, pend[r], t))
        if op.startswith("ds_"):
            alts = [st + ((False, ln, ()),) for st in alts]
    return n, bad


def _compile(tmp_path, src):
    out = tmp_path / (src + ".s")
    cmd = ([B._hipcc()] + B.HIPCC_FLAGS + B.SOURCE_FLAGS.get(src, []) +
           ["--cuda-device-only", "-S", "-x", "hip", os.path.join(B.CSRC, src), "-o", str(out)])
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


@pytest.mark.parametrize("src", ["moda_bwd.hip"])
def test_no_use_before_wait(tmp_path, src):
    n, bad = scan(_compile(tmp_path, src))
    assert n > 0, "no inline-asm transposed reads found: the check is looking at the wrong code"
    assert not bad, "\n".join(bad[:10])


def test_scanner_flags_a_use_on_a_branch_path():
    # the read is pending on the taken path of the branch, where v4 is used
    text = "\n".join(["kern:", ";;#ASMSTART", "ds_read_b64_tr_b16 v[4:5], v1", ";;#ASMEND",
                      "s_cbranch_scc1 .LBB0_2", "s_waitcnt lgkmcnt(0)", ".LBB0_2:", "v_mov_b32 v10, v4"])
    n, bad = scan(text)
    assert n == 1 and len(bad) == 1 and "v4" in bad[0]


def test_scanner_accepts_a_branch_that_leaves_the_registers_alone():
    text = "\n".join(["kern:", ";;#ASMSTART", "ds_read_b64_tr_b16 v[4:5], v1", ";;#ASMEND",
                      "s_cbranch_scc1 .LBB0_2", "v_mov_b32 v10, v7", ".LBB0_2:", "s_waitcnt lgkmcnt(0)",
                      "v_mov_b32 v10, v4"])
    n, bad = scan(text)
    assert n == 1 and not bad


def test_scanner_flags_a_read_pending_on_a_loop_edge():
    text = "\n".join(["kern:", ".LBB0_1:", ";;#ASMSTART", "ds_read_b64_tr_b16 v[4:5], v1", ";;#ASMEND",
                      "s_cbranch_scc1 .LBB0_1", "s_waitcnt lgkmcnt(0)"])
    n, bad = scan(text)
    assert n == 1 and len(bad) == 1 and "backward" in bad[0]


def test_scanner_flags_an_early_use():
    text = "\n".join([
        "kern:", ";;#ASMSTART", "ds_read_b64_tr_b16 v[4:5], v1", ";;#ASMEND",
        "v_mov_b32 v9, v5",
        "s_waitcnt lgkmcnt(0)",
        "v_mov_b32 v10, v4"])
    n, bad = scan(text)
    assert n == 1 and len(bad) == 1 and "v5" in bad[0]


def test_scanner_counts_outstanding_operations():
    # lgkmcnt(1) retires every LDS operation but the newest: the first read's
    # registers are usable, the second read's are not
    text = "\n".join([
        "kern:", ";;#ASMSTART", "ds_read_b64_tr_b16 v[4:5], v1", ";;#ASMEND",
        ";;#ASMSTART", "ds_read_b64_tr_b16 v[6:7], v1", ";;#ASMEND",
        "s_waitcnt lgkmcnt(1)",
        "v_mov_b32 v10, v4",
        "v_mov_b32 v11, v6"])
    n, bad = scan(text)
    assert n == 2 and len(bad) == 1 and "v6" in bad[0]


def test_scanner_counts_compiler_lds_operations():
    # a younger compiler-issued LDS read is one of the N most recent, so
    # lgkmcnt(1) after it already covers the async read
    text = "\n".join([
        "kern:", ";;#ASMSTART", "ds_read_b64_tr_b16 v[4:5], v1", ";;#ASMEND",
        "ds_read_b128 v[8:11], v2",
        "s_waitcnt lgkmcnt(1)",
        "v_mov_b32 v10, v4"])
    n, bad = scan(text)
    assert n == 1 and not bad
