"""Checks of the compiled gfx950 assembly that the compiler cannot make itself.

The tile loads of the forward, the backward's dq pass and the decode partials
are direct-to-LDS buffer loads issued as inline asm (see dma16 in
csrc/moda_tile.h), which the compiler's hazard recognizer does not look into.
One hazard of such a load is left to the surrounding compiled code: a vector
memory instruction reads an SGPR correctly only 5 wait states after a VALU
instruction wrote it.  Under SGPR pressure the compiler reloads a spilled
descriptor from VGPR lanes with v_readlane right before the asm statement; read
too early, a descriptor dword is stale and the load goes to a wrong address.
The build scans every kernel's assembly and refuses to link a library that has
such a load, so the asm itself needs no padding in the common case.
"""
import re

_FUNC = re.compile(r"^(_Z\S+):")
_SGPR = re.compile(r"s\[(\d+):(\d+)\]|s(\d+)$")

# Wait states a vector memory instruction needs after a VALU write of an SGPR it reads.
VMEM_SGPR_WAIT_STATES = 5


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


def _sgprs(tok):
    m = _SGPR.match(tok.strip())
    if not m:
        return set()
    if m.group(3) is not None:
        return {int(m.group(3))}
    return set(range(int(m.group(1)), int(m.group(2)) + 1))


def _sgpr_dests(text):
    """SGPRs a VALU instruction writes: its first operand (v_readlane, v_readfirstlane,
    v_cmp), and for the forms with a scalar carry or condition output (v_*_co_*,
    v_div_scale_*, v_mad_u64_u32, v_mad_i64_i32) also its second."""
    op, _, rest = text.partition(" ")
    ops = [o.strip() for o in rest.split(",")]
    out = _sgprs(ops[0]) if ops else set()
    if len(ops) > 1 and ("_co_" in op or "div_scale" in op or op.startswith(("v_mad_u64", "v_mad_i64"))):
        out |= _sgprs(ops[1])
    return out


def is_lds_load(text):
    t = text.strip().split(";")[0].strip()
    return t.startswith("buffer_load") and t.endswith(" lds")


def sgpr_hazards(lines, need=VMEM_SGPR_WAIT_STATES):
    """Direct-to-LDS loads whose descriptor SGPRs a VALU instruction wrote fewer than `need`
    wait states before them.  A branch target or the start of the listing inside that
    window counts as a violation (the path into it is not followed)."""
    bad = []
    for i, line in enumerate(lines):
        if not is_lds_load(line):
            continue
        t = line.strip().split(";")[0].strip()
        rsrc = _sgprs(t.split(None, 1)[1].split(",")[1])
        ws, j = 0, i - 1
        while ws < need:
            if j < 0:
                bad.append("line %d: kernel start within %d wait states of: %s" % (i, need, t))
                break
            u = lines[j].strip().split(";")[0].strip()
            j -= 1
            if u.endswith(":"):
                bad.append("line %d: branch target within %d wait states of: %s" % (i, need, t))
                break
            if not u or u.startswith("."):
                continue
            op = u.split()[0]
            if op.startswith("v_") and " " in u and _sgpr_dests(u) & rsrc:
                bad.append("line %d: %s written by '%s' %d wait states before: %s" % (i, sorted(rsrc), u, ws, t))
                break
            ws += int(u.split()[1], 0) + 1 if op == "s_nop" else 1
    return bad


def check_listing(asm_text):
    """[(kernel, violation)] for every kernel of one assembly listing."""
    out = []
    for name, lines in functions(asm_text).items():
        out += [(name, b) for b in sgpr_hazards(lines)]
    return out
