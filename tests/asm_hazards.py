"""Read gfx950 assembly text and find matrix-core instructions that read a
VGPR written by a vector-ALU instruction fewer than 2 wait states before.

A VALU write of a VGPR followed by an MFMA that reads it (as an operand or,
for the block-scaled forms, as a scale) needs 2 wait states in between; the
compiler inserts them for MFMAs written as builtins but cannot see into
inline assembly, so kernels that issue MFMAs from inline asm carry the
obligation themselves.  Wait states are counted as instructions issued in
between, an ``s_nop N`` counting N + 1.  Fall-through order is checked, and
every loop back edge: the last instructions before a branch to an earlier
label followed by the first ones after that label."""
import re

NEED = 2


def _regs(tok):
    tok = tok.strip().rstrip(",")
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.fullmatch(r"([va])(\d+)", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _instructions(text):
    out, labels, func = [], {}, None
    for ln, line in enumerate(text.splitlines(), 1):
        if re.match(r"^[A-Za-z_]\S*:", line) and not line.startswith("."):
            func = line.split(":")[0]
            continue
        m = re.match(r"^(\.LBB\w+):", line)
        if m:
            labels[(func, m.group(1))] = len(out)
            continue
        s = line.split(";")[0].strip()
        if not s or s.endswith(":") or s.startswith("."):
            continue
        parts = s.split(None, 1)
        ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
        out.append((func, ln, parts[0], ops, s))
    return out, labels


def _info(ins):
    _, _, op, ops, _ = ins
    if op.startswith("v_mfma"):
        srcs = set()
        for o in ops[1:]:
            if o:
                srcs |= _regs(o.split()[0])
        return 1, set(), srcs
    w = int(ops[0], 0) + 1 if op == "s_nop" else 1
    written = _regs(ops[0].split()[0]) if op.startswith("v_") and ops else set()
    return w, {r for r in written if r[0] == "v"}, None


def _scan(seq, start, found):
    for k in range(start, len(seq)):
        _, _, srcs = _info(seq[k])
        if srcs is None:
            continue
        ws, j = 0, k - 1
        while j >= 0 and ws < NEED:
            wj, written, _ = _info(seq[j])
            if written & srcs:
                found.add((seq[k][0], seq[k][1], seq[k][4], ws))
            ws += wj
            j -= 1


def find(text):
    """[(function, line, instruction, wait states seen)] for every violation."""
    ins, labels = _instructions(text)
    found = set()
    _scan(ins, 0, found)
    for i, x in enumerate(ins):
        if (x[2].startswith("s_cbranch") or x[2] == "s_branch") and x[3]:
            h = labels.get((x[0], x[3][0]))
            if h is not None and h <= i:
                tail = ins[max(0, i - 8):i + 1]
                _scan(tail + ins[h:h + 12], len(tail), found)
    return sorted(found)
