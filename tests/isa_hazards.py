"""Scan gfx950 assembly for two MFMA data hazards that the hardware does not
interlock and that the kernels' inline-asm MFMAs keep by hand.

The kernels issue many MFMAs as inline asm (fixed register classes), which the
compiler's hazard recognizer does not see; their guards (`s_nop` runs tied to
the operands and results) are placed by hand.  This scan checks the compiled
code for:

  1. a non-MFMA vector instruction (VALU, LDS, memory) reading or writing a
     register fewer wait states after an MFMA that writes it than the MFMA's
     passes require (CDNA3/CDNA4 hazard table: 4 passes -> 7, 8 passes -> 11,
     16 passes -> 19 wait states);
  2. an MFMA reading (A, B or C) a register that a VALU instruction wrote
     fewer than 2 wait states before.

Wait states: `s_nop N` counts N + 1, every other instruction 1.  The scan is
linear over the kernel's text (it follows fall-through, not branches), so it
checks every straight-line stretch the way it is laid out.  An MFMA right
after a label may also be reached by a branch: the branch itself counts 1
wait state, so the instruction before each branch to that label is checked
as well (3. below); the result guards do not rely on branch targets.

  3. an MFMA reached by a branch fewer than 2 wait states after a VALU write
     of a register it reads (an MFMA right at the label, after a branch whose
     previous instruction writes an operand).
"""
import re

# passes of the MFMA opcodes the kernels use (gfx950); unknown ones count 16
_PASSES = (("32x32x16_bf16", 8), ("32x32x16_f16", 8), ("16x16x32_bf16", 4),
           ("32x32x64_f8f6f4", 16), ("16x16x128_f8f6f4", 8))
_NEED = {4: 7, 8: 11, 16: 19}
_REG = re.compile(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b")


def _regs(tok):
    out = set()
    for m in _REG.finditer(tok):
        if m.group(1):
            out |= {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


def _passes(op):
    for key, p in _PASSES:
        if key in op:
            return p
    return 16


def kernels(asm_text):
    """{kernel symbol: [instruction lines]} for every kernel in the file."""
    out, cur = {}, None
    for line in asm_text.split("\n"):
        m = re.match(r"^(_Z\S*):", line)
        if m:
            cur = m.group(1)
            out[cur] = []
            continue
        if cur is None:
            continue
        s = line.split(";")[0].strip()
        if not s:
            continue
        if s.endswith(":"):
            s = "<label> " + s[:-1]   # a branch target
        elif s.startswith("."):
            continue
        out[cur].append(s)
        if s.startswith("s_endpgm"):
            cur = None
    return out


def _before_branches(lines, name):
    """The instruction ahead of each branch to label `name`."""
    out = []
    for j, s in enumerate(lines):
        w = s.split()
        if len(w) == 2 and w[0].startswith(("s_branch", "s_cbranch")) and w[1] == name:
            out.append(lines[j - 1] if j else "<label>")
    return out


def scan(lines):
    """Findings (index, opcode, register, wait states seen, needed) in one kernel."""
    clock = 0
    mfma_w = {}   # register -> (clock of the MFMA that last wrote it, wait states needed)
    valu_w = {}   # register -> clock of the last VALU write
    found = []
    label = None  # (clock, name) of the last label
    for i, s in enumerate(lines):
        op = s.split()[0]
        if op == "<label>":
            label = (clock, s.split()[1] if len(s.split()) > 1 else "")
            continue
        if op.startswith("s_nop"):
            clock += int(s.split()[1], 0) + 1
            continue
        clock += 1
        parts = [p.strip() for p in s[len(op):].split(",")]
        if "mfma" in op:
            reads = set().union(*[_regs(p) for p in parts[1:]])
            if label is not None and clock - label[0] - 1 == 0:
                # right at a branch target: the branch gives 1 wait state, so
                # the instruction ahead of it must not write an operand
                for prev in _before_branches(lines, label[1]):
                    if prev.startswith("<label>") or (prev.startswith("v_") and _regs(prev.split(",")[0]) & reads):
                        found.append((i, op, "branch target", 1, 2))
            for r in reads:
                if r in valu_w and clock - valu_w[r] < 3:
                    found.append((i, op, r, clock - valu_w[r] - 1, 2))
            need = _NEED[_passes(op)]
            for r in _regs(parts[0]):
                mfma_w[r] = (clock, need)
            continue
        if op.startswith(("v_", "ds_", "buffer_", "global_", "scratch_", "flat_")):
            for r in set().union(*[_regs(p) for p in parts]) if parts and parts[0] else ():
                if r in mfma_w:
                    c0, need = mfma_w[r]
                    if clock - c0 - 1 < need:
                        found.append((i, op, r, clock - c0 - 1, need))
            if op.startswith("v_") and parts and parts[0]:
                for r in _regs(parts[0]):
                    valu_w[r] = clock
    return found
