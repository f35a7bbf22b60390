"""Static checks on the gfx950 assembly of this library's kernels (the
compiler's own output for our sources, built with the library's flags).

For every MFMA instruction of a kernel:
  - overlap: its srcA or srcB registers lie inside its destination range;
  - near_valu_write: the nearest earlier instruction that writes one of its
    srcA/srcB registers with a vector-ALU op (including v_accvgpr_read_b32,
    the move from an accumulation register) sits fewer than `min_gap` wait
    states before it (each instruction counts one wait state, s_nop n counts
    n + 1; other MFMAs, loads, stores and scalar instructions are not such
    writers).
"""
import re

_REG = re.compile(r'\b([va])(?:\[(\d+):(\d+)\]|(\d+))\b')
_NOT_VALU_WRITE = ("ds_", "global_", "buffer_", "scratch_", "flat_", "s_", "v_cmp", "v_readlane", "v_readfirstlane",
                   "v_mfma", "v_writelane")


def regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(4) is not None:
            out.add((m.group(1), int(m.group(4))))
        else:
            out.update((m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def kernels(asm):
    """{kernel symbol: [instruction lines]} of an assembly file."""
    out = {}
    for m in re.finditer(r'^(_Z\w+):[^\n]*\n(.*?)^\s*s_endpgm', asm, re.S | re.M):
        lines = [l.split(";")[0].strip() for l in m.group(2).split("\n")]
        out[m.group(1)] = [l for l in lines if l and not l.startswith(".") and not l.endswith(":")]
    return out


def _wait_states(line):
    if line.startswith("s_nop"):
        return int(line.split()[1], 0) + 1
    return 1


def mfma_report(ins, min_gap=4, window=16):
    """(MFMA count, overlaps, near VALU writes) of one kernel's instructions;
    the last two are lists of (instruction, detail)."""
    n, overlaps, near = 0, [], []
    for i, line in enumerate(ins):
        if not line.startswith("v_mfma"):
            continue
        n += 1
        ops = [o.strip() for o in line.split(None, 1)[1].split(",")]
        dst, src = regs(ops[0]), regs(ops[1]) | regs(ops[2])
        if dst & src:
            overlaps.append((line, sorted(dst & src)))
        ws = 0
        for j in range(i - 1, -1, -1):
            prev = ins[j]
            if ws >= window:
                break
            if not prev.startswith(_NOT_VALU_WRITE) and prev.startswith("v_"):
                parts = prev.split(None, 1)
                if len(parts) == 2 and regs(parts[1].split(",")[0]) & src:
                    if ws < min_gap:
                        near.append((line, "%s, %d wait states before" % (prev, ws)))
                    break
            ws += _wait_states(prev)
    return n, overlaps, near


def accvgpr_reads(ins):
    return sum(1 for l in ins if l.startswith("v_accvgpr_read"))
