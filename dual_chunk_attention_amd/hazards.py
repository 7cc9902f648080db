"""Build-time check of the matrix-core hazards that inline assembly hides from the compiler.

The fused prefill kernel issues its score MFMAs as inline asm (so that the accumulator stays in
VGPRs and every MFMA keeps its place), without the wait states that the compiler would put in front
of a builtin MFMA.  On gfx950 an MFMA that reads a VGPR written by a VALU instruction needs two wait
states after that write.  The kernel relies on its operands coming from LDS reads (K fragments),
global loads (Q) or earlier MFMAs (the accumulator), never from a VALU write just before.  This
module checks that property on the generated assembly: no VALU instruction among the two
instructions in front of an inline-asm MFMA block writes any register that the block's MFMAs read
or write.  The build fails when it does not hold.
"""
import re
import subprocess

WAIT_STATES = 2   # VALU write of a VGPR -> MFMA read of it


def _regs(text):
    out = set()
    for m in re.finditer(r"\b([av])\[(\d+):(\d+)\]|\b([av])(\d+)\b", text):
        if m.group(1):
            out |= {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


def _is_instruction(line):
    s = line.strip()
    return bool(s) and not s.startswith((";", ".")) and not s.endswith(":")


def asm_mfma_violations(isa: str, wait_states: int = WAIT_STATES):
    """(line number, instruction) of every VALU write to an operand of an inline-asm MFMA block
    within `wait_states` instructions before the block, and the number of blocks checked."""
    lines = isa.split("\n")
    bad, blocks, i = [], 0, 0
    while i < len(lines):
        if "ASMSTART" not in lines[i]:
            i += 1
            continue
        j = i + 1
        body = []
        while j < len(lines) and "ASMEND" not in lines[j]:
            body.append(lines[j].strip())
            j += 1
        mfmas = [b for b in body if b.startswith("v_mfma")]
        if mfmas:
            blocks += 1
            operands = set()
            for m in mfmas:
                operands |= _regs(m.split(None, 1)[1])
            k, seen = i - 1, 0
            while k >= 0 and seen < wait_states:
                if _is_instruction(lines[k]):
                    seen += 1
                    s = lines[k].strip()
                    if s.startswith("v_") and not s.startswith("v_mfma") and " " in s:
                        if _regs(s.split(None, 1)[1].split(",")[0]) & operands:
                            bad.append((k + 1, s))
                k -= 1
        i = j + 1
    return bad, blocks


def device_isa(src: str, flags) -> str:
    """The gfx950 assembly hipcc generates for `src` with the library's flags."""
    cmd = ["hipcc", "-S", "-x", "hip", src, "-o", "-", "--cuda-device-only"] + [f for f in flags if f != "-fPIC"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed on {src}:\n{r.stderr}")
    return r.stdout


def check_source(src: str, flags) -> int:
    """Raise if the generated code of `src` breaks the rule; returns the number of blocks checked."""
    bad, blocks = asm_mfma_violations(device_isa(src, flags))
    if bad:
        where = "\n".join(f"  line {n}: {s}" for n, s in bad[:10])
        raise RuntimeError(f"{src}: VALU writes of inline-asm MFMA operands within {WAIT_STATES} "
                           f"instructions of the MFMA:\n{where}")
    if blocks == 0:
        raise RuntimeError(f"{src}: no inline-asm MFMA blocks found (the check would be vacuous)")
    return blocks
