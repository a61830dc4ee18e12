"""Wait-state check for the MFMAs the kernels issue as inline assembly.

The tile loop issues its MFMAs as assembly statements so that their order
against LDS reads and VALU work is fixed.  The compiler then does not know
these instructions are MFMAs: it inserts no wait states after them.  The
hardware needs them in two places (gfx950, as the compiler itself pads its
own MFMAs):
  * a VALU (or memory) instruction reading or overwriting an MFMA result
    must come at least 10 + 2 wait states (8-pass 32x32x16 f16/bf16) after
    the MFMA;
  * an MFMA reading a VGPR written by a VALU instruction needs 2 wait states.
Back-to-back MFMAs that accumulate into exactly the same registers need none.
This module scans the compiled assembly of every kernel and reports each
place where either rule is broken; the build fails if there is one.
"""

import re
import sys

RESULT_WAIT = {"v_mfma_f32_32x32x16_bf16": 12, "v_mfma_f32_32x32x16_f16": 12, "v_mfma_f32_32x32x2_f32": 18}
VALU_TO_MFMA_WAIT = 2


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def _split(line):
    parts = line.split(None, 1)
    if len(parts) < 2:
        return parts[0], []
    return parts[0], [o.strip() for o in re.split(r",\s*(?![^\[]*\])", parts[1].split(";")[0])]


def check_function(lines, name):
    """Returns a list of messages for one kernel's assembly lines."""
    problems = []
    in_asm = False
    pending = []   # [regs written by an asm MFMA, wait states still needed, line]
    recent = []    # [regs written by VALU, wait states still needed]
    for ln, raw in enumerate(lines):
        s = raw.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not s or s.startswith(";") or s.startswith(".") or s.endswith(":"):
            continue
        op, ops = _split(s)
        ws = int(ops[0], 0) + 1 if op == "s_nop" else 1
        is_mfma = op.startswith("v_mfma")
        if op != "s_nop" and not op.startswith("s_"):
            touched = set()
            for o in ops:
                touched |= _regs(o)
            for dst, rem, l0 in pending:
                if is_mfma and len(ops) >= 4 and _regs(ops[0]) == dst and _regs(ops[3]) == dst:
                    continue  # exact accumulation chain
                if touched & dst:
                    problems.append(f"{name}:{ln}: MFMA result (line {l0}) used {rem} wait states early: {s}")
            if is_mfma and in_asm:
                srcs = set()
                for o in ops[1:]:
                    srcs |= _regs(o)
                for regs, rem in recent:
                    if srcs & regs:
                        problems.append(f"{name}:{ln}: VALU result read by MFMA {rem} wait states early: {s}")
        pending = [(d, r - ws, l) for (d, r, l) in pending if r - ws > 0]
        recent = [(g, r - ws) for (g, r) in recent if r - ws > 0]
        if is_mfma and in_asm:
            pending.append((_regs(ops[0]), RESULT_WAIT.get(op, 18), ln))
        elif op.startswith("v_") and not is_mfma and ops:
            recent.append((_regs(ops[0]), VALU_TO_MFMA_WAIT))
    return problems


def check_asm(text):
    lines = text.split("\n")
    starts = [i for i, l in enumerate(lines) if re.match(r"^_Z\S+:", l)]
    problems = []
    for k, st in enumerate(starts):
        en = starts[k + 1] if k + 1 < len(starts) else len(lines)
        problems += check_function(lines[st:en], lines[st].split(":")[0])
    return problems


if __name__ == "__main__":
    probs = check_asm(open(sys.argv[1]).read())
    for p in probs[:50]:
        print(p)
    print(f"{len(probs)} problem(s)")
    sys.exit(1 if probs else 0)
