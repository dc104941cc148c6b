"""Static hazard check of the generated gfx950 assembly of the GEMM kernels.

The MFMAs of the mainloops are inline asm with the accumulators tied to
AGPRs, so the compiler's hazard recognizer does not know their latency.  If
the register allocator inserts an accumulator copy (v_accvgpr_read / write /
mov) too close to the inline-asm MFMA that writes the same AGPR, the copy can
read a value before the MFMA has written it (or overwrite it too early).

This check walks each kernel's instructions in program order and, for every
AGPR access, measures the wait states issued since the last MFMA that touched
an overlapping AGPR (each instruction counts 1, `s_nop N` counts N + 1).  The
access must be at least MIN_WAIT_STATES away -- more than the largest
requirement for a dependent VALU access after a 16-pass MFMA on gfx950.  The
build fails otherwise.  (Program order is the execution order inside the
straight-line stage bodies, where the MFMAs are; the wait-state block at the
end of every mainloop covers the branch into the epilogue.)
"""

import re
import subprocess
import sys

MIN_WAIT_STATES = 24
AGPR_OP = re.compile(r"^\s*v_accvgpr_(read|write|mov)_b32\s+(.*)$")
MFMA_OP = re.compile(r"^\s*v_mfma\w*\s+(a\[(\d+):(\d+)\]|a(\d+))")
NOP = re.compile(r"^\s*s_nop\s+(\d+)")
AREG = re.compile(r"a\[(\d+):(\d+)\]|\ba(\d+)\b")


def _agprs(operands):
    regs = set()
    for m in AREG.finditer(operands):
        if m.group(1) is not None:
            regs.update(range(int(m.group(1)), int(m.group(2)) + 1))
        else:
            regs.add(int(m.group(3)))
    return regs


def check_asm_text(text, min_wait=MIN_WAIT_STATES):
    """Returns a list of (kernel, line_no, instruction, wait_states)."""
    bad = []
    kernel = None
    clock = 0           # wait states issued so far in this kernel
    last_mfma = {}      # agpr -> clock right after the MFMA touching it issued
    for no, line in enumerate(text.splitlines(), 1):
        if re.match(r"^_ZN4coda\w*:", line):
            kernel, clock, last_mfma = line.split(":")[0], 0, {}
            continue
        if kernel is None:
            continue
        if line.startswith(".Lfunc_end"):
            kernel = None
            continue
        s = line.strip()
        if not s or s.startswith(";") or s.startswith(".") or s.endswith(":"):
            continue
        m = MFMA_OP.match(line)
        if m:
            lo, hi = (int(m.group(2)), int(m.group(3))) if m.group(2) else (int(m.group(4)),) * 2
            clock += 1
            for r in range(lo, hi + 1):
                last_mfma[r] = clock
            continue
        n = NOP.match(line)
        if n:
            clock += int(n.group(1)) + 1
            continue
        a = AGPR_OP.match(line)
        if a:
            regs = _agprs(a.group(2))
            for r in regs:
                if r in last_mfma and clock - last_mfma[r] < min_wait:
                    bad.append((kernel, no, s, clock - last_mfma[r]))
                    break
        clock += 1
    return bad


def check_source(hipcc, src, flags):
    """Compile `src` to device assembly and check it; raise on violations."""
    cmd = [hipcc] + flags + ["--cuda-device-only", "-S", src, "-o", "-"]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"assembly of {src} failed:\n{p.stderr}")
    bad = check_asm_text(p.stdout)
    if bad:
        lines = "\n".join(f"  {k} line {n}: {i} ({w} wait states)" for k, n, i, w in bad[:12])
        raise RuntimeError(f"{src}: accumulator access too close to an inline-asm MFMA "
                           f"({len(bad)} found):\n{lines}")
    return True


if __name__ == "__main__":
    v = check_asm_text(open(sys.argv[1]).read())
    for k, n, i, w in v[:20]:
        print(k, n, i, w)
    print(f"{len(v)} violations")
    sys.exit(1 if v else 0)
