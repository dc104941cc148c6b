"""Static hazard check of the generated gfx950 assembly of the GEMM kernels.

The MFMAs of the mainloops are inline asm with the accumulators tied to
AGPRs, so the compiler's hazard recognizer does not know their latency.  If
the register allocator inserts an accumulator copy (v_accvgpr_read / write /
mov) too close to the inline-asm MFMA that writes the same AGPR, the copy can
read a value before the MFMA has written it (or overwrite it too early).

This check follows each kernel's control flow (basic blocks split at labels
and branches, successors by fall-through and branch target) and, for every
AGPR access, finds the fewest wait states issued since an MFMA that touched
an overlapping AGPR on any path reaching it (each instruction counts 1,
`s_nop N` counts N + 1).  The access must be at least MIN_WAIT_STATES away --
more than the largest requirement for a dependent VALU access after a
16-pass MFMA on gfx950.  The build fails otherwise.
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


BRANCH = re.compile(r"^\s*(s_branch|s_cbranch_\w+)\s+(\S+)")
LABEL = re.compile(r"^(\.LBB\w+|_ZN4coda\w*):")


def _kernels(text):
    """Yields (kernel_name, [(line_no, text)]) for every coda kernel."""
    kernel, body = None, []
    for no, line in enumerate(text.splitlines(), 1):
        if re.match(r"^_ZN4coda\w*:", line):
            kernel, body = line.split(":")[0], []
            continue
        if kernel is None:
            continue
        if line.startswith(".Lfunc_end"):
            yield kernel, body
            kernel = None
            continue
        body.append((no, line))


def _blocks(body):
    """Basic blocks of one kernel: (label or None, [(line_no, instr)], successors)."""
    blocks, cur_label, cur = [], None, []

    def close():
        blocks.append([cur_label, list(cur), None])

    for no, line in body:
        m = LABEL.match(line)
        if m:
            if cur or cur_label is not None:
                close()
            cur_label, cur = m.group(1), []
            continue
        s = line.strip()
        if not s or s.startswith(";") or s.startswith("."):
            continue
        cur.append((no, s))
        if BRANCH.match(s) or s.startswith("s_endpgm"):
            close()
            cur_label, cur = None, []
    if cur or cur_label is not None:
        close()
    index = {blk[0]: k for k, blk in enumerate(blocks) if blk[0] is not None}
    for k, blk in enumerate(blocks):
        succ = []
        last = blk[1][-1][1] if blk[1] else ""
        m = BRANCH.match(last)
        if m:
            if m.group(2) in index:
                succ.append(index[m.group(2)])
            if m.group(1) != "s_branch" and k + 1 < len(blocks):
                succ.append(k + 1)
        elif not last.startswith("s_endpgm") and k + 1 < len(blocks):
            succ.append(k + 1)
        blk[2] = succ
    return blocks


def check_asm_text(text, min_wait=MIN_WAIT_STATES):
    """Returns a list of (kernel, line_no, instruction, wait_states).

    For every AGPR access, the fewest wait states issued since an MFMA that
    touched an overlapping AGPR, over every control-flow path reaching it
    (a forward data-flow over the kernel's basic blocks: at a join the
    smaller distance wins), must be at least `min_wait`."""
    bad = []
    for kernel, body in _kernels(text):
        blocks = _blocks(body)
        entry = [dict() for _ in blocks]   # agpr -> wait states since its last MFMA
        seen = [False] * len(blocks)
        work = [0] if blocks else []
        seen_bad = set()
        while work:
            k = work.pop()
            age = dict(entry[k])
            for no, s in blocks[k][1]:
                m = MFMA_OP.match(s)
                if m:
                    lo, hi = (int(m.group(2)), int(m.group(3))) if m.group(2) else (int(m.group(4)),) * 2
                    age = {r: a + 1 for r, a in age.items() if a + 1 < min_wait}
                    for r in range(lo, hi + 1):
                        age[r] = 0
                    continue
                a_op = AGPR_OP.match(s)
                if a_op:
                    for r in _agprs(a_op.group(2)):
                        if r in age and (no, s) not in seen_bad:
                            seen_bad.add((no, s))
                            bad.append((kernel, no, s, age[r]))
                            break
                n = NOP.match(s)
                step = int(n.group(1)) + 1 if n else 1
                age = {r: a + step for r, a in age.items() if a + step < min_wait}
            for t in blocks[k][2]:
                merged = dict(entry[t])
                for r, a in age.items():
                    if r not in merged or a < merged[r]:
                        merged[r] = a
                if not seen[t] or merged != entry[t]:
                    seen[t] = True
                    entry[t] = merged
                    work.append(t)
            seen[k] = True
    return bad


SPILL = re.compile(r"^\s+\.name:\s+(\S+)|^\s+\.(vgpr|sgpr)_spill_count:\s+(\d+)")


def spills(text):
    """Kernels of the assembly text that spill registers: [(name, kind, count)]."""
    out, name = [], None
    for line in text.splitlines():
        m = SPILL.match(line)
        if not m:
            continue
        if m.group(1):
            name = m.group(1)
        elif int(m.group(3)) > 0:
            out.append((name, m.group(2), int(m.group(3))))
    return out


def check_source(hipcc, src, flags):
    """Compile `src` to device assembly and check it; raise on hazards or on
    vector register spills (scratch memory traffic inside a GEMM kernel is a
    performance bug; scalar spills go to vector register lanes and are
    allowed)."""
    cmd = [hipcc] + flags + ["--cuda-device-only", "-S", src, "-o", "-"]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"assembly of {src} failed:\n{p.stderr}")
    sp = [x for x in spills(p.stdout) if x[1] == "vgpr"]
    if sp:
        raise RuntimeError(f"{src}: vector register spills: {sp}")
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
