"""Path-sensitive check of gfx950 assembly for in-flight LDS read hazards.

The DMA kernels issue their fragment reads from LDS as inline assembly, so the
compiler neither inserts the waits for them nor knows that their destination
registers are written when the data arrives rather than at issue.  The
kernels wait explicitly (s_waitcnt lgkmcnt); this check verifies on the
compiled code that no instruction names a register that an LDS read still in
flight will write (or that it reads from), along every control-flow path.

Model: LDS reads (ds_read*) complete in issue order; each adds its
destination registers to a queue, and s_waitcnt lgkmcnt(n) retires the oldest
until at most n remain.  From the kernel entry, both successors of every
conditional branch are followed to a fixpoint of (instruction, queue) states.
Any other instruction whose operands name a queued register is a hazard; a
later LDS read into the same registers is not (it lands later), but its
address operand is checked.  Scalar instructions are skipped: LDS reads write
vector registers only.
"""
import re

_LABEL = re.compile(r"^\.LBB\d+_\d+:$")


def _regs(text: str) -> set:
    out = set()
    for kind in ("v", "a"):
        for m in re.finditer(rf"\b{kind}\[(\d+):(\d+)\]", text):
            out |= {(kind, i) for i in range(int(m.group(1)), int(m.group(2)) + 1)}
        for m in re.finditer(rf"\b{kind}(\d+)\b", text):
            out.add((kind, int(m.group(1))))
    return out


def kernel_hazards(lines) -> dict:
    """Hazards of one function's assembly lines: {instruction: registers}."""
    f = [l.split(";")[0].strip() for l in lines]
    f = [l for l in f if l and (not l.startswith(".") or _LABEL.match(l))]
    labels = {l[:-1]: k for k, l in enumerate(f) if _LABEL.match(l)}
    found = {}
    seen = set()
    work = [(0, ())]
    while work:
        pc, pend = work.pop()
        while pc < len(f):
            if (pc, pend) in seen:
                break
            seen.add((pc, pend))
            line = f[pc]
            op = line.split()[0]
            if op.endswith(":"):
                pc += 1
                continue
            if op == "s_endpgm":
                break
            if op == "s_waitcnt":
                m = re.search(r"lgkmcnt\((\d+)\)", line)
                if m and len(pend) > int(m.group(1)):
                    pend = pend[len(pend) - int(m.group(1)):]
                pc += 1
                continue
            if op == "s_branch":
                pc = labels[line.split()[1]]
                continue
            if op.startswith("s_cbranch"):
                work.append((labels[line.split()[1]], pend))
                pc += 1
                continue
            if op.startswith("s_"):
                pc += 1
                continue
            args = line.split(None, 1)[1] if " " in line else ""
            operands = ",".join(args.split(",")[1:]) if op.startswith("ds_read") else args
            queued = set().union(*pend) if pend else set()
            hit = _regs(operands) & queued
            if hit:
                found.setdefault(line, sorted(hit))
            if op.startswith("ds_read"):
                pend = pend + (frozenset(_regs(args.split(",")[0])),)
            pc += 1
    return found


def file_hazards(text: str, name_pattern: str = r"gemm_dma_kernel") -> dict:
    """{kernel symbol: hazards} for every function of an assembly file whose
    symbol matches name_pattern; also returns how many were checked."""
    lines = text.split("\n")
    out = {}
    n = 0
    for i, l in enumerate(lines):
        m = re.match(r"^(_Z\S+):", l)
        if not m or not re.search(name_pattern, m.group(1)):
            continue
        e = i
        while not lines[e].startswith(".Lfunc_end"):
            e += 1
        n += 1
        h = kernel_hazards(lines[i:e])
        if h:
            out[m.group(1)] = h
    return out, n

