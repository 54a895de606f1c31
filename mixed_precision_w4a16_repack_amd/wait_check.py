"""Build check of the hand-counted memory waits of the staged GEMM kernels.

The tiled kernels (mfma_ring_kernel, mfma_lds_kernel, w4a8_ring_kernel) load
operand tiles straight into LDS with buffer loads that no register tracks,
so the compiler cannot wait for them; each pipeline step instead ends with a
hand-written ``s_waitcnt vmcnt(N)`` before its barrier. N is only right if the
compiler emits exactly the vector-memory instructions the source counts: a
dropped dead load, an extra spill or a hoisted load changes the count and
turns the pipeline into a race that may show only now and then.

This module reads the gfx950 assembly of a build (``hipcc --cuda-device-only
-S``), rebuilds each kernel's control-flow graph and, for every hand-written
wait that is followed by a hand-written barrier, counts along every path
backwards the vector-memory instructions between the wait and the loads
that must have landed:

* ``mfma_ring_kernel`` (three LDS stages): every load issued before the
  previous barrier must have landed, so N must equal the number of
  vector-memory instructions since that barrier;
* ``w4a8_ring_kernel`` (four stages): every load issued before the barrier
  two steps back must have landed;
* ``mfma_lds_kernel`` (two buffers, weights in registers): the step's last
  direct-to-LDS load must have landed, so N must equal the number of
  vector-memory instructions after it;
* ``mfma_splitk_kernel`` (NS stages, NS its last template argument): every
  load issued before the barrier NS - 2 steps back must have landed.

A path that reaches the kernel entry (the prologue, which issues more
stages than it waits for) only needs at least N instructions. Any other
count differing from N fails the check.

    python -m mixed_precision_w4a16_repack_amd.wait_check file.s [file.s ...]
"""

from __future__ import annotations

import re
import sys

def _splitk_rule(name: str):
    """The split-K ring waits across NS - 2 barriers (NS: the last template
    argument of the mangled name, ...ELi<NS>EEEv...)."""
    m = re.search(r"ELi(\d+)EEEv", name)
    if not m:
        raise ValueError(f"no stage count in {name}")
    return ("barriers", int(m.group(1)) - 2)


# kernel name fragment -> ("barriers", depth), ("lds", None), or a function
# of the mangled name returning one of those
RULES = {
    "mfma_ring_kernel": ("barriers", 1),
    "w4a8_ring_kernel": ("barriers", 2),
    "mfma_lds_kernel": ("lds", None),
    "mfma_splitk_kernel": _splitk_rule,
}

_VMEM = re.compile(r"^(buffer_|global_|flat_|scratch_)")
_TERM = re.compile(r"^(s_branch|s_cbranch_\w+|s_endpgm|s_setpc_b64)\b")


class Instr:
    __slots__ = ("text", "in_asm")

    def __init__(self, text: str, in_asm: bool):
        self.text = text
        self.in_asm = in_asm

    @property
    def vmem(self) -> bool:
        return bool(_VMEM.match(self.text))

    @property
    def lds_load(self) -> bool:
        return self.vmem and "_load" in self.text.split()[0] and re.search(r"\blds\b", self.text) is not None

    @property
    def hand_barrier(self) -> bool:
        return self.in_asm and self.text.startswith("s_barrier")

    def hand_wait(self) -> int | None:
        if not self.in_asm:
            return None
        m = re.match(r"s_waitcnt\s+vmcnt\((\d+)\)", self.text)
        return int(m.group(1)) if m else None


def _functions(asm: str):
    """Yields (name, list of lines) for every kernel in an assembly file."""
    lines = asm.split("\n")
    i = 0
    while i < len(lines):
        m = re.match(r"^(_Z\S+):", lines[i])
        if m:
            j = i + 1
            while j < len(lines) and not lines[j].startswith(".Lfunc_end"):
                j += 1
            yield m.group(1), lines[i + 1:j]
            i = j
        i += 1


def _blocks(lines):
    """Basic blocks of one function: list of (label, [Instr]) and the
    successor indices of each block."""
    blocks: list[tuple[str | None, list[Instr]]] = [(None, [])]
    in_asm = False
    for raw in lines:
        t = raw.split(";")[0].strip() if not raw.strip().startswith(";;#ASM") else raw.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not t or t.startswith("."):
            m = re.match(r"^(\.LBB\w+):", t)
            if m:
                blocks.append((m.group(1), []))
            continue
        if t.endswith(":"):
            continue
        for part in t.split("\n"):
            part = part.strip()
            if part:
                blocks[-1][1].append(Instr(part, in_asm))
                if not in_asm and _TERM.match(part):
                    blocks.append((None, []))
    blocks = [b for b in blocks if b[0] is not None or b[1]]
    index = {lab: k for k, (lab, _) in enumerate(blocks) if lab}
    succ: list[list[int]] = []
    for k, (_, ins) in enumerate(blocks):
        s: list[int] = []
        last = ins[-1].text if ins else ""
        m = re.match(r"^(s_branch|s_cbranch_\w+)\s+(\.LBB\w+)", last)
        if m:
            s.append(index[m.group(2)])
            if m.group(1) != "s_branch" and k + 1 < len(blocks):
                s.append(k + 1)
        elif last.startswith("s_endpgm") or last.startswith("s_setpc_b64"):
            pass
        elif k + 1 < len(blocks):
            s.append(k + 1)
        succ.append(s)
    pred: list[list[int]] = [[] for _ in blocks]
    for k, s in enumerate(succ):
        for t in s:
            pred[t].append(k)
    return blocks, pred


def _count_back(blocks, pred, bk: int, pos: int, rule: str, depth: int | None):
    """Set of (count, reached_entry) over every backward path from
    instruction pos of block bk (exclusive) to the rule's boundary."""
    results: set[tuple[int, bool]] = set()
    stack = [(bk, pos, 0, 0, frozenset())]
    while stack:
        b, p, crossed, count, seen = stack.pop()
        ins = blocks[b][1]
        stopped = False
        for k in range(p - 1, -1, -1):
            it = ins[k]
            if rule == "lds" and it.lds_load:
                results.add((count, False))
                stopped = True
                break
            if it.vmem:
                count += 1
            if rule == "barriers" and it.hand_barrier:
                crossed += 1
                if crossed == depth:
                    results.add((count, False))
                    stopped = True
                    break
        if stopped:
            continue
        if not pred[b]:
            results.add((count, True))
            continue
        key = (b, crossed)
        if key in seen:
            raise RuntimeError("a loop without a boundary on the way back from a hand-written wait")
        for q in pred[b]:
            stack.append((q, len(blocks[q][1]), crossed, count, seen | {key}))
    return results


def check_function(name: str, lines) -> list[str]:
    """Problems found in one kernel (empty list: every hand wait matches)."""
    rule = None
    for frag, r in RULES.items():
        if frag in name:
            rule = r
    if rule is None:
        return []
    kind, depth = rule(name) if callable(rule) else rule
    blocks, pred = _blocks(lines)
    problems = []
    waits = 0
    for b, (_, ins) in enumerate(blocks):
        for k, it in enumerate(ins):
            n = it.hand_wait()
            if n is None or n == 0:
                continue
            # Only waits that guard a stage: a hand barrier follows in the
            # same block before any other memory instruction.
            follows = [x for x in ins[k + 1:k + 6]]
            if not any(x.hand_barrier for x in follows):
                continue
            waits += 1
            for count, entry in sorted(_count_back(blocks, pred, b, k, kind, depth)):
                if entry and count >= n:
                    continue
                if not entry and count == n:
                    continue
                where = "from the kernel entry" if entry else "in a pipeline step"
                problems.append(f"{name}: s_waitcnt vmcnt({n}) but {count} vector-memory instructions {where}")
    if waits == 0:
        problems.append(f"{name}: no hand-written stage wait found")
    return problems


def check_asm(text: str) -> tuple[int, list[str]]:
    """(kernels checked, problems) for one assembly file."""
    checked, problems = 0, []
    for name, lines in _functions(text):
        if any(frag in name for frag in RULES):
            checked += 1
            problems += check_function(name, lines)
    return checked, problems


# gfx950 needs wait states between a VALU instruction and an MFMA that share
# a VGPR: 2 between a VALU write and an MFMA that reads the register, and,
# the other way round, up to a pass count's worth between an MFMA that reads
# a register (its accumulator input is read late) and a VALU write of it.
# The compiler inserts them for the instructions it emits, but an inline-asm
# instruction is opaque to its hazard tracking. An MFMA that read an
# inline-asm VALU result too soon was seen on MI355X to read the register's
# old value (a wrong operand dword).
MFMA_VALU_WAIT_STATES = 2  # VALU write -> MFMA read
VALU_AFTER_MFMA_WAIT_STATES = 16  # MFMA read -> VALU write (16 passes, the longest here)

_VREG = re.compile(r"^v\[(\d+):(\d+)\]$|^v(\d+)$")


def _vregs(tok: str) -> set[int]:
    m = _VREG.match(tok)
    if not m:
        return set()
    if m.group(3) is not None:
        return {int(m.group(3))}
    return set(range(int(m.group(1)), int(m.group(2)) + 1))


def mfma_operand_hazards(text: str) -> list[str]:
    """Every MFMA that reads a register written by an inline-asm VALU
    instruction fewer than MFMA_VALU_WAIT_STATES wait states before it, and
    every inline-asm VALU instruction that writes a register an MFMA read
    fewer than VALU_AFTER_MFMA_WAIT_STATES wait states before, in listing
    order (which covers the straight-line code the dequantisation runs in;
    a label does not reset the history, which can only add reports)."""
    problems = []
    for name, lines in _functions(text):
        # (wait states, VGPRs written, inline-asm VALU, VGPRs an MFMA read)
        hist: list[tuple[int, set[int], bool, set[int]]] = []
        in_asm = False
        for raw in lines:
            t = raw.strip()
            if t.startswith(";;#ASMSTART"):
                in_asm = True
                continue
            if t.startswith(";;#ASMEND"):
                in_asm = False
                continue
            t = t.split(";")[0].strip()
            if not t or t.startswith(".") or t.endswith(":"):
                continue
            parts = t.replace(",", " ").split()
            op = parts[0]
            if op == "s_nop":
                hist.append((int(parts[1], 0) + 1 if len(parts) > 1 else 1, set(), False, set()))
                continue
            written = _vregs(parts[1]) if len(parts) > 1 else set()
            asm_valu = in_asm and op.startswith("v_")
            read: set[int] = set()
            if op.startswith("v_mfma"):
                for tok in parts[2:5]:
                    read |= _vregs(tok)
                ws = 0
                for w, regs, prev_asm, _ in reversed(hist):
                    if ws >= MFMA_VALU_WAIT_STATES:
                        break
                    if prev_asm and regs & read:
                        problems.append(f"{name}: '{t}' reads an inline-asm VALU result after {ws} wait states")
                        break
                    ws += w
            if asm_valu and written:
                ws = 0
                for w, _, _, mread in reversed(hist):
                    if ws >= VALU_AFTER_MFMA_WAIT_STATES:
                        break
                    if mread & written:
                        problems.append(f"{name}: inline-asm '{t}' writes a register an MFMA read {ws} wait states before")
                        break
                    ws += w
            hist.append((1, written, asm_valu, read))
            hist = hist[-40:]
    return problems


def main(paths) -> int:
    total, bad = 0, []
    for p in paths:
        with open(p) as f:
            n, probs = check_asm(f.read())
        total += n
        bad += probs
    for line in bad:
        print(line)
    print(f"{total} staged kernels checked, {len(bad)} mismatches")
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
