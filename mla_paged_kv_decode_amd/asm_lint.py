"""Build-time check of the generated gfx950 assembly for MFMA hazards the compiler cannot see.

The score MFMAs of the split-KV kernel are issued through inline asm (their
accumulators must stay in VGPRs), so the compiler neither inserts the wait
states those MFMAs need nor knows that their results arrive only after the MFMA
has run.  This lint walks the assembly of every `mla_split_kv_partial`
instantiation and reports:

  * a non-MFMA instruction that reads a VGPR written by an MFMA before
    MFMA_RESULT_WAITS wait states have passed (a VALU use, a store, or a copy
    the register allocator inserted);
  * an MFMA that reads a VGPR written by a VALU instruction fewer than
    VALU_TO_MFMA_WAITS wait states earlier;
  * a scratch (spill) access inside the hot loop (the deepest loop level that
    holds MFMAs, and loops nested in it): a spill reload there is a vector-memory
    load, and waiting for it waits for every KV tile load in flight, once per
    tile.

Wait states are counted conservatively: one per instruction, N+1 per `s_nop N`;
stalls are not credited.  A label resets the tracking (control flow merges).
"""
from __future__ import annotations

import re

MFMA_RESULT_WAITS = 20   # 16-pass XDL result -> any read (vendor tables give ~19 on gfx950)
VALU_TO_MFMA_WAITS = 2   # non-dot VALU VGPR write -> MFMA source read (the compiler's own gfx950 figure)


def _regs(tok: str) -> set:
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    if m:
        return {int(m.group(1))}
    return set()


def lint_function(lines: list[str]) -> list[str]:
    problems = []
    pending = []   # (dst registers of an MFMA, wait states since, line index)
    recent = []    # (dst registers of a VALU op, wait states since, line index)
    for i, ln in enumerate(lines):
        s = ln.strip()
        if not s or s.startswith(";"):
            continue
        if s.endswith(":") or s.startswith("."):
            if s.startswith(".LBB") or (s.endswith(":") and not s.startswith(".")):
                pending, recent = [], []
            continue
        op = s.split()[0]
        args = [a.strip().split()[0] if a.strip() else "" for a in s[len(op):].split(",")]
        if op.startswith("s_nop"):
            n = int(s.split()[1], 0) + 1
            pending = [(d, w + n, l) for d, w, l in pending]
            recent = [(d, w + n, l) for d, w, l in recent]
            continue
        reads = set()
        for a in args[1:]:
            reads |= _regs(a)
        if op.startswith("v_mfma"):
            for d, w, l in recent:
                if d & reads and w < VALU_TO_MFMA_WAITS:
                    problems.append(f"line {i}: MFMA reads v{min(d & reads)} written by VALU at line {l} "
                                    f"after {w} wait states")
            dst = _regs(args[0]) if args else set()
            # reading the previous MFMA's result as A/B is a hazard; as the tied accumulator it is not
            srcab = (_regs(args[1]) if len(args) > 1 else set()) | (_regs(args[2]) if len(args) > 2 else set())
            for d, w, l in pending:
                if d & srcab and w < MFMA_RESULT_WAITS:
                    problems.append(f"line {i}: MFMA reads v{min(d & srcab)} as A/B, written by MFMA at line {l} "
                                    f"after {w} wait states")
            pending = [(d, w + 1, l) for d, w, l in pending if not (d & dst)]
            recent = [(d, w + 1, l) for d, w, l in recent if w < 8]
            if dst:
                pending.append((dst, 0, i))
            continue
        for d, w, l in pending:
            if d & reads and w < MFMA_RESULT_WAITS:
                problems.append(f"line {i}: '{s[:60]}' reads v{min(d & reads)} {w} wait states after the MFMA "
                                f"at line {l}")
        pending = [(d, w + 1, l) for d, w, l in pending]
        recent = [(d, w + 1, l) for d, w, l in recent if w < 8]
        if op.startswith("v_") and args:
            recent.append((_regs(args[0]), 0, i))
    return problems


def block_depths(lines: list[str]) -> list[int]:
    """Loop depth of every line, from the compiler's block annotations: a label line (`.LBBx_y:` or
    `; %bb.N:`) starts a block, `Depth=N` on it or on the comment lines right after it (a loop
    header's own `=> This Loop Header: Depth=N`) gives the block's depth, no annotation means 0."""
    depth, out, in_header = 0, [], False
    for ln in lines:
        s = ln.strip()
        if re.match(r"^(\.LBB\d+_\d+:|; %bb\.\d+:)", s):
            m = re.search(r"Depth=(\d+)", s)
            depth = int(m.group(1)) if m else 0
            in_header = True
        elif in_header and s.startswith(";"):
            m = re.search(r"Loop Header: Depth=(\d+)", s)
            if m:
                depth = int(m.group(1))
        else:
            in_header = False
        out.append(depth)
    return out


def loop_spills(lines: list[str]) -> list[str]:
    """Scratch accesses inside the hot loop: the loop blocks at the deepest level that holds MFMAs (the
    tile loop), and any loop nested in them.  Spills before or after that loop cost once per segment."""
    depths = block_depths(lines)
    hot = 0
    for ln, d in zip(lines, depths):
        if d and ln.strip().startswith("v_mfma"):
            hot = max(hot, d)
    if not hot:
        return []
    return [f"line {i}: '{ln.strip()[:60]}' inside the innermost loop"
            for i, (ln, d) in enumerate(zip(lines, depths)) if d >= hot and ln.strip().startswith("scratch_")]


def lint(asm_text: str, name_part: str = "mla_split_kv") -> dict:
    """{function name: [problems]} for every function whose name contains name_part."""
    out = {}
    for chunk in re.split(r"\n(?=_Z\w+:)", asm_text):
        name = chunk.split(":", 1)[0]
        if name_part in name:
            lines = chunk.split("\n")
            out[name] = lint_function(lines) + loop_spills(lines)
    return out
