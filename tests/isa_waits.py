"""Check of the LDS-read waits in the kernels' own gfx950 assembly.

The transposing LDS read of the NN kernels is issued as inline assembly, which
the compiler's wait-count pass does not see: nothing but the kernel's read
order (a compiler-visible LDS read after it, whose wait also covers it because
LDS operations complete in order) keeps its destination from being used early.
This module proves that property on the compiled code.  It walks every path of
each kernel's control-flow graph, keeping the queue of LDS operations still in
flight; ``s_waitcnt lgkmcnt(n)`` retires the oldest until at most n remain
(scalar-memory operations, which also count, are left out: that only retires
fewer, so the check stays conservative).  Any instruction other than a later
LDS read that names a VGPR/AGPR an in-flight LDS read will still write is
reported.
"""
from __future__ import annotations

import re

_LABEL = re.compile(r"^(\.LBB\w+|\w+):")
_REG = re.compile(r"(?<![\w.])([va])(?:\[(\d+):(\d+)\]|(\d+)\b)")
_LGKM = re.compile(r"lgkmcnt\((\d+)\)")
# the LDS/scalar counter is 4 bits: a wave has at most 15 such operations in
# flight (issue stalls beyond), which also bounds the states of the walk
MAX_LGKM = 15


def _regs(text: str) -> frozenset:
    out = set()
    for kind, lo, hi, one in _REG.findall(text):
        if one:
            out.add((kind, int(one)))
        else:
            out.update((kind, r) for r in range(int(lo), int(hi) + 1))
    return frozenset(out)


def kernel_bodies(asm: str, prefix: str) -> dict:
    """Map each function whose symbol starts with ``prefix`` to its lines
    (from its label to its .Lfunc_end label; a kernel may end in several
    s_endpgm)."""
    out, cur, name = {}, None, None
    for line in asm.splitlines():
        if cur is None:
            m = _LABEL.match(line)
            if m and m.group(1).startswith(prefix):
                name, cur = m.group(1), []
            continue
        if line.startswith(".Lfunc_end"):
            out[name] = cur
            cur = None
            continue
        cur.append(line)
    return out


def _blocks(lines):
    """Basic blocks as (label, [(line_no, mnemonic, operands)], successor labels)."""
    items = []  # ("label", name) or ("insn", no, mnem, ops)
    for no, raw in enumerate(lines):
        line = raw.split(";")[0].rstrip()
        m = _LABEL.match(line)
        if m:
            items.append(("label", m.group(1)))
            continue
        s = line.strip()
        if not s or s.startswith("."):
            continue
        mnem, _, ops = s.partition(" ")
        items.append(("insn", no, mnem, ops))
    blocks, cur_label, cur = [], "<entry>", []
    for it in items:
        if it[0] == "label":
            blocks.append([cur_label, cur, None])
            cur_label, cur = it[1], []
            continue
        cur.append(it[1:])
        mnem = it[2]
        if mnem.startswith("s_branch") or mnem.startswith("s_cbranch") or mnem == "s_endpgm":
            blocks.append([cur_label, cur, None])
            cur_label, cur = f"<after {it[1]}>", []
    if cur:
        blocks.append([cur_label, cur, None])
    index = {b[0]: i for i, b in enumerate(blocks)}
    for i, b in enumerate(blocks):
        last = b[1][-1] if b[1] else None
        nxt = [i + 1] if i + 1 < len(blocks) else []
        if last is None:
            b[2] = nxt
        elif last[1] == "s_endpgm":
            b[2] = []
        elif last[1] == "s_branch":
            b[2] = [index[last[2].strip()]]
        elif last[1].startswith("s_cbranch"):
            b[2] = [index[last[2].strip()]] + nxt
        else:
            b[2] = nxt
    return blocks


def check_kernel(lines) -> list:
    """Violations as (line index within the kernel, instruction text)."""
    blocks = _blocks(lines)
    seen, bad = set(), []
    work = [(0, ())]
    while work:
        bi, state = work.pop()
        if (bi, state) in seen:
            continue
        seen.add((bi, state))
        pending = list(state)  # oldest first: destination register sets
        _, insns, succ = blocks[bi]
        for no, mnem, ops in insns:
            if mnem == "s_waitcnt":
                m = _LGKM.search(ops)
                if m:
                    n = int(m.group(1))
                    while len(pending) > n:
                        pending.pop(0)
                continue
            if mnem.startswith("ds_"):
                is_read = "read" in mnem or mnem.startswith("ds_load")
                parts = [p.strip() for p in ops.split(",")]
                srcs = _regs(",".join(parts[1:] if is_read else parts))
                if any(srcs & p for p in pending):
                    bad.append((no, f"{mnem} {ops}"))
                pending.append(_regs(parts[0]) if is_read else frozenset())
                if len(pending) > MAX_LGKM:
                    pending.pop(0)
                continue
            used = _regs(ops)
            if used and any(used & p for p in pending):
                bad.append((no, f"{mnem} {ops}"))
        for s in succ:
            work.append((s, tuple(pending)))
    return sorted(set(bad))


def loop_vmcnt_zero(lines) -> int:
    """Number of waits for every outstanding vector-memory operation inside
    the kernel's main loops: the lines from a loop header label to the last
    branch (conditional or not) back to it, for loops that issue matrix-core
    instructions (a retry loop around an atomic has to wait for its result)."""
    count = 0
    for h, raw in enumerate(lines):
        m = _LABEL.match(raw)
        if not (m and "Loop Header" in raw):
            continue
        header = m.group(1)
        back = [i for i, l in enumerate(lines) if i > h and "branch" in l.split(";")[0]
                and l.split(";")[0].strip().endswith(header)]
        if not back:
            continue
        body = [l.split(";")[0].strip() for l in lines[h + 1:back[-1] + 1]]
        if not any(b.startswith("v_mfma") for b in body):
            continue
        for s in body:
            if s.startswith("s_waitcnt") and "vmcnt(0)" in s:
                count += 1
    return count


_ACC_STORE = re.compile(r"global_store_dwordx4 v\[\d+:\d+\], (a\[\d+:\d+\]), off\b")


def acc_store_sources(lines) -> list:
    """The accumulator registers each partial-sum store (inline assembly,
    storing straight from AGPRs) reads, in order.  Only stores inside inline
    assembly count (between the compiler's ;;#ASMSTART and ;;#ASMEND
    markers): a store the compiler emits itself from accumulator registers is
    padded by the compiler and may reuse its registers."""
    out, in_asm = [], False
    for l in lines:
        if ";;#ASMSTART" in l:
            in_asm = True
        elif ";;#ASMEND" in l:
            in_asm = False
        elif in_asm:
            m = _ACC_STORE.search(l.split(";")[0])
            if m:
                out.append(m.group(1))
    return out
