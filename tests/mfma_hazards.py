"""Static check of MFMA data hazards in gfx950 assembly (test infrastructure).

The kernels issue their MFMAs as inline assembly, which the compiler's
hazard recognizer does not look inside: the wait states an MFMA needs around
other instructions are placed by hand.  This module reads the assembly the
compiler writes (``hipcc -S --cuda-device-only``), follows each kernel's
control flow (basic blocks, branches, loops: a forward dataflow over the
blocks, merging the worst case of every predecessor) and reports three kinds
of hazard, with the distances counted in wait states (one per instruction,
N + 1 for ``s_nop N``):

* VALU_TO_MFMA: a VALU instruction writes a VGPR/AGPR that an MFMA then
  reads as srcA, srcB or srcC with fewer than ``VALU_TO_MFMA`` wait states in
  between.  CDNA3 ISA guide, "Manually inserted wait states": a VALU write
  of a VGPR read by a V_MFMA needs 2; the check asks for ``VALU_TO_MFMA``.
* LOAD_TO_MFMA: an LDS (ds_*) or vector-memory load writes a register that
  an MFMA reads while the load may still be outstanding, i.e. without an
  ``s_waitcnt`` whose lgkmcnt / vmcnt retires it (counters decrement in
  issue order; SMEM loads are counted with LDS as the hardware does).
* MFMA_RESULT: an instruction other than an MFMA accumulating into the same
  registers reads or writes an MFMA's destination within the MFMA's pass
  count + ``MFMA_RESULT_EXTRA`` wait states (the guide: XDL write followed by
  a VALU, VMEM or LDS access of the result needs passes + 3 for the
  multi-pass shapes; the check asks for one more), or an MFMA reads it as
  srcA/srcB that soon.  An MFMA reading the previous MFMA's destination as
  its own srcC with the same registers (an accumulation chain) is allowed
  back to back.
"""
from __future__ import annotations

import re
from collections import namedtuple

VALU_TO_MFMA = 2
MFMA_RESULT_EXTRA = 4

# passes of the MFMA shapes (gfx950): 16x16 blocks 8, 32x32 blocks 16, 4x4 2
def mfma_passes(opcode: str) -> int:
    m = re.search(r"_(\d+)x(\d+)x(\d+)", opcode)
    if not m:
        return 16
    return {4: 2, 16: 8, 32: 16}.get(int(m.group(1)), 16)


Hazard = namedtuple("Hazard", "kind function line text detail")
Instr = namedtuple("Instr", "op ops line text")

_REG = re.compile(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b")


def regs(operand: str):
    """VGPR/AGPR names ('v', n) / ('a', n) in an operand string."""
    out = set()
    for m in _REG.finditer(operand):
        if m.group(1):
            out.update((m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1))
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


def split_operands(rest: str):
    out, depth, cur = [], 0, ""
    for ch in rest:
        if ch == "[":
            depth += 1
        elif ch == "]":
            depth -= 1
        if ch == "," and depth == 0:
            out.append(cur.strip())
            cur = ""
        else:
            cur += ch
    if cur.strip():
        out.append(cur.strip())
    return out


def parse_functions(asm: str):
    """{function name: [label or Instr]} for every kernel in the file."""
    funcs, cur, name = {}, None, None
    for lineno, raw in enumerate(asm.splitlines(), 1):
        line = raw.split(";")[0].split("//")[0].rstrip()
        if not line.strip():
            continue
        m = re.match(r"^([A-Za-z_.$][\w.$]*):", line)
        if m:
            label = m.group(1)
            if not label.startswith("."):
                name, cur = label, []
                funcs[name] = cur
            elif cur is not None and label.startswith(".LBB"):
                cur.append(label)
            elif label.startswith(".Lfunc_end"):
                cur, name = None, None
            continue
        if cur is None:
            continue
        s = line.strip()
        if s.startswith("."):
            continue
        parts = s.split(None, 1)
        op = parts[0]
        ops = split_operands(parts[1]) if len(parts) > 1 else []
        cur.append(Instr(op, tuple(ops), lineno, s))
    return funcs


def classify(ins: Instr):
    """(kind, dests, sources): kind is mfma, valu, ds, vmem, smem, wait or other."""
    op, ops = ins.op, ins.ops
    allregs = [regs(o) for o in ops]
    if op.startswith("v_mfma") or op.startswith("v_smfmac"):
        return "mfma", allregs[0], allregs[1:4]
    if op.startswith("v_"):
        return "valu", (allregs[0] if allregs else set()), allregs[1:]
    if op.startswith("ds_"):
        returns = ("read" in op or "_rtn" in op or op in ("ds_swizzle_b32", "ds_permute_b32", "ds_bpermute_b32")
                   or op.startswith("ds_load"))
        if returns:
            return "ds", allregs[0], allregs[1:]
        return "ds", set(), allregs
    if op.split("_")[0] in ("buffer", "global", "flat", "scratch"):
        to_lds = "_lds" in op or any("lds" in o.split() for o in ops)
        if "load" in op and not to_lds:
            return "vmem", allregs[0], allregs[1:]
        return "vmem", set(), allregs
    if op.startswith("s_load") or op.startswith("s_buffer_load"):
        return "smem", set(), []
    if op == "s_waitcnt":
        return "wait", set(), []
    return "other", set(), []


def wait_states(ins: Instr) -> int:
    if ins.op == "s_nop":
        v = ins.ops[0]
        return (int(v, 0) if v else 0) + 1
    return 1


def parse_waitcnt(ins: Instr):
    """(vmcnt, lgkmcnt) limits of an s_waitcnt; None = not waited on."""
    text = " ".join(ins.ops)
    vm = re.search(r"vmcnt\((\d+)\)", text)
    lg = re.search(r"lgkmcnt\((\d+)\)", text)
    if not vm and not lg and re.fullmatch(r"\s*(0x0+|0)\s*", text or "0"):
        return 0, 0
    return (int(vm.group(1)) if vm else None), (int(lg.group(1)) if lg else None)


class State:
    """Dataflow state at a block boundary, as distances back from it."""
    __slots__ = ("valu", "mfma", "vm", "lgkm")

    def __init__(self):
        self.valu = {}   # reg -> wait states since its last VALU write
        self.mfma = {}   # reg -> (wait states since an MFMA wrote it, required, dest set)
        self.vm = []     # outstanding vector-memory ops, oldest first: sets of dest regs
        self.lgkm = []   # outstanding LDS/SMEM ops

    def __eq__(self, other):
        return (self.valu == other.valu and self.mfma == other.mfma and self.vm == other.vm
                and self.lgkm == other.lgkm)


def _merge_lists(a, b):
    n = max(len(a), len(b))
    a = [frozenset()] * (n - len(a)) + a
    b = [frozenset()] * (n - len(b)) + b
    return [x | y for x, y in zip(a, b)]


def merge(a: State, b: State) -> State:
    """The worst case of two predecessors: nearer writers, more loads outstanding."""
    s = State()
    s.valu = dict(a.valu)
    for k, v in b.valu.items():
        s.valu[k] = min(v, s.valu.get(k, v))
    s.mfma = dict(a.mfma)
    for k, v in b.mfma.items():
        if k not in s.mfma or v[0] - v[1] < s.mfma[k][0] - s.mfma[k][1]:
            s.mfma[k] = v
    s.vm = _merge_lists(a.vm, b.vm)
    s.lgkm = _merge_lists(a.lgkm, b.lgkm)
    return s


MAX_TRACK = 64  # distances beyond every requirement are dropped
MAX_OUTSTANDING = 64  # counter entries kept apart; older ones are merged into one


def _capped(lst):
    if len(lst) <= MAX_OUTSTANDING:
        return lst
    old = frozenset().union(*lst[:len(lst) - MAX_OUTSTANDING + 1])
    return [old] + lst[len(lst) - MAX_OUTSTANDING + 1:]


_CLASS = {}


def _classified(ins: Instr):
    c = _CLASS.get(ins)
    if c is None:
        kind, dests, srcs = classify(ins)
        src_all = frozenset().union(*srcs) if srcs else frozenset()
        srcC = frozenset(srcs[2]) if kind == "mfma" and len(srcs) > 2 else frozenset()
        extra = None
        if kind == "wait":
            extra = parse_waitcnt(ins)
        elif kind == "mfma":
            extra = mfma_passes(ins.op) + MFMA_RESULT_EXTRA
        c = (kind, frozenset(dests), src_all, srcC, wait_states(ins), extra)
        _CLASS[ins] = c
    return c


def run_block(entry: State, ins_list, report) -> State:
    """Applies a block to its entry state; returns the exit state.  Inside
    the block a clock counts wait states; a write is stored as the clock
    after it, so that a later instruction's distance is clock - stamp."""
    clock = 0
    valu = {r: -d for r, d in entry.valu.items()}
    mfma = {r: (-d, need, dset) for r, (d, need, dset) in entry.mfma.items()}
    vm, lgkm = list(entry.vm), list(entry.lgkm)
    for ins in ins_list:
        kind, dests, src_all, srcC, w, extra = _classified(ins)
        if kind == "mfma":
            for r in src_all:
                t = valu.get(r)
                if t is not None and clock - t < VALU_TO_MFMA:
                    report("VALU_TO_MFMA", ins, f"{r} written by a VALU {clock - t} wait states before")
                if vm and any(r in e for e in vm):
                    report("LOAD_TO_MFMA", ins, f"{r} loaded without a vmcnt wait")
                if lgkm and any(r in e for e in lgkm):
                    report("LOAD_TO_MFMA", ins, f"{r} loaded without a lgkmcnt wait")
                m = mfma.get(r)
                if m is not None:
                    dist = clock - m[0]
                    chain = r in srcC and m[2] == srcC and dests == srcC
                    if dist < m[1] and not chain:
                        report("MFMA_RESULT", ins, f"{r} written by an MFMA {dist} wait states before (needs {m[1]})")
        elif kind in ("valu", "ds", "vmem") and mfma:
            for r in src_all | dests:
                m = mfma.get(r)
                if m is not None and clock - m[0] < m[1]:
                    report("MFMA_RESULT", ins, f"{r} written by an MFMA {clock - m[0]} wait states before "
                           f"(needs {m[1]})")
        clock += w
        if kind == "wait":
            vmn, lgn = extra
            if vmn is not None and vmn < len(vm):
                vm = vm[len(vm) - vmn:] if vmn else []
            if lgn is not None and lgn < len(lgkm):
                lgkm = lgkm[len(lgkm) - lgn:] if lgn else []
        elif kind == "vmem":
            vm = _capped(vm + [dests])
        elif kind in ("ds", "smem"):
            lgkm = _capped(lgkm + [dests])
        if kind == "valu":
            for r in dests:
                valu[r] = clock
                mfma.pop(r, None)
        elif kind in ("ds", "vmem"):
            for r in dests:
                valu.pop(r, None)
                mfma.pop(r, None)
        elif kind == "mfma":
            for r in dests:
                mfma[r] = (clock, extra, dests)
                valu.pop(r, None)
    out = State()
    out.valu = {r: clock - t for r, t in valu.items() if clock - t < MAX_TRACK}
    out.mfma = {r: (clock - t, need, dset) for r, (t, need, dset) in mfma.items() if clock - t < MAX_TRACK}
    out.vm, out.lgkm = vm, lgkm
    return out


def blocks_of(body):
    """Basic blocks: (label, [Instr], successor labels, falls through)."""
    blocks, cur_label, cur = [], "__entry", []
    for item in body:
        if isinstance(item, str):
            blocks.append([cur_label, cur])
            cur_label, cur = item, []
        else:
            cur.append(item)
            if item.op.startswith("s_branch") or item.op.startswith("s_cbranch") or item.op in (
                    "s_endpgm", "s_setpc_b64"):
                blocks.append([cur_label, cur])
                cur_label, cur = f"__after{item.line}", []
    blocks.append([cur_label, cur])
    out = []
    for i, (label, ins) in enumerate(blocks):
        succ = []
        last = ins[-1] if ins else None
        uncond = last is not None and last.op in ("s_branch", "s_endpgm", "s_setpc_b64")
        if last is not None and (last.op.startswith("s_branch") or last.op.startswith("s_cbranch")):
            succ.append(last.ops[0])
        if not uncond and i + 1 < len(blocks):
            succ.append(blocks[i + 1][0])
        out.append((label, ins, succ))
    return out


def check_function(name, body):
    """Forward dataflow over the blocks to a fixpoint; the worklist takes the
    earliest block in program order first (close to reverse post-order)."""
    import heapq
    blocks = blocks_of(body)
    index = {b[0]: i for i, b in enumerate(blocks)}
    entry = [None] * len(blocks)
    entry[0] = State()
    found = {}
    work, queued = [0], {0}

    def report(kind, instr, detail):
        found.setdefault((kind, instr.line, detail), Hazard(kind, name, instr.line, instr.text, detail))

    while work:
        i = heapq.heappop(work)
        queued.discard(i)
        label, ins, succ = blocks[i]
        st = run_block(entry[i], ins, report)
        for s in succ:
            j = index.get(s)
            if j is None:
                continue
            new = st if entry[j] is None else merge(entry[j], st)
            if entry[j] is None or not new == entry[j]:
                entry[j] = new
                if j not in queued:
                    heapq.heappush(work, j)
                    queued.add(j)
    return list(found.values())


def check_asm(asm: str, name_filter=None):
    """Hazards in every function (or those whose name contains name_filter),
    and the number of MFMAs checked."""
    hazards, mfmas = [], 0
    for name, body in parse_functions(asm).items():
        if name_filter and name_filter not in name:
            continue
        mfmas += sum(1 for x in body if not isinstance(x, str) and x.op.startswith("v_mfma"))
        hazards += check_function(name, body)
    return hazards, mfmas
