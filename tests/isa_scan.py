"""Scans of gfx950 assembly for the hazards the hand-ordered kernels handle
themselves (the compiler's hazard recognizer does not see inside inline asm).

Each function takes the text of a `.s` file and returns a list of findings
(empty when clean) plus the number of sites it checked.  Wait states count one
per instruction and N+1 per `s_nop N`.
"""
import re

_SKIP = (".", ";")


def _instructions(text):
    out = []
    for line in text.split("\n"):
        t = line.split(";")[0].strip()
        if not t or t.startswith(_SKIP) or t.endswith(":"):
            continue
        out.append(t)
    return out


def _vregs(tok):
    tok = tok.strip().rstrip(",")
    m = re.match(r"[va]\[(\d+):(\d+)\]$", tok)
    if m:
        return {(tok[0], i) for i in range(int(m.group(1)), int(m.group(2)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _sregs(tok):
    tok = tok.strip().rstrip(",")
    m = re.match(r"s\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _operands(ins):
    """Operands of an instruction, without trailing modifiers (offset:, sc0 ...)."""
    parts = ins.split(None, 1)
    if len(parts) < 2:
        return []
    return [o.split()[0] for o in parts[1].split(",") if o.strip()]


def _waits(ins):
    return int(ins.split()[1]) + 1 if ins.startswith("s_nop") else 1


class _Program:
    """The instructions of an assembly text with their control-flow edges
    (fall-through, `s_branch`, both ways of `s_cbranch_*`), so that a hazard
    scan follows every path: a register copy the compiler puts at the top of
    a branch target is reached through the jump, not through the lines that
    precede it in the file."""

    def __init__(self, text):
        self.ins, labels = [], {}
        for line in text.split("\n"):
            t = line.split(";")[0].strip()
            if not t:
                continue
            if t.endswith(":"):
                labels[t[:-1]] = len(self.ins)
                continue
            if t.startswith("."):
                continue
            self.ins.append(t)
        n = len(self.ins)
        self.succ = []
        for i, t in enumerate(self.ins):
            if t.startswith("s_branch "):
                nxt = [labels[t.split()[1]]]
            elif t.startswith("s_cbranch_"):
                nxt = [i + 1, labels[t.split()[1]]]
            elif t.startswith(("s_endpgm", "s_setpc", "s_trap")):
                nxt = []
            else:
                nxt = [i + 1]
            self.succ.append([j for j in nxt if j < n])
        self.pred = [[] for _ in range(n)]
        for i, nxt in enumerate(self.succ):
            for j in nxt:
                self.pred[j].append(i)

    def walk(self, i, need, forward, visit):
        """Calls visit(j, ws) for every instruction j reachable from i (after
        it, or before it when not forward) within fewer than `need` wait
        states, ws being the wait states between the two.  visit returns True
        to stop the path at j."""
        edges = self.succ if forward else self.pred
        best = {}
        stack = [(j, 0) for j in edges[i]]
        while stack:
            j, ws = stack.pop()
            if ws >= need or best.get(j, need) <= ws:
                continue
            best[j] = ws
            u = self.ins[j]
            if u.startswith("s_nop"):
                step = _waits(u)
            else:
                if visit(j, ws):
                    continue
                step = 1
            stack.extend((k, ws + step) for k in edges[j])


def mfma_result_waits(text, need=18):
    """After an MFMA, no other instruction may touch its destination registers
    for `need` wait states (the hand-ordered kernel drains explicitly), on any
    path."""
    prog = _Program(text)
    bad, n = [], 0
    for i, t in enumerate(prog.ins):
        if not t.startswith("v_mfma"):
            continue
        n += 1
        dst = _vregs(_operands(t)[0])

        def visit(j, ws):
            u = prog.ins[j]
            touched = set()
            for o in _operands(u):
                touched |= _vregs(o)
            if touched & dst:
                if not u.startswith("v_mfma"):
                    bad.append(f"{t} -> {u} after {ws} wait states")
                return True
            return False

        prog.walk(i, need, True, visit)
    return bad, n


def valu_to_mfma_inputs(text, need=2):
    """A vector write of a VGPR followed by an MFMA reading it (as its A, B or
    C operand) needs `need` wait states, on any path into the MFMA."""
    prog = _Program(text)
    bad, n = [], 0
    for i, t in enumerate(prog.ins):
        if not t.startswith("v_mfma"):
            continue
        n += 1
        ops = _operands(t)
        src = _vregs(ops[1]) | _vregs(ops[2]) | (_vregs(ops[3]) if len(ops) > 3 else set())

        def visit(j, ws):
            u = prog.ins[j]
            if u.startswith("v_") and not u.startswith(("v_mfma", "v_readfirstlane", "v_readlane")):
                ops_u = _operands(u)
                if ops_u and _vregs(ops_u[0]) & src:
                    bad.append(f"{u} -> {t} after {ws} wait states")
            return False

        prog.walk(i, need, False, visit)
    return bad, n


_TRANS = ("v_exp_", "v_log_", "v_rcp_", "v_rsq_", "v_sqrt_", "v_sin_", "v_cos_")


def trans_result_use(text, need=1):
    """A vector instruction reading the result of a transcendental one (v_exp
    and the like) needs `need` wait states after it, on any path."""
    prog = _Program(text)
    bad, n = [], 0
    for i, t in enumerate(prog.ins):
        if not t.startswith(_TRANS):
            continue
        n += 1
        dst = _vregs(_operands(t)[0])

        def visit(j, ws):
            u = prog.ins[j]
            if u.startswith("v_"):
                srcs = set()
                for o in _operands(u)[1:]:
                    srcs |= _vregs(o)
                if srcs & dst:
                    bad.append(f"{t} -> {u} after {ws} wait states")
            return False

        prog.walk(i, need, True, visit)
    return bad, n


def lds_dma_scalar_base(text):
    """A direct global->LDS load with an SGPR base needs five wait states after
    a vector instruction (v_readfirstlane) writes that base, and one after the
    M0 write that gives it its LDS address."""
    ins = _instructions(text)
    bad, n = [], 0
    for i, t in enumerate(ins):
        if not t.startswith("global_load_lds"):
            continue
        ops = _operands(t)
        m0_ws = None
        ws = 0
        base = _sregs(ops[1]) if len(ops) > 1 else set()
        n += bool(base)
        for u in reversed(ins[max(0, i - 12):i]):
            if u.startswith("s_nop"):
                ws += _waits(u)
                continue
            ops_u = _operands(u)
            if m0_ws is None and ops_u and ops_u[0] == "m0":
                m0_ws = ws
            if base and u.startswith("v_") and ops_u and _sregs(ops_u[0]) & base and ws < 5:
                bad.append(f"{u} -> {t} after {ws} wait states")
            ws += 1
            if ws >= 6:
                break
        if m0_ws is not None and m0_ws < 1:
            bad.append(f"M0 written right before {t}")
    return bad, n


def untracked_loads_waited(text):
    """Registers filled by the asm 16-byte loads the compiler does not track
    (`global_load_dwordx4 v[..], v[..], off`) are neither read nor written
    before the wave's first `s_waitcnt vmcnt`."""
    bad, n = [], 0
    for m in re.finditer(r"^(_ZN4sdpa\w+):", text, re.M):
        body = _instructions(text[m.end():text.index(".Lfunc_end", m.end())])
        loads = [k for k, u in enumerate(body) if re.match(r"global_load_dwordx4 v\[\d+:\d+\], v\[\d+:\d+\], off", u)]
        waits = [k for k, u in enumerate(body) if u.startswith("s_waitcnt") and "vmcnt" in u]
        if not loads or not waits:
            continue
        first_wait = waits[0]
        regs = set()
        for k in loads:
            if k < first_wait:
                regs |= _vregs(_operands(body[k])[0])
                n += 1
        for u in body[loads[0] + 1:first_wait]:
            if re.match(r"global_load_dwordx4 v\[\d+:\d+\], v\[\d+:\d+\], off", u):
                continue
            touched = set()
            for o in _operands(u):
                touched |= _vregs(o)
            if touched & regs:
                bad.append(f"{m.group(1)[:60]}: {u} before the wait")
    return bad, n


def asm_lds_reads_waited(text):
    """The LDS reads written in inline asm (`ds_read_b128`, `ds_read_b64_tr_b16`
    and the like into explicit registers) are invisible to the compiler's wait
    count pass: on every path, no instruction may touch their destination
    registers before an `s_waitcnt lgkmcnt(N)` that covers the read (N at
    most the number of LDS instructions issued after it; LDS returns in
    order)."""
    prog = _Program(text)
    bad, n = [], 0
    for i, t in enumerate(prog.ins):
        if not t.startswith("ds_read"):
            continue
        dst = _vregs(_operands(t)[0])
        if not dst:
            continue
        n += 1
        seen = set()
        stack = [(j, 0) for j in prog.succ[i]]
        while stack:
            j, later = stack.pop()
            if (j, later) in seen or len(seen) > 20000:
                continue
            seen.add((j, later))
            u = prog.ins[j]
            m = re.search(r"lgkmcnt\((\d+)\)", u)
            if u.startswith("s_waitcnt") and m and int(m.group(1)) <= later:
                continue  # the read has landed on this path
            touched = set()
            for o in _operands(u):
                touched |= _vregs(o)
            if touched & dst:
                bad.append(f"{t} -> {u} with {later} LDS instructions after it and no covering wait")
                continue
            stack.extend((k, min(later + u.startswith("ds_"), 16)) for k in prog.succ[j])
    return bad, n
