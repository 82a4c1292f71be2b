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
        self._prune_constant_vcc_branches(labels)
        self.pred = [[] for _ in range(n)]
        for i, nxt in enumerate(self.succ):
            for j in nxt:
                self.pred[j].append(i)

    def _prune_constant_vcc_branches(self, labels):
        """The compiler's if/else flow blocks set a 64-bit SGPR to -1 or 0
        (s_mov_b64), derive VCC from it (s_andn2_b64 vcc, exec, X) and branch
        on VCC.  A forward constant propagation of those SGPRs over the
        control-flow graph finds where X is -1 on every path, so VCC is 0 and
        the branch can go one way only; the other edge is dropped."""
        n = len(self.ins)
        tracked = {_operands(t)[2] for t in self.ins
                   if t.startswith("s_andn2_b64") and _operands(t)[:2] == ["vcc", "exec"]}
        if not tracked:
            return
        UNK = object()

        def transfer(state, t):
            ops = _operands(t)
            if not ops:
                return state
            d = ops[0]
            if t.startswith("s_mov_b64") and d in tracked and ops[1] in ("-1", "0"):
                state = dict(state)
                state[d] = int(ops[1])
                return state
            written = _sregs(d)
            hit = [r for r in state if _sregs(r) & written]
            if hit:
                state = dict(state)
                for r in hit:
                    state[r] = UNK
            return state

        # every instruction without a predecessor starts a function: no
        # constant known there
        has_pred = [False] * n
        for nxt in self.succ:
            for j in nxt:
                has_pred[j] = True
        ins_state = [None] * n
        work = []
        for i in range(n):
            if not has_pred[i]:
                ins_state[i] = {}
                work.append(i)
        while work:
            i = work.pop()
            out = transfer(ins_state[i], self.ins[i])
            for j in self.succ[i]:
                cur = ins_state[j]
                if cur is None:
                    new = dict(out)
                else:
                    new = {r: (v if cur.get(r, UNK) == v and r in cur else UNK) for r, v in out.items()}
                    for r in cur:
                        if r not in out:
                            new[r] = UNK
                if new != cur:
                    ins_state[j] = new
                    work.append(j)
        for i, t in enumerate(self.ins):
            if not t.startswith(("s_cbranch_vccz", "s_cbranch_vccnz")) or i == 0:
                continue
            prev = self.ins[i - 1]
            ops = _operands(prev)
            if not (prev.startswith("s_andn2_b64") and ops[:2] == ["vcc", "exec"]) or ins_state[i - 1] is None:
                continue
            # only X = -1 is certain (VCC = 0); X = 0 gives VCC = EXEC, which
            # can be 0 in divergent code
            if ins_state[i - 1].get(ops[2], UNK) != -1:
                continue
            taken = t.startswith("s_cbranch_vccz")
            target = labels[t.split()[1]]
            self.succ[i] = [target] if taken else [i + 1]

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
    between the issue of their load and the wave's first `s_waitcnt vmcnt`
    (before the issue they still hold an earlier value, which may be read or
    moved)."""
    load_re = r"global_load_dwordx4 v\[\d+:\d+\], v\[\d+:\d+\], off"
    bad, n = [], 0
    for m in re.finditer(r"^(_ZN4sdpa\w+):", text, re.M):
        body = _instructions(text[m.end():text.index(".Lfunc_end", m.end())])
        loads = [k for k, u in enumerate(body) if re.match(load_re, u)]
        waits = [k for k, u in enumerate(body) if u.startswith("s_waitcnt") and "vmcnt" in u]
        if not loads or not waits:
            continue
        first_wait = waits[0]
        in_flight = set()
        for u in body[loads[0]:first_wait]:
            if re.match(load_re, u):
                if _vregs(_operands(u)[1]) & in_flight:
                    bad.append(f"{m.group(1)[:60]}: {u} addressed by a load in flight")
                in_flight |= _vregs(_operands(u)[0])
                n += 1
                continue
            touched = set()
            for o in _operands(u):
                touched |= _vregs(o)
            if touched & in_flight:
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


def global_loads_waited(text):
    """Every global load into registers (the inline-asm ones the compiler does
    not count included): on every path, nothing touches its destination
    registers (a use, a copy, a spill) before the next `s_waitcnt` on vmcnt.
    The kernels wait for their uncounted loads with explicit counts placed
    right before the first use; this scan checks that the compiler put no
    instruction on those registers ahead of that wait (the counts themselves
    follow the issue order the code fixes)."""
    prog = _Program(text)
    bad, n = [], 0
    for i, t in enumerate(prog.ins):
        if not t.startswith("global_load") or t.startswith("global_load_lds"):
            continue
        dst = _vregs(_operands(t)[0])
        if not dst:
            continue
        n += 1
        seen = set()
        stack = list(prog.succ[i])
        while stack:
            j = stack.pop()
            if j in seen:
                continue
            seen.add(j)
            u = prog.ins[j]
            if u.startswith("s_waitcnt") and "vmcnt" in u:
                continue
            touched = set()
            for o in _operands(u):
                touched |= _vregs(o)
            if touched & dst:
                bad.append(f"{t} -> {u} before any vmcnt wait")
                continue
            stack.extend(prog.succ[j])
    return bad, n
