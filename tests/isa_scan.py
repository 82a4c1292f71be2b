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


def mfma_result_waits(text, need=18):
    """After an MFMA, no other instruction may touch its destination registers
    for `need` wait states (the hand-ordered kernel drains explicitly)."""
    ins = _instructions(text)
    bad, n = [], 0
    for i, t in enumerate(ins):
        if not t.startswith("v_mfma"):
            continue
        n += 1
        dst = _vregs(_operands(t)[0])
        ws = 0
        for u in ins[i + 1:i + 200]:
            if u.startswith("s_nop"):
                ws += _waits(u)
                continue
            touched = set()
            for o in _operands(u):
                touched |= _vregs(o)
            if touched & dst:
                if not u.startswith("v_mfma") and ws < need:
                    bad.append(f"{t} -> {u} after {ws} wait states")
                break
            ws += 1
    return bad, n


def valu_to_mfma_inputs(text, need=2):
    """A vector write of a VGPR followed by an MFMA reading it as its A or B
    operand needs `need` wait states."""
    ins = _instructions(text)
    bad, n = [], 0
    for i, t in enumerate(ins):
        if not t.startswith("v_mfma"):
            continue
        n += 1
        ops = _operands(t)
        src = _vregs(ops[1]) | _vregs(ops[2])
        ws = 0
        for u in reversed(ins[max(0, i - 8):i]):
            if ws >= need:
                break
            if u.startswith("s_nop"):
                ws += _waits(u)
                continue
            if u.startswith("v_") and not u.startswith(("v_mfma", "v_readfirstlane", "v_readlane")):
                ops_u = _operands(u)
                if ops_u and _vregs(ops_u[0]) & src:
                    bad.append(f"{u} -> {t} after {ws} wait states")
            ws += 1
    return bad, n


_TRANS = ("v_exp_", "v_log_", "v_rcp_", "v_rsq_", "v_sqrt_", "v_sin_", "v_cos_")


def trans_result_use(text, need=1):
    """A vector instruction reading the result of a transcendental one (v_exp
    and the like) needs `need` wait states after it."""
    ins = _instructions(text)
    bad, n = [], 0
    for i, t in enumerate(ins):
        if not t.startswith(_TRANS):
            continue
        n += 1
        dst = _vregs(_operands(t)[0])
        ws = 0
        for u in ins[i + 1:i + 4]:
            if ws >= need:
                break
            if u.startswith("s_nop"):
                ws += _waits(u)
                continue
            if u.startswith("v_"):
                srcs = set()
                for o in _operands(u)[1:]:
                    srcs |= _vregs(o)
                if srcs & dst:
                    bad.append(f"{t} -> {u} after {ws} wait states")
            ws += 1
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
