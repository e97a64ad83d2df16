"""Static check of the generated instruction-scheduled blocks
(tiled_online_softmax_fwd_amd/csrc/*_pipe_asm.h), independent of the
generators' own bookkeeping.

The block text of each macro is parsed into instructions, a control-flow graph
is built from its labels and branches (loops included), and a forward dataflow
analysis runs to a fixpoint.  The state at each point holds, per vector
register, the wait states since its last write by a matrix op, by a vector op
and by a transcendental, and since its last read as a matrix op's
accumulator input; the ordered list of LDS reads still in flight; and the wait
states since the last writes of VCC and M0.  Joins take the worst case (the
smallest distances); differing in-flight LDS lists at a join are an error.

Rules checked (wait states = instructions issued in between, s_nop N counting
N + 1):
  * a register written by an LDS read is neither read nor written before an
    s_waitcnt lgkmcnt(n) has retired that read (LDS reads retire in order);
  * matrix-op result -> vector read or write of any of its registers: XDL_WS,
    except the accumulator chain into the next matrix op on the same range;
  * matrix-op read or write of a register written by a vector op (or a
    transcendental): VALU_MFMA_WS;
  * transcendental result -> vector read: TRANS_WS;
  * vector write of a register a matrix op still reads as accumulator input:
    XDL_WS;
  * vector write of VCC -> read of VCC; vector write -> permlane read of that
    register: SGPR_WS;
  * M0 write -> LDS DMA (global_load_lds): at least one wait state;
  * at the block's end no LDS read is in flight and every matrix-op result is
    at least XDL_WS old (the compiler's code after the block reads them).
At entry every register is taken as just written by a vector op (the
compiler's code before the block may have moved an input into it).
"""
import re

XDL_WS = 12
VALU_MFMA_WS = 2
TRANS_WS = 1
SGPR_WS = 2
FAR = 64                       # distances saturate here

_TRANS = ("v_exp_", "v_log_", "v_rcp_", "v_rsq_", "v_sqrt_", "v_sin_", "v_cos_")


def macros(text):
    """{macro name: [instruction or label lines]} of the *_ASM_* macros."""
    out = {}
    for name, body in re.findall(r'#define (ATTN_\w+_ASM_\w+) \\\n(.*?)(?=\n#define|\Z)', text, re.S):
        out[name] = re.findall(r'"([^"\\]*)\\n"', body)
    return out


def _regs(tok):
    """VGPR numbers named by an operand token (modifiers stripped)."""
    tok = tok.strip().lstrip("-")
    m = re.fullmatch(r"v(\d+)", tok)
    if m:
        return {int(m.group(1))}
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return set()


class Ins:
    """One parsed instruction: what it reads and writes."""

    def __init__(self, text):
        self.text = text
        parts = text.split(None, 1)
        self.op = parts[0]
        rest = parts[1] if len(parts) > 1 else ""
        rest = re.sub(r"\s+offset:\d+", "", rest)
        ops = [o.strip() for o in rest.split(",")] if rest else []
        self.ops = ops
        self.reads, self.writes = set(), set()
        self.kind = "other"
        self.reads_vcc = self.writes_vcc = self.writes_m0 = self.lds_dma = False
        self.srcab, self.srcc, self.acc = set(), set(), None
        op = self.op
        if op == "s_nop":
            self.ws = int(ops[0]) + 1
        else:
            self.ws = 1
        if op.startswith("v_mfma"):
            self.kind = "mfma"
            self.writes = _regs(ops[0])
            self.srcab = _regs(ops[1]) | _regs(ops[2])
            self.srcc = _regs(ops[3])
            self.reads = self.srcab | self.srcc
            self.acc = (min(self.writes), len(self.writes))
        elif op.startswith("ds_read"):
            self.kind = "lds"
            self.writes = _regs(ops[0])
            self.reads = _regs(ops[1])
        elif op.startswith("global_load_lds"):
            self.kind = "dma"
            self.lds_dma = True
            self.reads = _regs(ops[0])
        elif op.startswith("v_"):
            self.kind = "trans" if op.startswith(_TRANS) else "valu"
            if op.startswith("v_cmp"):
                self.writes_vcc = ops[0] == "vcc"
                for o in ops[1:]:
                    self.reads |= _regs(o)
            else:
                self.writes = _regs(ops[0])
                for o in ops[1:]:
                    self.reads |= _regs(o)
                if "vcc" in ops[1:]:
                    self.reads_vcc = True
                if op.startswith("v_dot2c") or op.startswith("v_permlane"):
                    self.reads |= self.writes
                if op.startswith("v_permlane"):
                    self.writes |= _regs(ops[1])
                    self.kind = "perm"
        elif op.startswith("s_"):
            self.kind = "salu"
            if ops and ops[0] == "m0":
                self.writes_m0 = True
            if "vcc" in ops[1:]:
                self.reads_vcc = True


class State:
    def __init__(self):
        self.xdl = {}       # reg -> (distance, accumulator range of the writer)
        self.valu = {}      # reg -> distance since a vector (or transcendental) write
        self.trans = {}     # reg -> distance since a transcendental write
        self.srcc = {}      # reg -> distance since a matrix op read it as accumulator input
        self.lds = ()       # in-flight LDS reads, oldest first: frozensets of destination registers
        self.vcc = FAR
        self.m0 = FAR

    def copy(self):
        s = State()
        s.xdl, s.valu, s.trans, s.srcc = dict(self.xdl), dict(self.valu), dict(self.trans), dict(self.srcc)
        s.lds, s.vcc, s.m0 = self.lds, self.vcc, self.m0
        return s

    def key(self):
        return (tuple(sorted(self.xdl.items())), tuple(sorted(self.valu.items())), tuple(sorted(self.trans.items())),
                tuple(sorted(self.srcc.items())), self.lds, self.vcc, self.m0)

    def advance(self, n):
        for d in (self.valu, self.trans, self.srcc):
            for r in list(d):
                d[r] = min(FAR, d[r] + n)
                if d[r] >= FAR:
                    del d[r]
        for r in list(self.xdl):
            dist, rg = self.xdl[r]
            if dist + n >= FAR:
                del self.xdl[r]
            else:
                self.xdl[r] = (dist + n, rg)
        self.vcc = min(FAR, self.vcc + n)
        self.m0 = min(FAR, self.m0 + n)


def join(a, b, where, errors):
    if a is None:
        return b.copy()
    s = State()
    for name in ("valu", "trans", "srcc"):
        da, db = getattr(a, name), getattr(b, name)
        getattr(s, name).update({r: min(da.get(r, FAR), db.get(r, FAR)) for r in set(da) | set(db)})
    for r in set(a.xdl) | set(b.xdl):
        xa, xb = a.xdl.get(r, (FAR, None)), b.xdl.get(r, (FAR, None))
        rg = xa[1] if xa[1] == xb[1] or xb[0] >= FAR else (xb[1] if xa[0] >= FAR else None)
        s.xdl[r] = (min(xa[0], xb[0]), rg)
    if a.lds != b.lds:
        errors.append(f"{where}: paths join with different LDS reads in flight")
    s.lds = a.lds if len(a.lds) >= len(b.lds) else b.lds
    s.vcc, s.m0 = min(a.vcc, b.vcc), min(a.m0, b.m0)
    return s


def step(ins, st, where, errors):
    """Check `ins` against the state before it; return the state after it."""
    def err(msg):
        errors.append(f"{where}: {ins.text}: {msg}")

    pending = set().union(*st.lds) if st.lds else set()
    if ins.kind in ("mfma", "valu", "trans", "perm", "lds", "dma"):
        for r in sorted((ins.reads | ins.writes) & pending):
            err(f"v{r} is the destination of an LDS read still in flight")
            break
    if ins.kind == "lds":
        for r in sorted(ins.writes):
            if r in st.xdl and st.xdl[r][0] < XDL_WS:
                err(f"v{r} written by a matrix op {st.xdl[r][0]} wait states before (needs {XDL_WS})")
                break
            if r in st.srcc and st.srcc[r] < XDL_WS:
                err(f"v{r} is read as accumulator input by a matrix op {st.srcc[r]} wait states before")
                break
    if ins.kind in ("valu", "trans", "perm"):
        for r in sorted(ins.reads | ins.writes):
            if r in st.xdl and st.xdl[r][0] < XDL_WS:
                err(f"v{r} written by a matrix op {st.xdl[r][0]} wait states before (needs {XDL_WS})")
                break
        for r in sorted(ins.reads):
            if r in st.trans and st.trans[r] < TRANS_WS:
                err(f"v{r} written by a transcendental {st.trans[r]} wait states before (needs {TRANS_WS})")
                break
        for r in sorted(ins.writes):
            if r in st.srcc and st.srcc[r] < XDL_WS:
                err(f"v{r} is read as accumulator input by a matrix op {st.srcc[r]} wait states before")
                break
        if ins.reads_vcc and st.vcc < SGPR_WS:
            err(f"VCC written {st.vcc} wait states before (needs {SGPR_WS})")
        if ins.kind == "perm":
            for r in sorted(ins.reads):
                if r in st.valu and st.valu[r] < SGPR_WS:
                    err(f"permlane input v{r} written {st.valu[r]} wait states before (needs {SGPR_WS})")
                    break
    if ins.kind == "mfma":
        for r in sorted(ins.reads | ins.writes):
            if r in st.xdl and st.xdl[r][0] < XDL_WS:
                chain = (st.xdl[r][1] == ins.acc and r in ins.srcc and r not in ins.srcab)
                if not chain:
                    err(f"v{r} written by a matrix op {st.xdl[r][0]} wait states before (needs {XDL_WS})")
                    break
        for r in sorted(ins.reads):
            if r in st.valu and st.valu[r] < VALU_MFMA_WS:
                err(f"v{r} written by a vector op {st.valu[r]} wait states before (needs {VALU_MFMA_WS})")
                break
    if ins.kind == "salu" and ins.reads_vcc and st.vcc < SGPR_WS:
        err(f"VCC written {st.vcc} wait states before (needs {SGPR_WS})")
    if ins.lds_dma and st.m0 < 1:
        err("M0 written right before an LDS DMA")

    st = st.copy()
    if ins.op == "s_waitcnt":
        m = re.search(r"lgkmcnt\((\d+)\)", ins.text)
        if m:
            n = int(m.group(1))
            st.lds = st.lds[len(st.lds) - n:] if n < len(st.lds) else st.lds
            if n == 0:
                st.lds = ()
    st.advance(ins.ws)
    # the instruction's own effects take place at distance 0
    if ins.kind == "mfma":
        for r in ins.writes:
            st.xdl[r] = (0, ins.acc)
            st.valu.pop(r, None)
            st.trans.pop(r, None)
        for r in ins.srcc:
            st.srcc[r] = 0
    elif ins.kind in ("valu", "trans", "perm"):
        for r in ins.writes:
            st.valu[r] = 0
            st.xdl.pop(r, None)
            st.srcc.pop(r, None)
            if ins.kind == "trans":
                st.trans[r] = 0
            else:
                st.trans.pop(r, None)
        if ins.writes_vcc:
            st.vcc = 0
    elif ins.kind == "lds":
        st.lds = st.lds + (frozenset(ins.writes),)
        for r in ins.writes:
            st.xdl.pop(r, None)
            st.valu.pop(r, None)
            st.trans.pop(r, None)
    if ins.writes_m0:
        st.m0 = 0
    return st


def check(lines, name="block"):
    """Errors (list of strings) of one block's instruction lines."""
    nodes, labels = [], {}
    for ln in lines:
        if re.fullmatch(r"\d+:", ln):
            labels.setdefault(ln[:-1], []).append(len(nodes))
        else:
            nodes.append(Ins(ln))

    def target(i, tok):
        lab, d = tok[:-1], tok[-1]
        idx = labels.get(lab, [])
        if d == "f":
            cand = [j for j in idx if j > i]
            return min(cand) if cand else None
        cand = [j for j in idx if j <= i]
        return max(cand) if cand else None

    succ = []
    errors = []
    for i, ins in enumerate(nodes):
        nxt = [i + 1]
        if ins.op in ("s_cbranch_scc1", "s_cbranch_scc0", "s_branch"):
            t = target(i, ins.ops[0])
            if t is None:
                errors.append(f"{name}: {ins.text}: branch target not found")
                t = len(nodes)
            nxt = [t] if ins.op == "s_branch" else [i + 1, t]
        succ.append(nxt)

    entry = State()
    for r in range(512):
        entry.valu[r] = 0
    state_in = [None] * (len(nodes) + 1)
    state_in[0] = entry
    work = [0]
    seen_err = set()
    while work:
        i = work.pop()
        if i >= len(nodes):
            continue
        errs = []
        out = step(nodes[i], state_in[i], f"{name}[{i}]", errs)
        for e in errs:
            if e not in seen_err:
                seen_err.add(e)
                errors.append(e)
        for j in succ[i]:
            new = join(state_in[j], out, f"{name}[{j}]", errors) if state_in[j] is not None else out.copy()
            if state_in[j] is None or new.key() != state_in[j].key():
                state_in[j] = new
                work.append(j)
    end = state_in[len(nodes)]
    if end is None:
        errors.append(f"{name}: the end of the block is unreachable")
    else:
        if end.lds:
            errors.append(f"{name}: LDS reads in flight at the end of the block")
        late = sorted(r for r, (d, _) in end.xdl.items() if d < XDL_WS)
        if late:
            errors.append(f"{name}: matrix-op results v{late[0]}.. younger than {XDL_WS} wait states at the end")
    return errors
