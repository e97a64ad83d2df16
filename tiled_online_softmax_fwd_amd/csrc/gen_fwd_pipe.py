#!/usr/bin/env python3
"""Writes fwd_pipe_asm.h: the hand-scheduled steady-state loop of the 16-bit
forward kernel (d = 128, 256 query rows per workgroup, 64-key tiles).

The loop covers the key tiles that need no masking for any row of the
workgroup (full tiles at or below the causal diagonal of the workgroup's first
row).  It is a two-stage software pipeline over key tiles: iteration t issues
the 16 score products S(t+1) = K(t+1) Q^T beside the vector work of tile t (the
rescale of l and O, the exponentials of the first 16 keys), then the 16 products
O += V(t)^T P(t)^T beside the rest of tile t's exponentials and the row maximum
and reference step of S(t+1).  Per row, every operation and its order are the
ones of the compiler-scheduled tile body in fwd_kernel.h, so the results are
bitwise equal; only the interleaving of independent instructions differs.

Hazards between instructions inside the block (matrix-core results read by
vector instructions, transcendental results, VCC and permlane inputs) are
resolved by counting issued instructions and inserting s_nop where a required
distance is short; LDS reads are waited for with exact lgkmcnt values.

Run: python gen_fwd_pipe.py  (rewrites fwd_pipe_asm.h beside this file).
"""
import os
import sys

# ---------------------------------------------------------------- register map
O = 0            # v[0:63]    O^T accumulators, o[db] = v[16db : 16db+15]
SA, SB = 64, 96  # v[64:127]  score tiles of two consecutive key tiles (P in place)
Q = 128          # v[128:159] Q^T operand, qf[ks] = v[128+4ks : +3]
NKR, NVR = 5, 5  # ring slots of K and V^T operands (4 registers each)
KR = 160                     # K operand ring
VR = KR + 4 * NKR            # V^T operand ring
KADDR = VR + 4 * NVR         # 8: LDS byte address of this lane's K chunk, per ks
VADDR = KADDR + 8            # 4: LDS byte address of this lane's V^T pair, per db
KOFF = VADDR + 4             # 2: byte offset of this lane's K copy chunks in the next K tile
VOFF = KOFF + 2              # 2: the same for V
M, L, NMC, ALPHA, MT, T0, T1 = range(VOFF + 2, VOFF + 9)
NREG = T1 + 1    # v0 .. v[NREG-1] are owned by the block
# registers the loop writes with matrix or transcendental results (hazard
# state assumed fresh for these where control flow joins)
LOOP_WRITTEN = list(range(O, SB + 32)) + [M, L, NMC, ALPHA, MT, T0, T1]
# registers bound to operands of the asm statement (everything else it
# writes is declared clobbered)
OPERAND_REGS = set(range(O, O + 64)) | set(range(Q, Q + 32)) | set(range(KADDR, KADDR + 8)) | \
    set(range(VADDR, VADDR + 4)) | {KOFF, KOFF + 1, VOFF, VOFF + 1, M, L}

TILE_BYTES = 64 * 128 * 2       # one K or V tile in LDS and in HBM
KB_BYTES = 32 * 128 * 2         # 32 key rows
NI = 2                          # copy instructions per wave per tile

XDL_WS = 12      # 8-pass matrix op result -> vector read/write, or srcC WAR
VALU_MFMA_WS = 2  # vector write -> matrix op operand read
TRANS_WS = 1     # v_exp result -> vector read
SGPR_WS = 2      # vector write of VCC / permlane input -> read


def rng(b, n):
    return f"v[{b}:{b + n - 1}]"


class Emitter:
    """Instruction stream with wait-state counting, automatic s_nop for the
    hazards listed above, and exact lgkmcnt waits for LDS reads.

    Hazard state per register: the wait-state position of its last write by
    each kind of instruction ('xdl' matrix op with its vdst range, 'trans',
    'valu'), and of its last read as srcC by a matrix op.  At control-flow
    joins the state is the conservative merge of the incoming paths."""

    def __init__(self):
        self.lines = []
        self.pos = 0              # wait-state counter
        self.wr = {}              # vgpr -> {kind: (pos, range)}
        self.srcc = {}            # vgpr -> pos of last matrix op reading it as srcC
        self.vcc_pos = -100
        self.lds = []             # ids of outstanding LDS reads, oldest first
        self.next_id = 0

    # -- state handling at branches
    def snapshot(self):
        return {"wr": {r: dict(k) for r, k in self.wr.items()}, "srcc": dict(self.srcc),
                "vcc": self.vcc_pos, "lds": list(self.lds), "pos": self.pos}

    def restore(self, s):
        self.wr = {r: dict(k) for r, k in s["wr"].items()}
        self.srcc = dict(s["srcc"])
        self.vcc_pos = s["vcc"]
        self.lds = list(s["lds"])
        self.pos = s["pos"]

    def merge_with(self, other):
        """Join the current state with snapshot `other` (both paths end here)."""
        pos = max(self.pos, other["pos"])
        sh_a, sh_b = pos - self.pos, pos - other["pos"]
        wr = {}
        for src, sh in ((self.wr, sh_a), (other["wr"], sh_b)):
            for r, kinds in src.items():
                for kind, (p, rg) in kinds.items():
                    q = p + sh
                    cur = wr.setdefault(r, {})
                    if kind not in cur or q > cur[kind][0]:
                        cur[kind] = (q, rg)
        srcc = {}
        for src, sh in ((self.srcc, sh_a), (other["srcc"], sh_b)):
            for r, p in src.items():
                srcc[r] = max(srcc.get(r, -10**9), p + sh)
        assert len(self.lds) == len(other["lds"]), "paths leave different LDS reads in flight"
        self.wr, self.srcc, self.pos = wr, srcc, pos
        self.vcc_pos = max(self.vcc_pos + sh_a, other["vcc"] + sh_b)

    def assume_recent(self, regs):
        """Loop head / label reached from several places: treat every listed
        register as just written by a matrix op and by a transcendental, and
        VCC as just written (conservative)."""
        for r in regs:
            self.wr[r] = {"xdl": (self.pos - 1, None), "trans": (self.pos - 1, None)}
        self.vcc_pos = self.pos - 1

    def nop_to(self, need, since):
        have = self.pos - since - 1
        if have < need:
            k = need - have
            while k > 0:
                n = min(k, 8)
                self.lines.append(f"s_nop {n - 1}")
                self.pos += n
                k -= n

    def raw(self, text, ws=1):
        self.lines.append(text)
        self.pos += ws

    def label(self, text):
        self.lines.append(text)

    def _hazards(self, reads, writes, mfma=None):
        """mfma = (srcab_regs, srcc_base or None) for a matrix op."""
        need = []
        for r in set(reads) | set(writes):
            kinds = self.wr.get(r, {})
            if "xdl" in kinds:
                p, rg = kinds["xdl"]
                chain = (mfma is not None and mfma[1] is not None and rg == (mfma[1], 16)
                         and r in range(mfma[1], mfma[1] + 16) and r not in mfma[0])
                if not chain:
                    need.append((XDL_WS, p))
            if "trans" in kinds and r in reads:
                need.append((TRANS_WS, kinds["trans"][0]))
            if "valu" in kinds and mfma is not None and r in reads:
                need.append((VALU_MFMA_WS, kinds["valu"][0]))
        if mfma is None:
            for r in writes:
                if r in self.srcc:
                    need.append((XDL_WS, self.srcc[r]))
        for n, p in need:
            self.nop_to(n, p)

    def _wrote(self, regs, kind, rg=None):
        for r in regs:
            self.wr[r] = {kind: (self.pos - 1, rg)}
            if kind != "xdl":
                self.srcc.pop(r, None)

    def valu(self, text, reads=(), writes=(), trans=False, reads_vcc=False, writes_vcc=False, perm=False):
        self._hazards(reads, writes)
        if reads_vcc:
            self.nop_to(SGPR_WS, self.vcc_pos)
        if perm:
            for r in reads:
                kinds = self.wr.get(r, {})
                for kind in ("valu", "trans"):
                    if kind in kinds:
                        self.nop_to(SGPR_WS, kinds[kind][0])
        self.raw(text)
        self._wrote(writes, "trans" if trans else "valu")
        if writes_vcc:
            self.vcc_pos = self.pos - 1

    def salu_reads_vcc(self, text):
        self.nop_to(SGPR_WS, self.vcc_pos)
        self.raw(text)

    def mfma(self, op, dst, a, b, c):
        """dst, a, b: base registers; c: base register or None for zero."""
        srcab = set(range(a, a + 4)) | set(range(b, b + 4))
        reads = sorted(srcab) + ([] if c is None else list(range(c, c + 16)))
        writes = list(range(dst, dst + 16))
        self._hazards(reads, writes, mfma=(srcab, c))
        cs = "0" if c is None else rng(c, 16)
        self.raw(f"{op} {rng(dst, 16)}, {rng(a, 4)}, {rng(b, 4)}, {cs}")
        self._wrote(writes, "xdl", (dst, 16))
        if c is not None:
            for r in range(c, c + 16):
                self.srcc[r] = self.pos - 1

    def lds_read(self, text, dst, n):
        rid = self.next_id
        self.next_id += 1
        self._hazards((), list(range(dst, dst + n)))
        self.raw(text)
        self._wrote(range(dst, dst + n), "lds")
        self.lds.append(rid)
        return rid

    def wait_lds(self, rid):
        if rid not in self.lds:
            return
        k = len(self.lds) - 1 - self.lds.index(rid)
        assert k <= 15, "lgkmcnt field overflow"
        self.raw(f"s_waitcnt lgkmcnt({k})")
        self.lds = self.lds[self.lds.index(rid) + 1:]

    def wait_all_lds(self):
        if self.lds:
            self.raw("s_waitcnt lgkmcnt(0)")
            self.lds = []


class Op:
    def __init__(self, fn, cost, lo=-1, hi=99):
        self.fn, self.cost, self.lo, self.hi = fn, cost, lo, hi


def spread(ops, nslots):
    """Assign each op a slot in [0, nslots-1] (program order kept): slot s is
    filled up to the smallest even rate that still meets every later deadline
    (op.hi) and the overall average; an op is not placed before op.lo."""
    n = len(ops)
    eff = [nslots - 1] * (n + 1)
    for i in range(n - 1, -1, -1):
        eff[i] = min(ops[i].hi, eff[i + 1], nslots - 1)
    cum = [0.0]
    for o in ops:
        cum.append(cum[-1] + o.cost)
    slots = [None] * n
    i = 0
    for s in range(nslots):
        placed = cum[i]
        target = (cum[n] - placed) / (nslots - s)
        for j in range(i, n):
            target = max(target, (cum[j + 1] - placed) / (eff[j] - s + 1))
        fill = 0.0
        while i < n and ops[i].lo <= s and (eff[i] <= s or fill + ops[i].cost / 2 <= target):
            slots[i] = s
            fill += ops[i].cost
            i += 1
    assert i == n, "infeasible VALU placement"
    for o, s in zip(ops, slots):
        assert o.lo <= s <= o.hi
    return slots


class Gen:
    def __init__(self, f16):
        self.f16 = f16
        self.mf = "v_mfma_f32_32x32x16_f16" if f16 else "v_mfma_f32_32x32x16_bf16"
        self.cvt = "v_cvt_pk_f16_f32" if f16 else "v_cvt_pk_bf16_f32"
        self.dot = "v_dot2c_f32_f16 v{l}, 0x3c003c00, v{p}" if f16 else "v_dot2c_f32_bf16 v{l}, 0x3f803f80, v{p}"
        self.e = Emitter()

    # ------------------------------------------------------------ vector ops
    def chunk_ops(self, cur, kb, h):
        """P for keys 16*ks2 .. of tile in `cur`, ks2 = 2kb + h: 8 exponentials,
        rounded to the input type in place (P lands in the first 4 registers of
        the 8), and summed into l."""
        e, ops = self.e, []
        base = cur + 16 * kb + 8 * h
        for i in range(8):
            r = base + i
            ops.append(Op(lambda r=r: e.valu(f"v_fma_f32 v{r}, %[c], v{r}, v{NMC}", (r, NMC), (r,)), 4))
        for i in range(8):
            r = base + i
            ops.append(Op(lambda r=r: e.valu(f"v_exp_f32 v{r}, v{r}", (r,), (r,), trans=True), 8))
        for i in range(0, 8, 2):
            d, a, b = base + i // 2, base + i, base + i + 1
            ops.append(Op(lambda d=d, a=a, b=b: e.valu(f"{self.cvt} v{d}, v{a}, v{b}", (a, b), (d,)), 4))
        for i in range(4):
            p = base + i
            ops.append(Op(lambda p=p: e.valu(self.dot.format(l=L, p=p), (L, p), (L,)), 4))
        return ops

    def lscale_op(self):
        e = self.e
        return Op(lambda: e.valu(f"v_mul_f32 v{L}, v{L}, v{ALPHA}", (L, ALPHA), (L,)), 4)

    def rescale_ops(self):
        e, ops = self.e, []
        for r in range(O, O + 64):
            ops.append(Op(lambda r=r: e.valu(f"v_mul_f32 v{r}, v{ALPHA}, v{r}", (ALPHA, r), (r,)), 4))
        return ops

    def max_ops(self, nxt, kb, first):
        e, ops = self.e, []
        base = nxt + 16 * kb
        j0 = 0
        if first:
            ops.append(Op(lambda: e.valu(f"v_max_f32 v{MT}, v{base}, v{base + 1}", (base, base + 1), (MT,)), 4))
            j0 = 2
        for j in range(j0, 16, 2):
            a, b = base + j, base + j + 1
            ops.append(Op(lambda a=a, b=b: e.valu(f"v_max3_f32 v{MT}, v{MT}, v{a}, v{b}", (MT, a, b), (MT,)), 4))
        return ops

    def refstep_ops(self):
        """Row maximum across the two wave halves, then the reference step:
        moved = c (mt - m) > slack (0: the exact running maximum); m' = moved
        ? mt : m; alpha = moved ? exp2(c (m - m')) : 1; -m' c for the
        exponents."""
        e = self.e
        ops = [
            Op(lambda: e.valu(f"v_mov_b32 v{T0}, v{MT}", (MT,), (T0,)), 4),
            Op(lambda: e.valu(f"v_permlane32_swap_b32 v{MT}, v{T0}", (MT, T0), (MT, T0), perm=True), 4),
            Op(lambda: e.valu(f"v_max_f32 v{MT}, v{MT}, v{T0}", (MT, T0), (MT,)), 4),
            Op(lambda: e.valu(f"v_sub_f32 v{T0}, v{MT}, v{M}", (MT, M), (T0,)), 4),
            Op(lambda: e.valu(f"v_mul_f32 v{T0}, %[c], v{T0}", (T0,), (T0,)), 4),
            Op(lambda: e.valu(f"v_cmp_lt_f32 vcc, %[slack], v{T0}", (T0,), (), writes_vcc=True), 4),
            Op(lambda: e.valu(f"v_cndmask_b32 v{T1}, v{M}, v{MT}, vcc", (M, MT), (T1,), reads_vcc=True), 4),
            Op(lambda: e.salu_reads_vcc("s_mov_b64 %[moved], vcc"), 1),
            Op(lambda: e.valu(f"v_sub_f32 v{ALPHA}, v{M}, v{T1}", (M, T1), (ALPHA,)), 4),
            Op(lambda: e.valu(f"v_mul_f32 v{ALPHA}, %[c], v{ALPHA}", (ALPHA,), (ALPHA,)), 4),
            Op(lambda: e.valu(f"v_exp_f32 v{ALPHA}, v{ALPHA}", (ALPHA,), (ALPHA,), trans=True), 8),
            Op(lambda: e.valu(f"v_cndmask_b32 v{ALPHA}, 1.0, v{ALPHA}, vcc", (ALPHA,), (ALPHA,), reads_vcc=True), 4),
        ]
        return ops

    def refstep_commit_ops(self):
        """Second half of the reference step: m and -m c of the next tile.  It
        must follow the last exponent fma of the current tile (which reads
        -m c)."""
        e = self.e
        return [Op(lambda: e.valu(f"v_mov_b32 v{M}, v{T1}", (T1,), (M,)), 4),
                Op(lambda: e.valu(f"v_mul_f32 v{NMC}, %[c], -v{T1}", (T1,), (NMC,)), 4)]

    def offset_ops(self, which):
        e, ops = self.e, []
        for base in which:
            for i in range(NI):
                r = base + i
                ops.append(Op(lambda r=r: e.valu(f"v_add_u32 v{r}, 0x{TILE_BYTES:x}, v{r}", (r,), (r,)), 4))
        return ops

    # ------------------------------------------------------------ memory
    def barrier(self):
        self.e.wait_all_lds()
        self.e.raw("s_waitcnt vmcnt(0)")
        self.e.raw("s_barrier")

    def dma(self, kind, buf):
        dst, base, off = ("%[kdst]", "%[kbase]", KOFF) if kind == "k" else ("%[vdst]", "%[vbase]", VOFF)
        for i in range(NI):
            self.e.raw(f"s_add_u32 m0, {dst}, 0x{buf * TILE_BYTES + i * 1024:x}")
            self.e.raw("s_nop 0")
            self.e.raw(f"global_load_lds_dwordx4 v{off + i}, {base}")

    def k_read(self, idx, kbuf, slot):
        kb, ks = idx // 8, idx % 8
        d = KR + 4 * slot
        return self.e.lds_read(f"ds_read_b128 {rng(d, 4)}, v{KADDR + ks} offset:{kbuf * TILE_BYTES + kb * KB_BYTES}", d, 4)

    def v_read(self, idx, vbuf, slot):
        ks2, db = idx // 4, idx % 4
        d = VR + 4 * slot
        off = vbuf * TILE_BYTES + ks2 * 4096
        self.e.lds_read(f"ds_read_b64_tr_b16 {rng(d, 2)}, v{VADDR + db} offset:{off}", d, 2)
        return self.e.lds_read(f"ds_read_b64_tr_b16 {rng(d + 2, 2)}, v{VADDR + db} offset:{off + 2048}", d + 2, 2)

    # ------------------------------------------------------------ phases
    def phase_s(self, nxt, kbuf, ops, pre_ops, vreads=None):
        """16 score products S = K Q^T into `nxt`, K operands from LDS buffer
        kbuf through the ring; `ops` spread over the 16 slots, `pre_ops` before
        the first product; vreads = (vbuf, count): V^T operands of the next
        phase issued in the last slots."""
        e = self.e
        kid = {}
        for i in range(NKR):
            kid[i] = self.k_read(i, kbuf, i % NKR)
        for o in pre_ops:
            o.fn()
        slots = spread(ops, 16)
        vid = {}
        vslot0 = 16 - (vreads[1] if vreads else 0)
        for i in range(16):
            kb, ks = i // 8, i % 8
            e.wait_lds(kid[i])
            e.mfma(self.mf, nxt + 16 * kb, KR + 4 * (i % NKR), Q + 4 * ks, None if ks == 0 else nxt + 16 * kb)
            if i + NKR < 16:
                kid[i + NKR] = self.k_read(i + NKR, kbuf, (i + NKR) % NKR)
            if vreads and i >= vslot0:
                j = i - vslot0
                vid[j] = self.v_read(j, vreads[0], j % NVR)
            for o, s in zip(ops, slots):
                if s == i:
                    o.fn()
        return vid

    def phase_pv(self, cur, vbuf, ops, vid, pre_ops=()):
        """16 products O^T += V^T P^T with P from `cur` (chunk ks2 in the first
        four registers of cur + 16 (ks2 / 2) + 8 (ks2 % 2)); V^T operands from
        LDS buffer vbuf; vid: reads already issued."""
        e = self.e
        vid = dict(vid)
        nxt_read = len(vid)
        while nxt_read < NVR and nxt_read < 16:
            vid[nxt_read] = self.v_read(nxt_read, vbuf, nxt_read % NVR)
            nxt_read += 1
        for o in pre_ops:
            o.fn()
        slots = spread(ops, 16)
        for j in range(16):
            ks2, db = j // 4, j % 4
            e.wait_lds(vid[j])
            pb = cur + 16 * (ks2 // 2) + 8 * (ks2 % 2)
            e.mfma(self.mf, O + 16 * db, VR + 4 * (j % NVR), pb, O + 16 * db)
            if nxt_read < 16 and nxt_read <= j + NVR:
                vid[nxt_read] = self.v_read(nxt_read, vbuf, nxt_read % NVR)
                nxt_read += 1
            for o, s in zip(ops, slots):
                if s == j:
                    o.fn()

    def iteration(self, cur, nxt, t_parity, k_dma, tag):
        """Iteration t: tile t's softmax and P.V, tile t+1's scores.
        t_parity = t % 2.  k_dma: 'yes', 'no' or 'cond' (only if %[has_next]).

        Two complete versions follow the copies, chosen by whether any row of
        the wave moved its reference on tile t: with the rescale of O (64
        multiplies) in phase A, the first half of S(t+1)'s maximum and the copy
        offset updates move to phase B to balance the two phases."""
        e = self.e
        kbn, vb = 1 - t_parity, t_parity
        self.barrier()
        if k_dma == "yes":
            self.dma("k", t_parity)
        elif k_dma == "cond":
            e.raw("s_cmp_eq_u32 %[has_next], 0")
            e.raw(f"s_cbranch_scc1 {tag}5f")
            self.dma("k", t_parity)
            e.label(f"{tag}5:")
        self.dma("v", 1 - t_parity)
        offs = (KOFF,) if k_dma != "no" else ()

        def version(rescale):
            a_pre = [self.lscale_op()] + self.chunk_ops(cur, 0, 0)[:16]
            a_ops = self.chunk_ops(cur, 0, 0)[16:]
            mx_a = self.max_ops(nxt, 0, True)
            off_ops = self.offset_ops(offs) + self.offset_ops((VOFF,))
            if rescale:
                a_ops += self.rescale_ops()
            else:
                a_ops += off_ops
                for o in mx_a:
                    o.lo = 11
                a_ops += mx_a
            a_ops += self.chunk_ops(cur, 0, 1)[:16]      # fma + exp of chunk 1
            vid = self.phase_s(nxt, kbn, a_ops, a_pre, vreads=(vb, 4))
            # phase B: P chunk ks2 must be ready before the products of ks2
            # (slot 4 ks2 - 1 is the last slot before them)
            b_ops = self.chunk_ops(cur, 0, 1)[16:]      # conversion + sum of chunk 1
            for o in b_ops:
                o.hi = 2
            if rescale:
                b_ops += off_ops + mx_a
            c2 = self.chunk_ops(cur, 1, 0)
            for o in c2:
                o.hi = 6
            c3 = self.chunk_ops(cur, 1, 1)
            for o in c3:
                o.hi = 10
            b_ops += self.max_ops(nxt, 1, False) + c2 + c3 + self.refstep_ops() + self.refstep_commit_ops()
            self.phase_pv(cur, vb, b_ops, vid)

        e.raw("s_cmp_eq_u64 %[moved], 0")
        e.raw(f"s_cbranch_scc1 {tag}1f")
        snap = e.snapshot()
        version(True)
        e.raw(f"s_branch {tag}2f")
        end1 = e.snapshot()
        e.label(f"{tag}1:")
        e.restore(snap)
        version(False)
        e.merge_with(end1)
        e.label(f"{tag}2:")

    def prologue(self):
        """Tile 0: scores, maximum and reference step; K(1) copy issued."""
        e = self.e
        self.barrier()
        self.dma("k", 1)
        ops = self.offset_ops((KOFF,)) + self.max_ops(SA, 0, True) + self.max_ops(SA, 1, False)
        for o in ops[NI:]:
            o.lo = 15
        self.phase_s(SA, 0, ops, [])
        for o in self.refstep_ops() + self.refstep_commit_ops():
            o.fn()

    def epilogue(self, cur, vb):
        """Last steady tile (t = n-1): softmax and P.V only; V(n) copy issued
        if there is a next tile."""
        e = self.e
        self.barrier()
        e.raw("s_cmp_eq_u32 %[has_next], 0")
        e.raw("s_cbranch_scc1 7f")
        self.dma("v", 1 - vb)
        e.label("7:")
        pre = [self.lscale_op()] + self.rescale_ops() + self.chunk_ops(cur, 0, 0) + self.chunk_ops(cur, 0, 1)
        ops = self.chunk_ops(cur, 1, 0)
        for o in ops:
            o.hi = 6
        c3 = self.chunk_ops(cur, 1, 1)
        for o in c3:
            o.hi = 10
        self.phase_pv(cur, vb, ops + c3, {}, pre_ops=pre)

    def program(self):
        e = self.e
        e.raw("s_mov_b32 %[m0save], m0")
        self.prologue()
        e.raw("s_cmp_eq_u32 %[pairs], 0")
        e.raw("s_cbranch_scc1 3f")
        e.label("4:")
        e.assume_recent(LOOP_WRITTEN)
        self.iteration(SA, SB, 0, "yes", "1")
        self.iteration(SB, SA, 1, "yes", "2")
        e.raw("s_sub_u32 %[pairs], %[pairs], 1")
        e.raw("s_cmp_lg_u32 %[pairs], 0")
        e.raw("s_cbranch_scc1 4b")
        e.label("3:")
        e.assume_recent(LOOP_WRITTEN)
        self.iteration(SA, SB, 0, "cond", "3")
        self.epilogue(SB, 1)
        e.wait_all_lds()
        e.raw("s_mov_b32 m0, %[m0save]")
        e.raw("s_nop 7")
        e.raw("s_nop 7")
        return e.lines


def render(f16):
    lines = Gen(f16).program()
    return "".join(f'    "{ln}\\n"\n' for ln in lines)


HEADER = """// fwd_pipe_asm.h -- generated by gen_fwd_pipe.py; do not edit.
//
// Steady-state loop of fwd_m32_h16<T, 128, 256, 64>: a two-stage software
// pipeline over the key tiles that need no masking (see gen_fwd_pipe.py for
// the schedule and fwd_kernel.h for the per-row arithmetic it reproduces).
// Registers v0..v{last} belong to the block; operands are bound to them.
#pragma once
"""


def main():
    here = os.path.dirname(os.path.abspath(__file__))
    text = HEADER.format(last=NREG - 1)
    clob = [f'"v{r}"' for r in range(NREG) if r not in OPERAND_REGS] + ['"vcc"', '"scc"', '"memory"']
    text += "\n// registers the block writes that are not operands\n#define ATTN_PIPE_CLOBBERS"
    for i in range(0, len(clob), 12):
        text += " \\\n    " + ", ".join(clob[i:i + 12]) + ("," if i + 12 < len(clob) else "")
    text += "\n"
    v = lambda r: f'"{{v{r}}}"'
    vr = lambda r, n: f'"{{v[{r}:{r + n - 1}]}}"'
    outs = [f'"+{{v[{O + 16 * i}:{O + 16 * i + 15}]}}"(o[{i}])' for i in range(4)]
    outs += [f'"+{{v{M}}}"(m)', f'"+{{v{L}}}"(l)', f'"+{{v{KOFF}}}"(ko0)', f'"+{{v{KOFF + 1}}}"(ko1)',
             f'"+{{v{VOFF}}}"(vo0)', f'"+{{v{VOFF + 1}}}"(vo1)',
             '[pairs] "+s"(pairs)', '[moved] "=&s"(moved)', '[m0save] "=&s"(m0save)']
    ins = [f'{vr(Q + 4 * i, 4)}(qf[{i}])' for i in range(8)]
    ins += [f'{v(KADDR + i)}(ka[{i}])' for i in range(8)] + [f'{v(VADDR + i)}(va[{i}])' for i in range(4)]
    ins += ['[c] "s"(c)', '[slack] "s"(slack)', '[kbase] "s"(kbase)', '[vbase] "s"(vbase)', '[kdst] "s"(kdst)',
            '[vdst] "s"(vdst)', '[has_next] "s"(has_next)']
    text += ("\n// operands: fixed registers of the block bound to the kernel's variables\n"
             "#define ATTN_PIPE_OPERANDS \\\n    : " + ", \\\n      ".join(outs) +
             " \\\n    : " + ", \\\n      ".join(ins) + " \\\n    : ATTN_PIPE_CLOBBERS\n")
    for name, f16 in (("ATTN_PIPE_ASM_BF16", False), ("ATTN_PIPE_ASM_F16", True)):
        text += f"\n#define {name} \\\n" + render(f16).rstrip("\n").replace("\n", " \\\n") + "\n"
    path = os.path.join(here, "fwd_pipe_asm.h")
    if "--check" in sys.argv:
        with open(path) as f:
            sys.exit(0 if f.read() == text else 1)
    with open(path, "w") as f:
        f.write(text)
    print(path)


if __name__ == "__main__":
    main()
