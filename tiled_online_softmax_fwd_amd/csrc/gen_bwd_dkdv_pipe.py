#!/usr/bin/env python3
"""Writes bwd_dkdv_pipe_asm.h: the instruction-scheduled steady state of the
gradient kernel bwd_dkdv<T, 128, 8, 1> (dK and dV; 32 keys per wave, 256 per
workgroup).

The block covers the 32-query steps whose rows see every key of the
workgroup.  Per step t the wave computes S = Q K^T and dP = dO V^T (8
products each; dP accumulates onto -D, which the workspace holds), P =
exp2(S c - lse2), dS = P (dP - D), both rounded to the input type, then
dV += P^T dO and dK += dS^T Q (8 products each).  It is a two-stage software
pipeline over steps; iteration t issues, in this order,
    S(t+1)   beside dS(t) and its rounding,
    dK(t)    beside the rounding of P(t),
    dV(t)    beside the exponentials of step t+1 (-D of step t+1 is read
             into the dP accumulator after the last dK product),
    dP(t+1)  beside the rest of those exponentials.
Per element, every operation and its order are those of the compiler-scheduled
loop in bwd.hip, so the results are bitwise equal; only the interleaving of
independent instructions differs.

LDS layouts are operand-ordered: each read instruction of the block reads one
contiguous run (1024 bytes for a row operand, 512 for a transposing read), so
one address register per kind serves every read through the instruction's
offset field, and no read has a bank conflict.  Q and dO are each copied twice,
once in the row-read layout (steps t+2, read in iteration t+1) and once in the
transposing-read layout (step t+1, read in iteration t+1), so that every
buffer alternates with period 2.  lse2 and D of each step are copied into a
slot private to the wave.

Run: python gen_bwd_dkdv_pipe.py  (rewrites bwd_dkdv_pipe_asm.h beside this file).
"""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from gen_fwd_pipe import Emitter, Op, rng, spread  # noqa: E402

# ---------------------------------------------------------------- register map
DK, DV = 0, 64                  # v[0:63] dK, v[64:127] dV; block db = v[base+16db : +15]
KW = 128                        # v[128:159] K^T operand, kw[ks] = v[128+4ks : +3]
SETS = (160, 176)               # S / P of the two step parities, 16 registers each
DPS = 192                       # dP / dS of the current step
NRING = 5
RING = 208                      # ring of row operands, V^T operands and lse2 / D vectors
NTR = 3
TR = RING + 4 * NRING           # ring of transposed operands
KA = TR + 4 * NTR               # LDS byte address of this lane's row-operand chunk (buffer base)
TRA = KA + 1                    # ... of this lane's 8 transposed bytes
VWA = KA + 2                    # ... of this lane's V^T operand, ks = 0
LDA = KA + 3                    # ... of this lane's lse2 vector in the wave's slot 0
OFFR = KA + 4                   # global byte offset of this lane's chunk: next row copy
OFFT = KA + 5                   # ... next transposed-layout copy
OFFL = KA + 6                   # ... next lse2 / D copy (relative to the head's D)
NREG = OFFL + 1

OPERAND_REGS = set(range(DK, KW + 32)) | set(range(KA, NREG))
LOOP_WRITTEN = list(range(DK, DV + 64)) + list(range(SETS[0], DPS + 16))

TILE = 32 * 128 * 2             # one 32-row step of Q or dO (bytes)
ROWQ, ROWG, TRQ, TRG = 0, 2 * TILE, 4 * TILE, 6 * TILE   # two buffers each
LDSLOT = 256                    # one step's lse2 (32 floats) then D (32 floats)


class VOp(Op):
    """A vector op that may consume ring reads: fn(regs) gets their registers."""
    def __init__(self, fn, cost, lo=-1, hi=99, reads=()):
        super().__init__(fn, cost, lo, hi)
        self.reads = list(reads)


class Gen:
    def __init__(self, f16):
        self.mf = "v_mfma_f32_32x32x16_f16" if f16 else "v_mfma_f32_32x32x16_bf16"
        self.cvt = "v_cvt_pk_f16_f32" if f16 else "v_cvt_pk_bf16_f32"
        self.e = Emitter()

    # ------------------------------------------------------------ reads (pool, emit(dst) -> id)
    def rd_row(self, kind, ks, buf):
        e = self.e
        if kind == "v":
            text = lambda d: f"ds_read_b128 {rng(d, 4)}, v{VWA} offset:{ks * 1024}"
        else:
            region = ROWQ if kind == "q" else ROWG
            text = lambda d: f"ds_read_b128 {rng(d, 4)}, v{KA} offset:{region + buf * TILE + ks * 1024}"
        return ("ring", lambda d: e.lds_read(text(d), d, 4))

    def rd_ld(self, kind, g4, buf):
        e = self.e
        assert kind == "l"
        off = buf * LDSLOT + g4 * 32
        return ("ring", lambda d: e.lds_read(f"ds_read_b128 {rng(d, 4)}, v{LDA} offset:{off}", d, 4))

    def rd_tr(self, kind, tt, db, buf):
        e = self.e
        off = (TRQ if kind == "q" else TRG) + buf * TILE + (tt * 4 + db) * 2 * 512

        def emit(d):
            e.lds_read(f"ds_read_b64_tr_b16 {rng(d, 2)}, v{TRA} offset:{off}", d, 2)
            return e.lds_read(f"ds_read_b64_tr_b16 {rng(d + 2, 2)}, v{TRA} offset:{off + 512}", d + 2, 2)
        return ("tr", emit)

    # ------------------------------------------------------------ scheduling
    def run(self, mfmas, ops):
        """mfmas: list of (reads, fn(regs)); ops: VOps spread over the matrix
        slots (an op in slot i follows matrix op i, program order kept)."""
        slots = spread(ops, len(mfmas)) if ops else []
        seq = []
        for i, (rd, fn) in enumerate(mfmas):
            seq.append((rd, fn))
            for o, s in zip(ops, slots):
                if s == i:
                    seq.append((o.reads, o.fn))
        self.consume(seq)

    def consume(self, seq):
        """Emit the consumers of seq (each (reads, fn(regs))) in order.  Reads
        go through their pools in consumption order, each issued as soon as the
        slot it reuses has been consumed; a consumer waits for its newest read."""
        e = self.e
        size, base = {"ring": NRING, "tr": NTR}, {"ring": RING, "tr": TR}
        stream = {"ring": [], "tr": []}
        cons = []
        for rd, _ in seq:
            lst = []
            for pool, emit in rd:
                stream[pool].append(emit)
                lst.append((pool, len(stream[pool]) - 1))
            cons.append(lst)
        nxt = {"ring": 0, "tr": 0}
        done = {k: [False] * len(v) for k, v in stream.items()}
        rid = {}

        def issue():
            for pool in ("ring", "tr"):
                while nxt[pool] < len(stream[pool]):
                    k = nxt[pool]
                    if k >= size[pool] and not done[pool][k - size[pool]]:
                        break
                    rid[(pool, k)] = stream[pool][k](base[pool] + 4 * (k % size[pool]))
                    nxt[pool] += 1

        issue()
        for (rd, fn), lst in zip(seq, cons):
            for key in lst:
                assert key in rid, "operand read not issued before its use"
            if lst:
                e.wait_lds(max(rid[key] for key in lst))
            fn([base[pool] + 4 * (k % size[pool]) for pool, k in lst])
            for pool, k in lst:
                done[pool][k] = True
            issue()
        assert all(all(v) for v in done.values())

    # ------------------------------------------------------------ memory
    def barrier(self):
        self.e.wait_all_lds()
        self.e.raw("s_waitcnt vmcnt(0)")
        self.e.raw("s_barrier")

    def dma16(self, region, buf, base, off):
        self.e.raw(f"s_add_u32 m0, %[kdst], 0x{region + buf * TILE:x}")
        self.e.raw("s_nop 0")
        self.e.raw(f"global_load_lds_dwordx4 v{off}, {base}")

    def dma_ld(self, buf):
        """lse2 / D of a step into the wave's slot buf; the offset moves on."""
        e = self.e
        e.raw(f"s_add_u32 m0, %[ldst], 0x{buf * LDSLOT:x}")
        e.raw("s_nop 0")
        e.raw(f"global_load_lds_dword v{OFFL}, %[dbase]")
        e.valu(f"v_add_u32 v{OFFL}, 0x80, v{OFFL}", (OFFL,), (OFFL,))

    def offset_ops(self, regs):
        e = self.e
        return [VOp(lambda _, r=r: e.valu(f"v_add_u32 v{r}, 0x{TILE:x}, v{r}", (r,), (r,)), 4) for r in regs]

    # ------------------------------------------------------------ work of one step
    def ds_ops(self, cur, hi_ds, hi_p):
        """dS = P (dP - D) in place in DPS (the dP accumulator started at -D),
        then dS and P rounded to the input type in place (chunk tt packed into
        the first 4 registers of base + 8 tt)."""
        e, ops = self.e, []
        for j in range(16):
            a, b = cur + j, DPS + j
            ops.append(VOp(lambda _, a=a, b=b: e.valu(f"v_mul_f32 v{b}, v{a}, v{b}", (a, b), (b,)), 4, hi=hi_ds))
        for base, hi in ((DPS, hi_ds), (cur, hi_p)):
            for tt in range(2):
                for i in range(0, 8, 2):
                    d, a, b = base + 8 * tt + i // 2, base + 8 * tt + i, base + 8 * tt + i + 1
                    ops.append(VOp(lambda _, d=d, a=a, b=b: e.valu(f"{self.cvt} v{d}, v{a}, v{b}", (a, b), (d,)), 4,
                                   hi=hi))
        return ops

    def read_nd(self, buf):
        """-D of a step's rows (8 g4 + 4 hh + i) from the wave's slot buf
        straight into the dP accumulator; returns the last read's id."""
        e, rid = self.e, None
        for g4 in range(4):
            d = DPS + 4 * g4
            rid = e.lds_read(f"ds_read_b128 {rng(d, 4)}, v{LDA} offset:{buf * LDSLOT + 128 + g4 * 32}", d, 4)
        return rid

    def exp_ops(self, s, buf, lo):
        """P = exp2(S c - lse2) in place (lse2 of rows 8 g4 + 4 hh + i)."""
        e, ops = self.e, []
        for g4 in range(4):
            def fn(regs, g4=g4):
                for i in range(4):
                    r = s + 4 * g4 + i
                    e.valu(f"v_fma_f32 v{r}, %[c], v{r}, -v{regs[0] + i}", (r, regs[0] + i), (r,))
            ops.append(VOp(fn, 16, lo=lo, reads=[self.rd_ld("l", g4, buf)]))
        for j in range(16):
            r = s + j
            ops.append(VOp(lambda _, r=r: e.valu(f"v_exp_f32 v{r}, v{r}", (r,), (r,), trans=True), 8, lo=lo))
        return ops

    def mf_s(self, dst, buf):
        e = self.e
        return [([self.rd_row("q", ks, buf)],
                 lambda regs, ks=ks: e.mfma(self.mf, dst, regs[0], KW + 4 * ks, None if ks == 0 else dst))
                for ks in range(8)]

    def mf_dp(self, buf):
        """dP accumulated onto the -D already read into DPS (self.nd_rid)."""
        e = self.e

        def first(regs):
            e.wait_lds(self.nd_rid)
            e.mfma(self.mf, DPS, regs[0], regs[1], DPS)
        return [([self.rd_row("g", ks, buf), self.rd_row("v", ks, None)],
                 first if ks == 0 else (lambda regs: e.mfma(self.mf, DPS, regs[0], regs[1], DPS)))
                for ks in range(8)]

    def mf_grad(self, kind, src, buf, after_last=None):
        """dV += P^T dO (kind 'g') or dK += dS^T Q (kind 'q'), chunks tt = 0, 1
        of the step's 32 rows for each 32-column block db; after_last() is
        emitted right after the last product."""
        e = self.e
        acc = DV if kind == "g" else DK
        items = [(tt, db) for tt in range(2) for db in range(4)]

        def fn(regs, tt, db, last):
            e.mfma(self.mf, acc + 16 * db, src + 8 * tt, regs[0], acc + 16 * db)
            if last and after_last is not None:
                after_last()
        return [([self.rd_tr(kind, tt, db, buf)],
                 lambda regs, tt=tt, db=db, last=(n == len(items) - 1): fn(regs, tt, db, last))
                for n, (tt, db) in enumerate(items)]

    # ------------------------------------------------------------ program
    def iteration(self, p, last):
        """Iteration t (t % 2 = p); last: t = n-2 (no copies of step t+2)."""
        cur, nxt = SETS[p], SETS[1 - p]
        self.barrier()
        if not last:
            self.dma16(ROWQ, p, "%[qbase]", OFFR)
            self.dma16(ROWG, p, "%[gbase]", OFFR)
            # the slot held lse2 and -D of step t, both read in iteration t-1
            self.dma_ld(p)
        self.dma16(TRQ, 1 - p, "%[qbase]", OFFT)
        self.dma16(TRG, 1 - p, "%[gbase]", OFFT)

        def nd():
            self.nd_rid = self.read_nd(1 - p)
        mf = (self.mf_s(nxt, 1 - p) + self.mf_grad("q", DPS, p, after_last=nd) + self.mf_grad("g", cur, p) +
              self.mf_dp(1 - p))
        ops = self.offset_ops(((OFFR,) if not last else ()) + (OFFT,))
        ops += self.ds_ops(cur, 7, 15)
        ops += self.exp_ops(nxt, 1 - p, 9)
        self.run(mf, ops)

    def prologue(self):
        """Step 0's products and exponentials (its row copies and lse2 / D were
        issued before the block); copies of step 1 (rows, lse2 / D) and step 0
        (transposed layout)."""
        self.barrier()
        self.dma16(ROWQ, 1, "%[qbase]", OFFR)
        self.dma16(ROWG, 1, "%[gbase]", OFFR)
        self.dma16(TRQ, 0, "%[qbase]", OFFT)
        self.dma16(TRG, 0, "%[gbase]", OFFT)
        self.dma_ld(1)
        self.nd_rid = self.read_nd(0)
        ops = self.offset_ops((OFFR, OFFT)) + self.exp_ops(SETS[0], 0, 9)
        self.run(self.mf_s(SETS[0], 0) + self.mf_dp(0), ops)

    def epilogue(self):
        """Last step (t = n-1, odd): dS and the rounding (nothing left to
        overlap them with), then dK and dV."""
        cur = SETS[1]
        self.barrier()
        self.consume([(o.reads, o.fn) for o in self.ds_ops(cur, 99, 99)])
        self.run(self.mf_grad("q", DPS, 1) + self.mf_grad("g", cur, 1), [])

    def program(self):
        e = self.e
        e.raw("s_mov_b32 %[m0save], m0")
        self.prologue()
        e.raw("s_cmp_eq_u32 %[pairs], 0")
        e.raw("s_cbranch_scc1 3f")
        e.label("4:")
        e.assume_recent(LOOP_WRITTEN)
        self.iteration(0, False)
        self.iteration(1, False)
        e.raw("s_sub_u32 %[pairs], %[pairs], 1")
        e.raw("s_cmp_lg_u32 %[pairs], 0")
        e.raw("s_cbranch_scc1 4b")
        e.label("3:")
        e.assume_recent(LOOP_WRITTEN)
        self.iteration(0, True)
        self.epilogue()
        e.wait_all_lds()
        e.raw("s_mov_b32 m0, %[m0save]")
        e.raw("s_nop 7")
        e.raw("s_nop 7")
        return e.lines


def render(f16):
    lines = Gen(f16).program()
    return "".join(f'    "{ln}\\n"\n' for ln in lines)


HEADER = """// bwd_dkdv_pipe_asm.h -- generated by gen_bwd_dkdv_pipe.py; do not edit.
//
// Steady state of bwd_dkdv<T, 128, 8, 1>: a two-stage software pipeline over
// the 32-query steps whose rows see every key of the workgroup (see
// gen_bwd_dkdv_pipe.py for the schedule and the LDS layouts, and bwd.hip for
// the per-element arithmetic it reproduces).  Registers v0..v{last} belong to
// the block; operands are bound to them.
#pragma once
"""


def main():
    here = os.path.dirname(os.path.abspath(__file__))
    text = HEADER.format(last=NREG - 1)
    clob = [f'"v{r}"' for r in range(NREG) if r not in OPERAND_REGS] + ['"scc"', '"memory"']
    text += "\n// registers the block writes that are not operands\n#define ATTN_DKDV_PIPE_CLOBBERS"
    for i in range(0, len(clob), 12):
        text += " \\\n    " + ", ".join(clob[i:i + 12]) + ("," if i + 12 < len(clob) else "")
    text += "\n"
    v = lambda r: f'"{{v{r}}}"'
    vr = lambda r, n: f'"{{v[{r}:{r + n - 1}]}}"'
    outs = [f'"+{{v[{DK + 16 * i}:{DK + 16 * i + 15}]}}"(dk0[{i}])' for i in range(4)]
    outs += [f'"+{{v[{DV + 16 * i}:{DV + 16 * i + 15}]}}"(dv0[{i}])' for i in range(4)]
    outs += [f'"+{{v{OFFR}}}"(offr)', f'"+{{v{OFFT}}}"(offt)', f'"+{{v{OFFL}}}"(offl)',
             '[pairs] "+s"(pairs)', '[m0save] "=&s"(m0save)']
    ins = [f'{vr(KW + 4 * i, 4)}(kw0[{i}])' for i in range(8)]
    ins += [f'{v(KA)}(ka)', f'{v(TRA)}(tra)', f'{v(VWA)}(vwa)', f'{v(LDA)}(lda)']
    ins += ['[c] "s"(c)', '[qbase] "s"(qbase)', '[gbase] "s"(gbase)', '[dbase] "s"(dbase)',
            '[kdst] "s"(kdst)', '[ldst] "s"(ldst)']
    text += ("\n// operands: fixed registers of the block bound to the kernel's variables\n"
             "#define ATTN_DKDV_PIPE_OPERANDS \\\n    : " + ", \\\n      ".join(outs) +
             " \\\n    : " + ", \\\n      ".join(ins) + " \\\n    : ATTN_DKDV_PIPE_CLOBBERS\n")
    for name, f16 in (("ATTN_DKDV_PIPE_ASM_BF16", False), ("ATTN_DKDV_PIPE_ASM_F16", True)):
        text += f"\n#define {name} \\\n" + render(f16).rstrip("\n").replace("\n", " \\\n") + "\n"
    path = os.path.join(here, "bwd_dkdv_pipe_asm.h")
    if "--check" in sys.argv:
        with open(path) as f:
            sys.exit(0 if f.read() == text else 1)
    with open(path, "w") as f:
        f.write(text)
    print(path)


if __name__ == "__main__":
    main()
