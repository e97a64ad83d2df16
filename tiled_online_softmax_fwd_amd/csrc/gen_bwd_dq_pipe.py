#!/usr/bin/env python3
"""Writes bwd_dq_pipe_asm.h: the instruction-scheduled steady-state loop of the
gradient kernel bwd_dq<T, 128, 8> (dQ; 32 query rows per wave, 256 per
workgroup).

The loop covers the 32-key tiles that every row of the workgroup sees in
full.  Per tile t it computes S^T = K Q^T and dP^T = V dO^T (16 products), then
P = exp2(S c - lse2), dS = P (dP - D) rounded to the input type, then
dQ^T += K^T dS^T (8 products).  It is a two-stage software pipeline over
tiles: iteration t issues the products of tile t+1 beside tile t's vector work
(phase A), then tile t's dQ products (phase B).  Per element, every operation
and its order are the ones of the compiler-scheduled loop in bwd.hip, so the
results are bitwise equal; only the interleaving of independent instructions
differs.

Copies (one 16-byte LDS copy instruction per wave per tile): K is brought in
twice, once for the row reads of the score products and once for the
transposed reads of the dQ products, so that each buffer is in use for one
iteration only and every buffer, like the two register sets of scores,
alternates with period 2.  Iteration t copies K and V of tile t+2 (row
buffers) and K of tile t+1 (transposed-read buffer).  The LDS layouts are
operand-ordered: each read instruction reads one contiguous run (1024 bytes
for a row operand, 512 for a transposing read), so one address register per
kind serves every read through the instruction's offset field, and no read
has a bank conflict.  Q^T and dO^T stay in registers.

Run: python gen_bwd_dq_pipe.py  (rewrites bwd_dq_pipe_asm.h beside this file).
"""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from gen_fwd_pipe import Emitter, Op, rng, spread  # noqa: E402

# ---------------------------------------------------------------- register map
DQ = 0                          # v[0:63]    dQ^T accumulators, dq[db] = v[16db : 16db+15]
QW = 64                         # v[64:95]   Q^T operand, qw[ks] = v[64+4ks : +3]
GW = 96                         # v[96:127]  dO^T operand, gw[ks] = v[96+4ks : +3]
SETS = ((128, 144), (160, 176)) # (S^T / P / dS, dP^T) of the two tile parities, 16 registers each
NRING = 6
RING = 192                      # operand ring of K rows and V rows (4 registers a slot)
NTR = 4
TR = RING + 4 * NRING           # ring of transposed K operands (4 registers a slot)
KA = TR + 4 * NTR               # LDS byte address of this lane's row-operand chunk (buffer base)
TRA = KA + 1                    # ... of this lane's 8 transposed bytes
OFFA = KA + 2                   # global byte offset of this lane's chunk in the row copies' next tile
OFFB = KA + 3                   # ... in the transposed-read copy's next tile
L2, DSUM = KA + 4, KA + 5       # lse2 and minus D of this lane's query
NREG = DSUM + 1

OPERAND_REGS = set(range(DQ, GW + 32)) | set(range(KA, NREG))
LOOP_WRITTEN = list(range(DQ, DQ + 64)) + list(range(SETS[0][0], SETS[1][1] + 16))

TILE = 32 * 128 * 2             # one 32-key tile of K or V (bytes, LDS and HBM)
ROWS_K, KT, ROWS_V = 0, 2 * TILE, 4 * TILE   # LDS regions, two buffers each


class Gen:
    def __init__(self, f16):
        self.mf = "v_mfma_f32_32x32x16_f16" if f16 else "v_mfma_f32_32x32x16_bf16"
        self.cvt = "v_cvt_pk_f16_f32" if f16 else "v_cvt_pk_bf16_f32"
        self.e = Emitter()

    # ------------------------------------------------------------ vector work of one tile
    def vector_ops(self, cur):
        """P = exp2(S c - lse2), dS = P (dP - D), then dS rounded to the input
        type in place (chunk ks2 packed into the first 4 registers of
        s + 8 ks2)."""
        e, ops = self.e, []
        s, dp = cur
        for j in range(16):
            r = s + j
            ops.append(Op(lambda r=r: e.valu(f"v_fma_f32 v{r}, %[c], v{r}, -v{L2}", (r, L2), (r,)), 4))
        for j in range(16):
            r = s + j
            ops.append(Op(lambda r=r: e.valu(f"v_exp_f32 v{r}, v{r}", (r,), (r,), trans=True), 8))
        for j in range(16):
            r = dp + j
            ops.append(Op(lambda r=r: e.valu(f"v_add_f32 v{r}, v{r}, v{DSUM}", (r, DSUM), (r,)), 4))
        for j in range(16):
            a, b = s + j, dp + j
            ops.append(Op(lambda a=a, b=b: e.valu(f"v_mul_f32 v{a}, v{a}, v{b}", (a, b), (a,)), 4))
        for ks2 in range(2):
            for i in range(0, 8, 2):
                d, a, b = s + 8 * ks2 + i // 2, s + 8 * ks2 + i, s + 8 * ks2 + i + 1
                ops.append(Op(lambda d=d, a=a, b=b: e.valu(f"{self.cvt} v{d}, v{a}, v{b}", (a, b), (d,)), 4))
        return ops

    def offset_ops(self, regs):
        e = self.e
        return [Op(lambda r=r: e.valu(f"v_add_u32 v{r}, 0x{TILE:x}, v{r}", (r,), (r,)), 4) for r in regs]

    # ------------------------------------------------------------ memory
    def barrier(self):
        self.e.wait_all_lds()
        self.e.raw("s_waitcnt vmcnt(0)")
        self.e.raw("s_barrier")

    def dma(self, region, buf, base, off):
        self.e.raw(f"s_add_u32 m0, %[kdst], 0x{region + buf * TILE:x}")
        self.e.raw("s_nop 0")
        self.e.raw(f"global_load_lds_dwordx4 v{off}, {base}")

    def read_row(self, kind, ks, buf, slot):
        d = RING + 4 * slot
        region = ROWS_K if kind == "k" else ROWS_V
        return self.e.lds_read(f"ds_read_b128 {rng(d, 4)}, v{KA} offset:{region + buf * TILE + ks * 1024}", d, 4)

    def read_tr(self, ks2, db, buf, slot):
        d = TR + 4 * slot
        off = KT + buf * TILE + (ks2 * 4 + db) * 2 * 512
        self.e.lds_read(f"ds_read_b64_tr_b16 {rng(d, 2)}, v{TRA} offset:{off}", d, 2)
        return self.e.lds_read(f"ds_read_b64_tr_b16 {rng(d + 2, 2)}, v{TRA} offset:{off + 512}", d + 2, 2)

    # ------------------------------------------------------------ phases
    def phase_products(self, nxt, rbuf, ops, pre_ops=(), tr_first=None):
        """16 products of the next tile into `nxt`: for ks = 0..7, S^T += K row
        chunk ks x Q^T ks, then dP^T += V row chunk ks x dO^T ks; operands
        through the ring (reads in use order, issued ahead); `ops` spread over
        the 16 slots.  tr_first = buf: the first transposed reads of phase B
        issued in the last slots."""
        e = self.e
        s, dp = nxt
        reads = []
        for ks in range(8):
            reads += [("k", ks), ("v", ks)]
        rid, nxt_read = {}, 0

        def issue_upto(limit):
            nonlocal nxt_read
            while nxt_read < len(reads) and nxt_read < limit:
                kind, ks = reads[nxt_read]
                rid[nxt_read] = self.read_row(kind, ks, rbuf, nxt_read % NRING)
                nxt_read += 1

        issue_upto(NRING)
        for o in pre_ops:
            o.fn()
        slots = spread(ops, 16)
        trid = {}
        for i in range(16):
            ks = i // 2
            a = 2 * ks + (i % 2)
            e.wait_lds(rid[a])
            if i % 2 == 0:
                e.mfma(self.mf, s, RING + 4 * (a % NRING), QW + 4 * ks, None if ks == 0 else s)
            else:
                e.mfma(self.mf, dp, RING + 4 * (a % NRING), GW + 4 * ks, None if ks == 0 else dp)
            issue_upto(a + 1 + NRING)
            if tr_first is not None and i >= 16 - NTR:
                j = i - (16 - NTR)
                trid[j] = self.read_tr(j // 4, j % 4, tr_first, j % NTR)
            for o, sl in zip(ops, slots):
                if sl == i:
                    o.fn()
        return trid

    def phase_dq(self, cur, kbuf, ops, trid):
        """8 products dQ^T[db] += K^T chunk (ks2, db) x dS chunk ks2 of `cur`;
        K^T operands from the transposed-read buffer kbuf; trid: reads already
        issued."""
        e = self.e
        s = cur[0]
        trid = dict(trid)
        nxt = len(trid)
        while nxt < NTR:
            trid[nxt] = self.read_tr(nxt // 4, nxt % 4, kbuf, nxt % NTR)
            nxt += 1
        slots = spread(ops, 8) if ops else []
        for j in range(8):
            ks2, db = j // 4, j % 4
            e.wait_lds(trid[j])
            e.mfma(self.mf, DQ + 16 * db, TR + 4 * (j % NTR), s + 8 * ks2, DQ + 16 * db)
            if nxt < 8:
                trid[nxt] = self.read_tr(nxt // 4, nxt % 4, kbuf, nxt % NTR)
                nxt += 1
            for o, sl in zip(ops, slots):
                if sl == j:
                    o.fn()

    def iteration(self, p, dma_rows):
        """Iteration t (t % 2 = p): copies of tiles t+2 (rows, if dma_rows) and
        t+1 (transposed reads); products of tile t+1 beside tile t's vector
        work; tile t's dQ products."""
        cur, nxt = SETS[p], SETS[1 - p]
        self.barrier()
        if dma_rows:
            self.dma(ROWS_K, p, "%[kbase]", OFFA)
            self.dma(ROWS_V, p, "%[vbase]", OFFA)
        self.dma(KT, 1 - p, "%[kbase]", OFFB)
        ops = self.vector_ops(cur)
        # the packed chunk ks2 must be complete before the dQ products: all
        # vector work stays in phase A; offsets advance after their copies
        ops += self.offset_ops(((OFFA,) if dma_rows else ()) + (OFFB,))
        trid = self.phase_products(nxt, 1 - p, ops, tr_first=p)
        self.phase_dq(cur, p, [], trid)

    def prologue(self):
        """Tile 0's products (its row copies were issued before the block);
        copies of tile 1 (rows) and tile 0 (transposed reads)."""
        self.barrier()
        self.dma(ROWS_K, 1, "%[kbase]", OFFA)
        self.dma(ROWS_V, 1, "%[vbase]", OFFA)
        self.dma(KT, 0, "%[kbase]", OFFB)
        self.phase_products(SETS[0], 0, self.offset_ops((OFFA, OFFB)))

    def epilogue(self):
        """Last tile (t = n-1, odd): vector work, then its dQ products."""
        cur = SETS[1]
        self.barrier()
        for o in self.vector_ops(cur):
            o.fn()
        self.phase_dq(cur, 1, [], {})

    def program(self):
        e = self.e
        e.raw("s_mov_b32 %[m0save], m0")
        self.prologue()
        e.raw("s_cmp_eq_u32 %[pairs], 0")
        e.raw("s_cbranch_scc1 3f")
        e.label("4:")
        e.assume_recent(LOOP_WRITTEN)
        self.iteration(0, True)
        self.iteration(1, True)
        e.raw("s_sub_u32 %[pairs], %[pairs], 1")
        e.raw("s_cmp_lg_u32 %[pairs], 0")
        e.raw("s_cbranch_scc1 4b")
        e.label("3:")
        e.assume_recent(LOOP_WRITTEN)
        self.iteration(0, False)
        self.epilogue()
        e.wait_all_lds()
        e.raw("s_mov_b32 m0, %[m0save]")
        e.raw("s_nop 7")
        e.raw("s_nop 7")
        return e.lines


def render(f16):
    lines = Gen(f16).program()
    return "".join(f'    "{ln}\\n"\n' for ln in lines)


HEADER = """// bwd_dq_pipe_asm.h -- generated by gen_bwd_dq_pipe.py; do not edit.
//
// Steady-state loop of bwd_dq<T, 128, 8>: a two-stage software pipeline over
// the 32-key tiles every row of the workgroup sees (see gen_bwd_dq_pipe.py for
// the schedule and bwd.hip for the per-element arithmetic it reproduces).
// Registers v0..v{last} belong to the block; operands are bound to them.
#pragma once
"""


def main():
    here = os.path.dirname(os.path.abspath(__file__))
    text = HEADER.format(last=NREG - 1)
    clob = [f'"v{r}"' for r in range(NREG) if r not in OPERAND_REGS] + ['"scc"', '"memory"']
    text += "\n// registers the block writes that are not operands\n#define ATTN_DQ_PIPE_CLOBBERS"
    for i in range(0, len(clob), 12):
        text += " \\\n    " + ", ".join(clob[i:i + 12]) + ("," if i + 12 < len(clob) else "")
    text += "\n"
    v = lambda r: f'"{{v{r}}}"'
    vr = lambda r, n: f'"{{v[{r}:{r + n - 1}]}}"'
    outs = [f'"+{{v[{DQ + 16 * i}:{DQ + 16 * i + 15}]}}"(dq[{i}])' for i in range(4)]
    outs += [f'"+{{v{OFFA}}}"(offa)', f'"+{{v{OFFB}}}"(offb)', '[pairs] "+s"(pairs)', '[m0save] "=&s"(m0save)']
    ins = [f'{vr(QW + 4 * i, 4)}(qw[{i}])' for i in range(8)] + [f'{vr(GW + 4 * i, 4)}(gw[{i}])' for i in range(8)]
    ins += [f'{v(KA)}(ka)', f'{v(TRA)}(tra)', f'{v(L2)}(l2)', f'{v(DSUM)}(ndsum)']
    ins += ['[c] "s"(c)', '[kbase] "s"(kbase)', '[vbase] "s"(vbase)', '[kdst] "s"(kdst)']
    text += ("\n// operands: fixed registers of the block bound to the kernel's variables\n"
             "#define ATTN_DQ_PIPE_OPERANDS \\\n    : " + ", \\\n      ".join(outs) +
             " \\\n    : " + ", \\\n      ".join(ins) + " \\\n    : ATTN_DQ_PIPE_CLOBBERS\n")
    for name, f16 in (("ATTN_DQ_PIPE_ASM_BF16", False), ("ATTN_DQ_PIPE_ASM_F16", True)):
        text += f"\n#define {name} \\\n" + render(f16).rstrip("\n").replace("\n", " \\\n") + "\n"
    path = os.path.join(here, "bwd_dq_pipe_asm.h")
    if "--check" in sys.argv:
        with open(path) as f:
            sys.exit(0 if f.read() == text else 1)
    with open(path, "w") as f:
        f.write(text)
    print(path)


if __name__ == "__main__":
    main()
