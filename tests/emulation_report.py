"""Deviation sweeps of the precision-emulating model (CPU only; test
infrastructure).  Not collected by pytest; run as

    python -m tests.emulation_report [--out reports]

The model (oracle/emulate.c) re-runs the flash algorithm and baseline attention
with each intermediate held in a chosen format and compares them with the fp64
plain definition, as the microbenchmark of Golden et al., "Is Flash Attention
Stable?", sec. III and IV-A does.  Two flash models are reported:

  R1  this library's precision: dot products, sums and the running state in
      fp32 (registers), P rounded to the input format, O stored in fp32;
  R2  stored state: as R1, but the running sum and unnormalised output are
      rounded to the input format between key tiles (the key/value-outer nest
      of the original FlashAttention, which keeps its state in memory).

Baseline: S and P stored in the input format, fp32 accumulation, fp32 output.

Sweeps (rows sampled; statistics of |delta| over their elements):
  formats   bf16, fp16, tf32, fp32 and significand widths 6..24 (Figs. 3, 4)
  seqlen    N = 256 .. 4096, bf16, Bc = 64 (Fig. 5)
  tiles     Bc = 16 .. 128, ascending / descending key tiles (Fig. 6)
  gpu       R1 on the seeded inputs of the GPU deviation reports, next to the
            figures measured on MI355X (reports/deviation_*.json), if present.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402
from oracle import emulate as E  # noqa: E402


def say(*a):
    print("[emu]", *a, flush=True)


def stats(x, ref):
    a = np.abs(np.asarray(x) - ref)
    return {"max": float(a.max()), "mean": float(a.mean()), "std": float(a.std())}


def f3(s):
    return f"{s['max']:.2e} | {s['mean']:.2e} | {s['std']:.2e}"


def rows_of(B, H, N, per_head, seed):
    rng = np.random.default_rng(seed)
    out = []
    for bh in range(B * H):
        out.append(bh * N + np.sort(rng.choice(N, size=min(per_head, N), replace=False)))
    return np.concatenate(out)


def models(q, k, v, scale, rows, fmt, bc=64, order=0, causal=False):
    """(R1, R2, baseline) outputs on `rows` with inputs and storage in `fmt`."""
    r1 = E.flash_rows(q, k, v, scale, rows, causal, acc="f32", p=fmt, state="f32", out="f32", bc=bc, order=order)
    r2 = E.flash_rows(q, k, v, scale, rows, causal, acc="f32", p=fmt, state=fmt, out="f32", bc=bc, order=order,
                      kv_outer=True)
    bl = E.baseline_rows(q, k, v, scale, rows, causal, acc="f32", store=fmt, out="f32")
    return r1, r2, bl


def round_inputs(p, fmt):
    return [E.round_fmt(x, fmt) for x in (p.q64, p.k64, p.v64)]


def sweep_formats():
    B, H, N, d = 1, 2, 1024, 64
    p = synth.make_qkv(B, H, N, d, "f32", 31)
    rows = rows_of(B, H, N, 96, 1)
    res = []
    names = ["bf16", "f16", "tf32", "f32"] + [E.fmt_bits(b) for b in (6, 10, 12, 14, 16, 20)]
    for fmt in names:
        label = fmt if isinstance(fmt, str) else f"p={fmt[0]}"
        say("formats", label)
        q, k, v = round_inputs(p, fmt)
        ro, _ = oracle.attn_rows(q, k, v, 0.125, rows, False)
        r1, r2, bl = models(q, k, v, 0.125, rows, fmt)
        bits = E.FORMATS[fmt][0] if isinstance(fmt, str) else fmt[0]
        res.append({"format": label, "bits": bits, "R1": stats(r1, ro), "R2": stats(r2, ro), "baseline": stats(bl, ro),
                    "R1_vs_baseline": stats(r1, bl), "R2_vs_baseline": stats(r2, bl)})
    res.sort(key=lambda r: r["bits"])
    md = ["## Numerical format (Figs. 3 and 4): B1 H2 N1024 d64, 192 rows, inputs rounded to the format", "",
          "| format | significand bits | R1 vs fp64 max | mean | std | R2 vs fp64 max | mean | std | "
          "baseline vs fp64 max | mean | std | max R1-baseline | max R2-baseline |",
          "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in res:
        md.append(f"| {r['format']} | {r['bits']} | {f3(r['R1'])} | {f3(r['R2'])} | {f3(r['baseline'])} | "
                  f"{r['R1_vs_baseline']['max']:.2e} | {r['R2_vs_baseline']['max']:.2e} |")
    return res, md


def sweep_seqlen():
    res = []
    for N in (256, 512, 1024, 2048, 4096):
        say("seqlen", N)
        p = synth.make_qkv(1, 2, N, 64, "bf16", 32)
        rows = rows_of(1, 2, N, 64, 2)
        ro, _ = oracle.attn_rows(p.q64, p.k64, p.v64, 0.125, rows, False)
        r1, r2, bl = models(p.q64, p.k64, p.v64, 0.125, rows, "bf16")
        res.append({"N": N, "R1": stats(r1, ro), "R2": stats(r2, ro), "baseline": stats(bl, ro),
                    "R1_vs_baseline": stats(r1, bl), "R2_vs_baseline": stats(r2, bl)})
    md = ["## Sequence length (Fig. 5): B1 H2 d64 bf16, Bc = 64, 128 rows", "",
          "| N | R1 vs fp64 max | mean | std | R2 vs fp64 max | mean | std | baseline vs fp64 max | mean | std | "
          "R2-baseline max | mean | std |", "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in res:
        md.append(f"| {r['N']} | {f3(r['R1'])} | {f3(r['R2'])} | {f3(r['baseline'])} | {f3(r['R2_vs_baseline'])} |")
    return res, md


def sweep_tiles():
    N = 2048
    p = synth.make_qkv(1, 2, N, 64, "bf16", 33)
    rows = rows_of(1, 2, N, 64, 3)
    ro, _ = oracle.attn_rows(p.q64, p.k64, p.v64, 0.125, rows, False)
    res = []
    for bc in (16, 32, 64, 128):
        for order in (0, 1):
            say("tiles", bc, order)
            r1, r2, bl = models(p.q64, p.k64, p.v64, 0.125, rows, "bf16", bc=bc, order=order)
            res.append({"bc": bc, "order": order, "R1": stats(r1, ro), "R2": stats(r2, ro)})
    md = ["## Tile size and order (Fig. 6): B1 H2 N2048 d64 bf16, 128 rows", "",
          "| Bc | order | R1 vs fp64 max | mean | std | R2 vs fp64 max | mean | std |", "|---|---|---|---|---|---|---|---|"]
    for r in res:
        md.append(f"| {r['bc']} | {'desc' if r['order'] else 'asc'} | {f3(r['R1'])} | {f3(r['R2'])} |")
    md += ["", "Br (query rows per tile) does not enter either model: each row's arithmetic is independent of "
               "how rows are grouped, so square versus rectangular tiles cannot change the result.", ""]
    return res, md


def gpu_cross_check(report_dir):
    md = ["## Model R1 against the deviation measured on MI355X", ""]
    res = {}
    tiles = os.path.join(report_dir, "deviation_tiles_B2_H16_N4096_d128_bf16.json")
    if os.path.exists(tiles):
        g = json.load(open(tiles))
        p = synth.make_qkv(2, 16, 4096, 128, "bf16", 3, qk_factor=4.0)
        scale = float(np.float32(1 / math.sqrt(128)))
        rows = rows_of(2, 16, 4096, 8, 4)
        ro, _ = oracle.attn_rows(p.q64, p.k64, p.v64, scale, rows, False)
        md += ["Tile sweep workload (B2 H16 N4096 d128 bf16, Q and K x4, seed [3, 4096, 0]); model on 256 sampled "
               "rows, GPU on all 16.8 M outputs (fp32-stored flavour).", "",
               "| Bc | order | model mean | model max | GPU mean | GPU max |", "|---|---|---|---|---|---|"]
        res["tiles"] = []
        for bc in (16, 32, 64, 128):
            for order in (0, 1):
                say("gpu check tiles", bc, order)
                e = E.flash_rows(p.q64, p.k64, p.v64, scale, rows, False, acc="f32", p="bf16", state="f32", out="f32",
                                 bc=bc, order=order)
                s = stats(e, ro)
                gr = [t for t in g["tiles"] if t["bc"] == bc and t["kv_order"] == order and t["br"] == 64][0]
                res["tiles"].append({"bc": bc, "order": order, "model": s, "gpu": gr["flash_f32out"]})
                md.append(f"| {bc} | {'desc' if order else 'asc'} | {s['mean']:.3e} | {s['max']:.3e} | "
                          f"{gr['flash_f32out']['mean']:.3e} | {gr['flash_f32out']['max']:.3e} |")
        md.append("")
    seq = os.path.join(report_dir, "deviation_seqlen_B1_H8_d64.json")
    if os.path.exists(seq):
        g = json.load(open(seq))
        md += ["Sequence-length workload (B1 H8 d64 bf16, seed [4, N, 0], default tiles Br 256, Bc 64); model on "
               "256 sampled rows.", "", "| N | model mean | model max | GPU mean | GPU max |", "|---|---|---|---|---|"]
        res["seqlen"] = []
        for N in (512, 1024, 2048, 4096):
            say("gpu check seqlen", N)
            p = synth.make_qkv(1, 8, N, 64, "bf16", 4)
            rows = rows_of(1, 8, N, 32, 5)
            ro, _ = oracle.attn_rows(p.q64, p.k64, p.v64, 0.125, rows, False)
            e = E.flash_rows(p.q64, p.k64, p.v64, 0.125, rows, False, acc="f32", p="bf16", state="f32", out="f32", bc=64)
            s = stats(e, ro)
            gr = [r for r in g["rows"] if r["dtype"] == "bf16" and r["N"] == N][0]
            res["seqlen"].append({"N": N, "model": s, "gpu": gr["flash"]})
            md.append(f"| {N} | {s['mean']:.3e} | {s['max']:.3e} | {gr['flash']['mean']:.3e} | {gr['flash']['max']:.3e} |")
        md.append("")
    return res, md


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=os.path.join(ROOT, "reports"))
    ap.add_argument("--gpu-reports", default=os.path.join(ROOT, "reports"))
    args = ap.parse_args()
    os.makedirs(args.out, exist_ok=True)
    t0 = time.time()
    out, md = {}, ["# Precision-emulating model: deviation from fp64", "",
                   "Command: `python -m tests.emulation_report` (repository root, CPU only). Model R1 is this "
                   "library's precision (fp32 arithmetic and state, P rounded to the input format); R2 also rounds "
                   "the running sum and output to the input format between key tiles (key/value-outer nest); the "
                   "baseline stores S and P in the input format. Statistics of |delta| against the fp64 plain "
                   "definition on sampled rows: max | mean | std.", ""]
    for name, fn in (("formats", sweep_formats), ("seqlen", sweep_seqlen), ("tiles", sweep_tiles)):
        r, m = fn()
        out[name] = r
        md += m + [""]
    r, m = gpu_cross_check(args.gpu_reports)
    out["gpu"] = r
    md += m
    out["oracle_threads"] = oracle.num_threads()
    md.append(f"Run time {time.time() - t0:.0f} s on {oracle.num_threads()} threads.")
    with open(os.path.join(args.out, "emulation_sweeps.json"), "w") as f:
        json.dump(out, f, indent=1)
    with open(os.path.join(args.out, "emulation_sweeps.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print("\n".join(md), flush=True)


if __name__ == "__main__":
    main()
