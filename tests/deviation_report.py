"""Deviation reports of the GPU forward against the fp64 oracle (test
infrastructure; needs a GPU).  Not collected by pytest; run as

    python -m tests.deviation_report --which c3 c4 --out <dir>

It reproduces, on seeded synthetic inputs, the two measurements of the news
write-up of "Is Flash Attention Stable?": the deviation of the flash forward
from the fp64 "golden value" against sequence length (its Fig. 5, next to the
materialising baseline attention in the same precision), and against tile size
and block order (its Fig. 6).  Statistics are over every output element: max,
mean and std of |delta| and the mean of the signed delta.

  c3: B2 H16 N4096 d128 bf16, Q and K scaled by 4, non-causal; every
      (Br, Bc) in {16, 32, 64, 128}^2, both key-tile orders; plus the naive GPU
      baseline.
  c4: B1 H8 d64, N in {512, ..., 16384}, bf16, fp16 and fp32, non-causal, default
      tiles; flash vs fp64, naive vs fp64, flash vs naive.

The 16-bit rows use the fp32-output flavour (same kernel, fp32 store) so the
figures show the arithmetic, not the final rounding of O to bf16; the
bf16-stored output of the flash kernel is reported beside it.

Writes <out>/deviation_<which>.json and .md and prints the markdown.
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


def say(*a):
    print("[report]", *a, flush=True)


def stats(x, ref):
    d = np.asarray(x, np.float64) - ref
    a = np.abs(d)
    return {"max": float(a.max()), "mean": float(a.mean()), "std": float(a.std()), "signed_mean": float(d.mean())}


def host(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def fmt(s):
    return f"{s['max']:.3e} | {s['mean']:.3e} | {s['std']:.3e}"


def run_c3(A, torch):
    B, H, N, d = 2, 16, 4096, 128
    p = synth.make_qkv(B, H, N, d, "bf16", 3, qk_factor=4.0)
    scale = float(np.float32(1 / math.sqrt(d)))
    say("c3 oracle (full tensor)")
    t = time.perf_counter()
    ro, _ = oracle.attn(p.q64, p.k64, p.v64, scale)
    say(f"c3 oracle done in {time.perf_counter() - t:.1f} s")
    q, k, v = synth.upload(p)
    rows = []
    for br in (16, 32, 64, 128):
        for bc in (16, 32, 64, 128):
            for order in (0, 1):
                say("c3 flash", br, bc, order)
                o32, _ = A.fwd(q, k, v, scale=scale, br=br, bc=bc, kv_order=order, out_fp32=True)
                o16, _ = A.fwd(q, k, v, scale=scale, br=br, bc=bc, kv_order=order)
                torch.cuda.synchronize()
                rows.append({"br": br, "bc": bc, "kv_order": order,
                             "flash_f32out": stats(host(o32), ro), "flash_bf16out": stats(host(o16), ro)})
    say("c3 naive")
    on, _ = A.naive_fwd(q, k, v, scale=scale, out_fp32=True)
    torch.cuda.synchronize()
    naive = stats(host(on), ro)
    res = {"workload": "B2 H16 N4096 d128 bf16, Q and K x4, non-causal", "seed": [3, N, 0],
           "tiles": rows, "naive_f32out": naive}
    md = ["# Deviation from fp64 against tile size and key-tile order (B2 H16 N4096 d128 bf16, Q,K x4)", "",
          "Command: `python -m tests.deviation_report --which c3` (repository root, one MI355X).", "",
          "Statistics of |O_gpu - O_fp64| over all 16.8 M output elements; seeded inputs "
          "`default_rng([3, 4096, 0])`.  `f32 out` is the same kernel storing O in fp32.", "",
          "| Br | Bc | order | f32 out max | mean | std | bf16 out max | mean | std |", "|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        md.append(f"| {r['br']} | {r['bc']} | {'desc' if r['kv_order'] else 'asc'} | {fmt(r['flash_f32out'])} | "
                  f"{fmt(r['flash_bf16out'])} |")
    md += ["", f"Naive GPU baseline (S and P stored in bf16, fp32 accumulation, fp32 out): {fmt(naive)} "
               "(max | mean | std).", ""]
    return res, md


def run_c4(A, torch):
    d, H = 64, 8
    tiles = {dt: A.default_tiles({"bf16": A.BF16_OUT_F32, "f16": A.F16_OUT_F32, "f32": A.F32}[dt], d, False)
             for dt in ("bf16", "f16", "f32")}
    tile_txt = ", ".join(f"{dt} {br}x{bc}" for dt, (br, bc) in tiles.items())
    res = {"workload": f"B1 H8 d64 non-causal, default tiles (Br x Bc: {tile_txt})", "rows": []}
    md = ["# Deviation from fp64 against sequence length (B1 H8 d64, non-causal)", "",
          "Command: `python -m tests.deviation_report --which c4` (repository root, one MI355X).", "",
          "Statistics of |delta| over all output elements; seeded inputs `default_rng([4, N, 0])`. "
          "16-bit rows use fp32-stored outputs for both kernels. "
          f"Flash tiles (the defaults, Br x Bc): {tile_txt}.", "",
          "| dtype | N | flash vs fp64 max | mean | std | naive vs fp64 max | mean | std | flash vs naive max | mean | std |",
          "|---|---|---|---|---|---|---|---|---|---|---|"]
    for dtype in ("bf16", "f16", "f32"):
        for N in (512, 1024, 2048, 4096, 8192, 16384):
            p = synth.make_qkv(1, H, N, d, dtype, 4)
            say("c4 oracle", dtype, N)
            ro, _ = oracle.attn(p.q64, p.k64, p.v64, 0.125)
            q, k, v = synth.upload(p)
            say("c4 gpu", dtype, N)
            of, _ = A.fwd(q, k, v, scale=0.125, out_fp32=dtype != "f32")
            on, _ = A.naive_fwd(q, k, v, scale=0.125, out_fp32=dtype != "f32")
            torch.cuda.synchronize()
            hf, hn = host(of), host(on)
            r = {"dtype": dtype, "N": N, "flash": stats(hf, ro), "naive": stats(hn, ro), "flash_vs_naive": stats(hf, hn)}
            res["rows"].append(r)
            md.append(f"| {dtype} | {N} | {fmt(r['flash'])} | {fmt(r['naive'])} | {fmt(r['flash_vs_naive'])} |")
            del q, k, v, of, on
            torch.cuda.empty_cache()
    md.append("")
    return res, md


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--which", nargs="+", default=["c3", "c4"], choices=["c3", "c4"])
    ap.add_argument("--out", default=os.path.join(ROOT, "gpurun_out", "reports"))
    args = ap.parse_args()
    import torch
    import tiled_online_softmax_fwd_amd as A
    assert torch.cuda.is_available(), "needs a GPU"
    A.lib()
    os.makedirs(args.out, exist_ok=True)
    for w in args.which:
        res, md = {"c3": run_c3, "c4": run_c4}[w](A, torch)
        res["oracle_threads"] = oracle.num_threads()
        with open(os.path.join(args.out, f"deviation_{w}.json"), "w") as f:
            json.dump(res, f, indent=1)
        with open(os.path.join(args.out, f"deviation_{w}.md"), "w") as f:
            f.write("\n".join(md) + "\n")
        print("\n".join(md), flush=True)


if __name__ == "__main__":
    main()
