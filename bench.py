#!/usr/bin/env python3
"""Benchmark of the exact-attention forward on one MI355X.

Workload (the headline shape): B=1, H=32, N=8192, d=128, bf16 Q/K/V drawn
i.i.d. N(0,1) from a fixed seed, causal, scale = fp32(1/sqrt(128)).  One step
is one attn_fwd call over the whole batch (every step of the hot path: score
tiles, masking, online softmax, P.V, normalisation, lse).  Inputs are resident
in HBM before timing starts.

Prints ONE JSON line: throughput in TFLOP/s of algorithmic work
(4*B*H*N^2*d, halved for causal), the roofline of the kernel (HIP-event
duration per launch against the bf16 matrix-core peak), and the fp64 oracle
timed on the host cores on a bounded row sample of the same workload; the
sampled rows also give max/mean/std |delta| of the timed launch's output
against the fp64 definition.

Other modes (not the headline): --workload decode times attn_decode_fwd (a
query block against a key/value cache; priced against HBM bandwidth) and
--workload backward times attn_bwd (the gradient; 2.5x the forward's FLOPs),
--workload sparse times attn_fwd_sparse (block-sparse flags, FLOPs counted over
the attended pairs only).
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # 256 CU x 4096 dense bf16 FLOP/clk x 2.4 GHz (MI355X spec)
METRIC = "attention fwd TFLOP/s and % bf16 MFMA peak; max|Δ| vs FP64 oracle"
# default sources of a traffic record: the forward kernels, the generated
# pipeline and the host planner (which picks tiles and the persistent grid)
KERNEL_SOURCES = ["fwd_kernel.h", "fwd_pipe_asm.h", "attn_host.h"]
# sources of the gradient kernels' traffic record
BWD_SOURCES = ["bwd.hip", "bwd.h", "bwd_dq_pipe_asm.h", "bwd_dkdv_pipe_asm.h", "fwd_kernel.h", "attn_host.h"]
# ... and of the block-sparse forward's
SPARSE_SOURCES = ["fwd_kernel.h", "fwd_inst_sparse.hip", "attn_host.h"]


def kernel_hash(sources=None):
    h = hashlib.sha256()
    for f in (sources or KERNEL_SOURCES):
        with open(os.path.join(ROOT, "tiled_online_softmax_fwd_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_record(workload_key):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload_key)
    if not rec or rec.get("kernel_hash") != kernel_hash(rec.get("sources")):
        return None
    return rec


def environment(torch, A):
    """What a timing and a deviation depend on besides the inputs: the GPU and
    the software versions (the tutorial's reproducibility checklist names GPU,
    library versions, dtype, sizes and masking; the sizes and masking are in
    the config)."""
    props = torch.cuda.get_device_properties(0)
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"gpu": props.name, "arch": getattr(props, "gcnArchName", None), "rocm": rocm,
            "hip_runtime": torch.version.hip, "torch": torch.__version__,
            "libattn_version": int(A.lib().attn_version()), "dropout": None,
            "host_cpu": cpu, "host_threads": len(os.sched_getaffinity(0))}


def flops(B, H, N, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--B", type=int, default=1)
    ap.add_argument("--H", type=int, default=32)
    ap.add_argument("--N", type=int, default=8192)
    ap.add_argument("--d", type=int, default=128)
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "f16", "f32"])
    ap.add_argument("--no-causal", action="store_true")
    ap.add_argument("--br", type=int, default=0)
    ap.add_argument("--bc", type=int, default=0)
    ap.add_argument("--kv-order", type=int, default=0)
    ap.add_argument("--ref-slack", type=int, default=0,
                    help="lag allowed to the merge reference, base-2 units (0 = exact running maximum)")
    ap.add_argument("--generic-loop", action="store_true",
                    help="force the compiler-scheduled tile loop (no software-pipelined steady state)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for cpu_baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    ap.add_argument("--no-check", action="store_true", help="accepted for compatibility; the check is part of the cpu_baseline leg")
    ap.add_argument("--naive", action="store_true", help="accepted for compatibility: the baseline runs by default")
    ap.add_argument("--no-naive", action="store_true",
                    help="skip the materialising baseline (timed before the forward; it also brings the clock up)")
    ap.add_argument("--padding", default="none", choices=["none", "c2"],
                    help="key-padding mask of the forward: none, or c2 (batch 0 a random valid length, "
                         "batch 1 fully padded, the rest unpadded)")
    ap.add_argument("--workload", default="prefill", choices=["prefill", "decode", "backward", "sparse"],
                    help="prefill: the causal forward (default); decode: Nq query rows against a key/value "
                         "cache; backward: gradient of the forward; sparse: block-sparse forward")
    ap.add_argument("--pattern", default="local_global", choices=["local_global", "random"],
                    help="sparse: block flags (sliding window of blocks plus global blocks, or i.i.d.)")
    ap.add_argument("--block", type=int, default=64, help="sparse: block edge")
    ap.add_argument("--band", type=int, default=4, help="sparse local_global: window half-width in blocks")
    ap.add_argument("--n-global", type=int, default=1, help="sparse local_global: global row/column blocks")
    ap.add_argument("--density", type=float, default=0.5, help="sparse random: fraction of blocks on")
    ap.add_argument("--Nq", type=int, default=1, help="decode: query rows per head")
    ap.add_argument("--Nk", type=int, default=8192, help="decode: cached keys per head")
    ap.add_argument("--decode-B", type=int, default=8, help="decode: batch")
    ap.add_argument("--splits", type=int, default=0, help="decode: key chunks per head (0 = library choice)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the kernel shards over heads with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import tiled_online_softmax_fwd_amd as A

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    A.lib()

    if args.copy_probe:
        n = args.copy_probe * (1 << 20)
        src = torch.ones((n,), dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)
        return

    if args.workload == "decode":
        return run_decode(args, torch, synth, A)
    if args.workload == "backward":
        return run_backward(args, torch, synth, A)
    if args.workload == "sparse":
        return run_sparse(args, torch, synth, A)

    B, H, N, d = args.B, args.H, args.N, args.d
    causal = not args.no_causal
    scale = float(np.float32(1.0 / math.sqrt(d)))
    print(f"[bench] generating inputs B{B} H{H} N{N} d{d} {args.dtype} causal={causal}", file=sys.stderr, flush=True)
    p = synth.make_qkv(B, H, N, d, args.dtype, 5)
    q, k, v = synth.upload(p)
    pad = synth.c2_mask(B, N) if args.padding == "c2" else None
    pad_t = torch.from_numpy(pad).cuda() if pad is not None else None
    out = torch.empty((B, H, N, d), dtype=q.dtype, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    br, bc = A.default_tiles({"bf16": A.BF16, "f16": A.F16, "f32": A.F32}[args.dtype], d, causal)
    br = args.br or br
    bc = args.bc or bc

    # The materialising baseline (the pages' "baseline attention": S and P
    # stored in the input type) on the same inputs, timed first.  Besides
    # giving the comparison, its ~0.1 s of GPU work brings the shader clock up
    # before the forward's warm-up, so the forward is timed at its steady clock.
    naive = None
    o_naive = None
    if not args.no_naive and pad is None:
        need = A.lib().attn_naive_workspace_bytes(B, H, N, {"bf16": A.BF16, "f16": A.F16, "f32": A.F32}[args.dtype])
        ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
        o_naive = torch.empty_like(out)
        print(f"[bench] naive baseline (workspace {need / 2**30:.2f} GiB)", file=sys.stderr, flush=True)
        A.naive_fwd(q, k, v, scale=scale, causal=causal, out=o_naive, workspace=ws)
        torch.cuda.synchronize()
        stream0 = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream0)
        for _ in range(3):
            A.naive_fwd(q, k, v, scale=scale, causal=causal, out=o_naive, workspace=ws)
        e1.record(stream0)
        torch.cuda.synchronize()
        nms = e0.elapsed_time(e1) / 3
        fl0 = flops(B, H, N, d, causal)
        naive = {"ms": nms, "tflops": fl0 / (nms * 1e-3) / 1e12, "workspace_bytes": int(need),
                 "kernel": "naive (S and P stored in the input type)"}
        print(f"[bench] naive baseline {nms:.3f} ms", file=sys.stderr, flush=True)
        del ws

    def step():
        A.fwd(q, k, v, scale=scale, causal=causal, key_padding_mask=pad_t, out=out, lse=lse, br=br, bc=bc,
              kv_order=args.kv_order, ref_slack=args.ref_slack, generic_loop=args.generic_loop)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps, HIP events around every launch on the launch stream
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    free1 = torch.cuda.mem_get_info()[0]
    kms = np.array([a.elapsed_time(b) for a, b in ev])
    ms_per_step = wall * 1e3 / args.steps
    fl = flops(B, H, N, d, causal)
    value = fl / (ms_per_step * 1e-3) / 1e12
    kernel_tflops = fl / (kms.mean() * 1e-3) / 1e12
    print(f"[bench] {args.steps} steps: {ms_per_step:.4f} ms/step wall, kernel mean {kms.mean():.4f} ms "
          f"(median {np.median(kms):.4f}, min {kms.min():.4f})", file=sys.stderr, flush=True)

    # The matrix-core rate this part sustains at the clock it runs now: the
    # probe (independent bf16 matrix products only) timed on the same stream
    # right after the forward; the best of three launches of about 20 ms.
    ceiling = None
    if args.dtype != "f32":
        stream_p = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 64
        e0.record(stream_p)
        flp = A.probe_mfma(reps)
        e1.record(stream_p)
        torch.cuda.synchronize()
        reps = max(64, int(reps * 20.0 / max(e0.elapsed_time(e1), 1e-3)))
        best = 0.0
        for _ in range(3):
            e0.record(stream_p)
            flp = A.probe_mfma(reps)
            e1.record(stream_p)
            torch.cuda.synchronize()
            best = max(best, flp / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        ceiling = best
        print(f"[bench] matrix-core probe {ceiling:.0f} TFLOP/s", file=sys.stderr, flush=True)

    # cpu_baseline: the oracle on a bounded row sample of the same workload.  The
    # rows it computes are also compared with the output of the last timed launch
    # (max, mean and std of |delta| against the fp64 definition).
    cpu = None
    check = None
    if not args.no_cpu:
        import oracle
        threads = oracle.num_threads()
        rng = np.random.default_rng([99, N])

        def row_flops(rows):
            i = rows % N
            vis = (i + 1) if causal else np.full_like(i, N)
            return float(np.sum(4.0 * vis * d))

        def time_rows(nr):
            rows = np.sort(rng.choice(B * H * N, size=nr, replace=False))
            t = time.perf_counter()
            ro, rl = oracle.attn_rows(p.q64, p.k64, p.v64, scale, rows, causal, pad)
            return time.perf_counter() - t, row_flops(rows), rows, ro, rl

        dt, f, rows, _, _ = time_rows(min(B * H * N, 256))
        rate = f / max(dt, 1e-6)
        target = int(min(B * H * N, max(256, args.cpu_seconds * rate / (4.0 * d * (N / 2 if causal else N)))))
        print(f"[bench] cpu_baseline: {threads} threads, sampling {target} rows", file=sys.stderr, flush=True)
        dt, f, rows, ro, rl = time_rows(target)
        cpu = {"value": f / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
               "sample": f"{rows.size} uniformly drawn query rows of B{B} H{H} N{N} d{d} "
                         f"{'causal' if causal else 'full'} (fp64 plain definition, {dt:.1f} s)"}
        # one thread on the two small workloads, in full
        one = {}
        oracle.set_threads(1)
        try:
            for name, (b1, h1, n1, d1, dt1, causal1, mask1) in {
                    "C1 B1 H1 N128 d64 fp32": (1, 1, 128, 64, "f32", False, None),
                    "C2 B4 H16 N1024 d64 bf16 causal, key padding": (4, 16, 1024, 64, "bf16", True,
                                                                     synth.c2_mask(4, 1024))}.items():
                p1 = synth.make_qkv(b1, h1, n1, d1, dt1, 1 if name.startswith("C1") else 2)
                t = time.perf_counter()
                oracle.attn(p1.q64, p1.k64, p1.v64, 0.125, causal1, mask1)
                dt = time.perf_counter() - t
                one[name] = {"s": dt, "TFLOP/s": flops(b1, h1, n1, d1, causal1) / dt / 1e12}
        finally:
            oracle.set_threads(threads)
        cpu["one_thread"] = one
        o_host = out.to(torch.float64).cpu().numpy().reshape(-1, d)[rows]
        l_host = lse.cpu().numpy().astype(np.float64).reshape(-1)[rows]
        err = np.abs(o_host - ro)
        fin = np.isfinite(rl)
        check = {"rows": int(rows.size), "max_abs": float(err.max()), "mean_abs": float(err.mean()),
                 "std_abs": float(err.std()), "lse_max_abs": float(np.abs(l_host[fin] - rl[fin]).max()),
                 "output": args.dtype}
        if o_naive is not None:
            en = np.abs(o_naive.to(torch.float64).cpu().numpy().reshape(-1, d)[rows] - ro)
            check["naive_vs_fp64"] = {"max_abs": float(en.max()), "mean_abs": float(en.mean()),
                                      "std_abs": float(en.std())}
        if not fin.all():
            # rows with no visible key: exactly (0, -inf) on both sides
            check["empty_rows"] = int((~fin).sum())
            check["empty_rows_exact"] = bool(np.all(np.isneginf(l_host[~fin])) and np.all(o_host[~fin] == 0))

    wk = f"B{B}_H{H}_N{N}_d{d}_{args.dtype}_{'causal' if causal else 'full'}_br{br}_bc{bc}"
    if pad is not None:
        wk += f"_pad{args.padding}"
    if args.ref_slack:
        wk += f"_slack{args.ref_slack}"
    if args.generic_loop:
        wk += "_generic"
    tr = traffic_record(wk)
    roof = {"bound": "mfma", "achieved": kernel_tflops, "peak": PEAK_BF16_TFLOPS if args.dtype != "f32" else 157.3,
            "unit": "TFLOP/s", "frac": kernel_tflops / (PEAK_BF16_TFLOPS if args.dtype != "f32" else 157.3),
            "traffic": (tr["hbm_bytes_per_launch"] if tr else None),
            "kernel": ("fwd_m32_h16" if args.dtype != "f32"
                       else "fwd_m32_f32_db" if 4 * bc * d * 4 <= 128 * 1024 else "fwd_m32_f32"),
            "kernel_ms_mean": float(kms.mean()), "kernel_ms_median": float(np.median(kms)), "kernel_ms_min": float(kms.min()),
            "achieved_median": fl / (np.median(kms) * 1e-3) / 1e12}
    if ceiling:
        roof["measured_ceiling"] = ceiling
        roof["frac_of_measured_ceiling"] = kernel_tflops / ceiling
        roof["ceiling_probe"] = "independent bf16 32x32x16 matrix products only (attn_probe_mfma), timed after the forward"
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": f"B{B} H{H} N{N} d{d} {args.dtype} {'causal' if causal else 'non-causal'} attention forward",
                   "B": B, "H": H, "N": N, "d": d, "causal": causal, "br": br, "bc": bc,
                   "kv_order": args.kv_order, "ref_slack": args.ref_slack, "key_padding": args.padding,
                   "generic_loop": bool(args.generic_loop), "global_batch": B, "seq_len": N, "parallelism": "single GPU"},
        "pct_peak": 100.0 * value / (PEAK_BF16_TFLOPS if args.dtype != "f32" else 157.3),
        "check_vs_fp64_oracle": check,
        "roofline": roof,
        "cpu_baseline": cpu,
        # the library keeps no workspace: free device memory is unchanged over
        # the timed calls, while the score matrix alone would have taken this
        "memory": {"library_workspace_bytes": 0, "device_free_delta_bytes": int(free0 - free1),
                   "score_matrix_bytes_if_stored": int(B * H * N * N * (4 if args.dtype == "f32" else 2))},
    }
    if naive:
        line["naive_baseline"] = naive
    line["env"] = environment(torch, A)
    print(json.dumps(line), flush=True)


def run_backward(args, torch, synth, A):
    """Gradient of the forward on the prefill shape; algorithmic work is the five
    products S, dP, dV, dK, dQ (2.5x the forward's FLOPs, halved for causal)."""
    B, H, N, d = args.B, args.H, args.N, args.d
    if args.dtype == "f32":
        print("the backward takes 16-bit inputs", file=sys.stderr)
        sys.exit(2)
    causal = not args.no_causal
    scale = float(np.float32(1.0 / math.sqrt(d)))
    print(f"[bench] backward inputs B{B} H{H} N{N} d{d} {args.dtype}", file=sys.stderr, flush=True)
    p = synth.make_qkv(B, H, N, d, args.dtype, 5)
    g = synth.make_qkv(B, H, N, d, args.dtype, 5, variant=1)
    q, k, v = synth.upload(p)
    dout = synth.to_torch(g.q, args.dtype)
    o, lse = A.fwd(q, k, v, scale=scale, causal=causal)
    ws = torch.empty((max(A.lib().attn_bwd_workspace_bytes(B, H, N), 16),), dtype=torch.uint8, device="cuda")
    res = {}

    def step():
        res["g"] = A.bwd(q, k, v, o, dout, lse, scale=scale, causal=causal, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kms = np.array([a.elapsed_time(b) for a, b in ev])
    fl = 2.5 * flops(B, H, N, d, causal)
    tf = fl / (kms.mean() * 1e-3) / 1e12
    print(f"[bench] backward {args.steps} steps: mean {kms.mean():.3f} ms, {tf:.0f} TFLOP/s", file=sys.stderr)
    check = cpu = None
    if not args.no_cpu:
        import oracle
        heads = min(H, 2)
        t = time.perf_counter()
        rq, rk, rv = oracle.attn_bwd(p.q64[:, :heads], p.k64[:, :heads], p.v64[:, :heads], g.q64[:, :heads],
                                     scale, causal)
        dt = time.perf_counter() - t
        sample_fl = 2.5 * flops(1, heads, N, d, causal)
        cpu = {"value": sample_fl / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"gradient of {heads} of the {B * H} heads (fp64 chain rule, {dt:.1f} s)"}
        check = {"heads_checked": heads, "time_s": dt}
        for name, x, r in zip(("dq", "dk", "dv"), res["g"], (rq, rk, rv)):
            e = np.abs(x[:, :heads].to(torch.float64).cpu().numpy() - r)
            check[name] = {"max_abs": float(e.max()), "mean_abs": float(e.mean()), "max_ref": float(np.abs(r).max())}
    # HBM bytes of the three kernels of one call, from the committed counter
    # summary when it was taken on the current gradient sources
    tr = traffic_record(f"backward_B{B}_H{H}_N{N}_d{d}_{args.dtype}_{'causal' if causal else 'full'}")
    line = {
        "metric": "attention backward TFLOP/s (5 products, halved for causal)", "value": fl / (wall / args.steps) / 1e12,
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": args.dtype, "data": "synthetic",
        "config": {"workload": f"backward B{B} H{H} N{N} d{d} {args.dtype} {'causal' if causal else 'non-causal'}",
                   "B": B, "H": H, "N": N, "d": d, "causal": causal},
        "check_vs_fp64_oracle": check,
        "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / PEAK_BF16_TFLOPS, "traffic": (tr["hbm_bytes_per_launch"] if tr else None),
                     "kernel": "bwd_pre + bwd_dkdv + bwd_dq",
                     "kernel_ms_mean": float(kms.mean()), "kernel_ms_median": float(np.median(kms)), "kernel_ms_min": float(kms.min())},
        "cpu_baseline": cpu,
    }
    line["env"] = environment(torch, A)
    print(json.dumps(line), flush=True)


def attended_pairs(bm, N, block, causal):
    """Number of (row, key) pairs the block flags bm [B, H, nb, nb] switch on,
    after causality (counting only)."""
    nb = bm.shape[-1]
    starts = np.arange(nb, dtype=np.int64) * block
    width = np.minimum(block, N - starts)                         # rows (= keys) per block
    full = width[:, None] * width[None, :]                        # [row block, key block]
    if causal:
        # blocks are square and aligned: below the diagonal every pair, above
        # none, on it the r(r + 1)/2 pairs with key <= row
        a = np.arange(nb)[:, None]
        b = np.arange(nb)[None, :]
        per_block = np.where(b < a, full, np.where(b == a, width[:, None] * (width[:, None] + 1) // 2, 0))
    else:
        per_block = full
    return int((bm.astype(np.int64) * per_block[None, None]).sum())


def run_sparse(args, torch, synth, A):
    """Block-sparse forward on the prefill shape; algorithmic work is 4*d FLOPs
    per attended (row, key) pair."""
    B, H, N, d = args.B, args.H, args.N, args.d
    if args.dtype == "f32":
        print("the block-sparse forward takes 16-bit inputs", file=sys.stderr)
        sys.exit(2)
    causal = not args.no_causal
    scale = float(np.float32(1.0 / math.sqrt(d)))
    blk = args.block
    bm = synth.block_mask(B, H, N, blk, 5, args.pattern, args.density, args.band, args.n_global)
    pairs = attended_pairs(bm, N, blk, causal)
    pat = (f"window +-{args.band} blocks + {args.n_global} global" if args.pattern == "local_global"
           else f"random density {args.density}")
    print(f"[bench] sparse B{B} H{H} N{N} d{d} {args.dtype} block {blk} {pat}, "
          f"{pairs / (B * H * N * N):.4f} of all pairs", file=sys.stderr, flush=True)
    p = synth.make_qkv(B, H, N, d, args.dtype, 5)
    q, k, v = synth.upload(p)
    bmt = torch.from_numpy(bm).cuda()
    out = torch.empty((B, H, N, d), dtype=q.dtype, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")

    def step():
        A.fwd_sparse(q, k, v, bmt, block=blk, scale=scale, causal=causal, out=out, lse=lse,
                     br=args.br or None, bc=args.bc or None)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kms = np.array([a.elapsed_time(b) for a, b in ev])
    fl = 4.0 * d * pairs
    tf = fl / (kms.mean() * 1e-3) / 1e12
    print(f"[bench] sparse {args.steps} steps: mean {kms.mean():.4f} ms, {tf:.0f} TFLOP/s", file=sys.stderr)
    check = cpu = None
    if not args.no_cpu:
        import oracle
        heads = H                     # every head of the first batch entry (about a second of CPU work)
        t = time.perf_counter()
        ro, rl = oracle.attn_blockmask(p.q64[:1, :heads], p.k64[:1, :heads], p.v64[:1, :heads], scale,
                                       bm[:1, :heads], blk, causal)
        dt = time.perf_counter() - t
        o64 = out[:1, :heads].to(torch.float64).cpu().numpy()
        l64 = lse[:1, :heads].to(torch.float64).cpu().numpy()
        e = np.abs(o64 - ro)
        fin = np.isfinite(rl)
        sample_pairs = attended_pairs(bm[:1, :heads], N, blk, causal)
        check = {"heads_checked": heads, "rows_checked": int(heads * N), "time_s": dt, "max_abs": float(e.max()),
                 "mean_abs": float(e.mean()), "lse_max_abs": float(np.abs(l64[fin] - rl[fin]).max()),
                 "output": args.dtype}
        cpu = {"value": 4.0 * d * sample_pairs / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
               "kind": "oracle", "sample": f"all rows of {heads} of the {B * H} heads, {sample_pairs} attended pairs "
                                           f"(fp64 plain definition, {dt:.2f} s)"}
    # HBM bytes per launch, from the committed counter summary when it was
    # taken on the current sources (only the default window pattern has one)
    tr = None
    if args.pattern == "local_global" and not args.br and not args.bc:
        tr = traffic_record(f"sparse_B{B}_H{H}_N{N}_d{d}_{args.dtype}_{'causal' if causal else 'full'}_block{blk}_"
                            f"band{args.band}_global{args.n_global}")
    line = {
        "metric": "block-sparse attention fwd TFLOP/s over attended pairs", "value": fl / (wall / args.steps) / 1e12,
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": args.dtype, "data": "synthetic",
        "config": {"workload": f"block-sparse B{B} H{H} N{N} d{d} {args.dtype} {'causal' if causal else 'non-causal'}, "
                               f"block {blk}, {pat}", "B": B, "H": H, "N": N, "d": d, "causal": causal,
                   "attended_fraction": pairs / (B * H * N * N)},
        "check_vs_fp64_oracle": check,
        "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / PEAK_BF16_TFLOPS, "traffic": (tr["hbm_bytes_per_launch"] if tr else None),
                     "kernel": "fwd_m32_h16 (block-sparse)",
                     "kernel_ms_mean": float(kms.mean()), "kernel_ms_median": float(np.median(kms)), "kernel_ms_min": float(kms.min())},
        "cpu_baseline": cpu,
    }
    line["env"] = environment(torch, A)
    print(json.dumps(line), flush=True)


def run_decode(args, torch, synth, A):
    """Key/value-cache decoding: Nq query rows per head against Nk cached keys.
    Bound by reading K and V once; priced against the HBM bandwidth."""
    B, H, Nq, Nk, d = args.decode_B, args.H, args.Nq, args.Nk, args.d
    if args.dtype == "f32":
        print("the decode path takes 16-bit inputs", file=sys.stderr)
        sys.exit(2)
    causal = not args.no_causal
    scale = float(np.float32(1.0 / math.sqrt(d)))
    print(f"[bench] decode inputs B{B} H{H} Nq{Nq} Nk{Nk} d{d} {args.dtype}", file=sys.stderr, flush=True)
    kv = synth.make_qkv(B, H, Nk, d, args.dtype, 7)
    qq = synth.make_qkv(B, H, Nq, d, args.dtype, 7, variant=1)
    q = synth.to_torch(qq.q, args.dtype)
    k = synth.to_torch(kv.k, args.dtype)
    v = synth.to_torch(kv.v, args.dtype)
    out = torch.empty((B, H, Nq, d), dtype=q.dtype, device="cuda")
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    need = A.lib().attn_decode_workspace_bytes(B, H, Nq, Nk, d, args.splits)
    ws = torch.empty((max(need, 16),), dtype=torch.uint8, device="cuda")

    def step():
        A.decode_fwd(q, k, v, scale=scale, causal=causal, out=out, lse=lse, num_splits=args.splits, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kms = np.array([a.elapsed_time(b) for a, b in ev])
    esz = 2
    algo_bytes = B * H * (2 * Nk * d * esz + 2 * Nq * d * esz + 4 * Nq)     # K, V, Q, O, lse
    gbs = algo_bytes / (kms.mean() * 1e-3) / 1e9
    tr = traffic_record(f"decode_B{B}_H{H}_Nq{Nq}_Nk{Nk}_d{d}_{args.dtype}_{'causal' if causal else 'full'}_s{args.splits}")
    print(f"[bench] decode {args.steps} steps: kernel mean {kms.mean() * 1e3:.1f} us, {gbs:.0f} GB/s", file=sys.stderr)
    check = cpu = None
    if not args.no_cpu:
        import oracle
        t = time.perf_counter()
        ro, rl = oracle.attn_kv(qq.q64, kv.k64, kv.v64, scale, causal)
        dt = time.perf_counter() - t
        o_host = out.to(torch.float64).cpu().numpy()
        err = np.abs(o_host - ro)
        check = {"rows": int(B * H * Nq), "max_abs": float(err.max()), "mean_abs": float(err.mean()),
                 "std_abs": float(err.std()), "output": args.dtype}
        flops = 4.0 * B * H * Nq * Nk * d
        cpu = {"value": algo_bytes / dt / 1e9, "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"all {B * H * Nq} rows (fp64 plain definition, {dt:.2f} s, {flops / dt / 1e9:.1f} GFLOP/s)"}
    line = {
        "metric": "decode attention HBM GB/s (K and V read once)", "value": gbs, "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": args.dtype, "data": "synthetic",
        "config": {"workload": f"decode B{B} H{H} Nq{Nq} Nk{Nk} d{d} {args.dtype}", "B": B, "H": H, "Nq": Nq,
                   "Nk": Nk, "d": d, "causal": causal, "num_splits": args.splits, "workspace_bytes": int(need)},
        "check_vs_fp64_oracle": check,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": 8000.0, "unit": "GB/s", "frac": gbs / 8000.0,
                     "traffic": (tr["hbm_bytes_per_launch"] if tr else None), "kernel": "dec_split + dec_merge", "kernel_ms_mean": float(kms.mean()), "kernel_ms_median": float(np.median(kms)), "kernel_ms_min": float(kms.min())},
        "cpu_baseline": cpu,
    }
    line["env"] = environment(torch, A)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
