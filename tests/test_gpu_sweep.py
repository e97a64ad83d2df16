"""GPU: a seeded sweep of irregular shapes through the default forward (at
d = 128 in 16 bits: the pipelined steady state, the compiler-scheduled
diagonal and ragged tiles, and the persistent grid where the planner picks it)
and through the gradient (its pipelined blocks and loops), every element
against the fp64 oracle.

N values straddle the 32-row step, the 64-key tile and the 256-row workgroup;
B and H vary, causal and not, bf16 and fp16.  The cases are drawn once from a
fixed seed, so the sweep is the same on every run.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

_NS = [31, 32, 33, 63, 64, 65, 127, 129, 255, 256, 257, 300, 383, 511, 512, 513, 640, 767, 768, 769, 1000, 1025]


def _cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        out.append((int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.choice(_NS)),
                    bool(rng.integers(0, 2)), str(rng.choice(["bf16", "f16"]))))
    return out


FWD = _cases(24, 2024)
BWD = _cases(12, 2025)


@pytest.fixture(scope="module")
def attn():
    import torch
    assert torch.cuda.is_available()
    import tiled_online_softmax_fwd_amd as A
    A.lib()
    return A


def say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("B,H,N,causal,dtype", FWD)
def test_forward_sweep(attn, B, H, N, causal, dtype):
    import torch
    p = synth.make_qkv(B, H, N, 128, dtype, 90, variant=B * 100 + H)
    scale = float(np.float32(1 / math.sqrt(128)))
    say("forward sweep", B, H, N, "causal", causal, dtype)
    q, k, v = synth.upload(p)
    o, l = attn.fwd(q, k, v, scale=scale, causal=causal, out_fp32=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attn(p.q64, p.k64, p.v64, scale, causal)
    what = f"fwd B{B} H{H} N{N} causal={causal} {dtype}"
    gu.assert_close(gu.host(o), ro, gu.TOL_H16, what)
    gu.assert_lse(gu.host(l), rl, gu.TOL_LSE_H16, what)


@pytest.mark.parametrize("B,H,N,causal,dtype", BWD)
def test_backward_sweep(attn, B, H, N, causal, dtype):
    import torch
    p = synth.make_qkv(B, H, N, 128, dtype, 91, variant=B * 100 + H)
    g = synth.make_qkv(B, H, N, 128, dtype, 91, variant=B * 100 + H + 50)
    scale = float(np.float32(1 / math.sqrt(128)))
    say("backward sweep", B, H, N, "causal", causal, dtype)
    q, k, v = synth.upload(p)
    dout = synth.to_torch(g.q, dtype)
    o, lse = attn.fwd(q, k, v, scale=scale, causal=causal)
    grads = attn.bwd(q, k, v, o, dout, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    refs = oracle.attn_bwd(p.q64, p.k64, p.v64, g.q64, scale, causal)
    for name, x, r in zip(("dq", "dk", "dv"), grads, refs):
        err = gu.max_abs(gu.host(x), r)
        top = float(np.abs(r).max())
        assert err <= max(2e-2 * top, 1e-4), f"bwd B{B} H{H} N{N} causal={causal} {dtype} {name}: {err:.3e} vs {top:.3e}"
