"""GPU: ATTN_TRACE=1 names what each launching entry point actually ran.

One child process (the variable is read once per process) makes a forward at
the benchmarked shape (persistent grid, pipelined loop), a small forward
(one workgroup per query tile), a padded forward, the fp32 forward, a cache
decode, the naive baseline and the backward, and the parent checks the
"attn: " lines it wrote to stderr, in call order."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROG = r"""
import sys
sys.path.insert(0, sys.argv[1])
import torch
import tiled_online_softmax_fwd_amd as A
dev = "cuda:0"
cus = torch.cuda.get_device_properties(0).multi_processor_count
print("cus", cus, flush=True)
def qkv(B, H, N, d, dt=torch.bfloat16):
    g = torch.Generator(device="cpu").manual_seed(N)
    return [torch.randn(B, H, N, d, generator=g).to(dt).to(dev) for _ in range(3)]
q, k, v = qkv(1, 32, 8192, 128)
A.fwd(q, k, v, scale=128 ** -0.5, causal=True)
q, k, v = qkv(1, 8, 1024, 128)
A.fwd(q, k, v, scale=128 ** -0.5, causal=True)
mask = torch.zeros(1, 1024, dtype=torch.uint8, device=dev)
mask[:, 1000:] = 1
A.fwd(q, k, v, scale=128 ** -0.5, causal=False, key_padding_mask=mask)
qf, kf, vf = qkv(1, 2, 300, 64, torch.float32)
A.fwd(qf, kf, vf, scale=0.125)
qd = q[:, :, :1].contiguous()
A.decode_fwd(qd, k, v, scale=128 ** -0.5, causal=True)
A.naive_fwd(qf, kf, vf, scale=-0.125)
o, lse = A.fwd(q, k, v, scale=128 ** -0.5, causal=True)
A.bwd(q, k, v, o, torch.randn_like(o), lse, scale=128 ** -0.5, causal=True)
torch.cuda.synchronize()
print("done", flush=True)
"""


def test_trace_names_the_launched_kernels():
    env = dict(os.environ)
    env["ATTN_TRACE"] = "1"
    print("[case] ATTN_TRACE child process", flush=True)
    r = subprocess.run([sys.executable, "-u", "-c", PROG, ROOT], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "done" in r.stdout
    cus = int(r.stdout.split()[1])
    lines = [l for l in r.stderr.splitlines() if l.startswith("attn: ")]
    assert len(lines) == 8, "\n".join(lines)
    big, small, padded, f32, dec, naive, fwd2, bwd = lines
    assert "attn_fwd kernel=fwd_m32_h16<bf16,d128,256x64> B=1 H=32 N=8192 causal=1 mask=0" in big
    assert "loop=pipelined" in big
    if cus == 256:
        # 32 heads x 16 causal pairs of query tiles over 256 compute units
        assert f"grid=256 block=512 persistent=1 xcd_affine=1" in big
    assert "kernel=fwd_m32_h16<bf16,d128,256x64> B=1 H=8 N=1024 causal=1" in small
    assert "loop=pipelined grid=32 block=512 persistent=0" in small
    assert "kernel=fwd_m32_h16_masked<bf16,d128,256x64>" in padded and "mask=1" in padded
    assert "loop=generic" in padded
    assert "kernel=fwd_m32_f32_db<f32,d64,128x64> B=1 H=2 N=300" in f32 and "grid=6 block=256" in f32
    assert "attn_decode_fwd kernel=dec_split+dec_merge<bf16,d128> B=1 H=8 Nq=1 Nk=1024" in dec
    assert "attn_naive_fwd kernel=gemm_simt+row_softmax+gemm_simt<f32,d64>" in naive
    assert "attn_fwd kernel=fwd_m32_h16<bf16,d128,256x64> B=1 H=8 N=1024" in fwd2
    assert "attn_bwd kernel=bwd_pre+bwd_dkdv+bwd_dq<bf16,d128>" in bwd and "loops=pipelined" in bwd
