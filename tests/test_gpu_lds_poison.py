"""GPU: the LDS-poisoning debug build against the release build.

libattn_poison.so (built from the same sources with ATTN_LDS_POISON) writes
NaN into the LDS slots of every tile copy before issuing it, after the wait
that freed them.  A kernel whose reads are all ordered after the copies they
need never sees the NaN, so every output must be bitwise equal to the release
build's (the poisoned build runs the compiler-scheduled loop, which the
release build's generic_loop option also runs).  A missing wait or barrier
would read NaN instead of the previous tile's finite data and fail here.

Each library runs in a child process of its own; the cases cover the 16-bit
forward (plain, causal, ragged, padded, both fold orders), the fp32 forward,
the block-sparse walk, the cache path and the gradient (whose pipelined loops
in the release build are thereby checked bitwise against the C++ loops).
"""
import os
import subprocess
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "tiled_online_softmax_fwd_amd")

CHILD = r"""
import sys
import numpy as np
sys.path.insert(0, sys.argv[1])
import torch
import tiled_online_softmax_fwd_amd as A
A.LIB_PATH = sys.argv[2]
A.lib()
out = sys.argv[3]
dev = "cuda:0"
res = {}
def t(B, H, N, d, dt, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return [torch.randn(B, H, N, d, generator=g).to(dt).to(dev) for _ in range(3)]
def put(name, *ts):
    torch.cuda.synchronize()
    for i, x in enumerate(ts):
        res[f"{name}_{i}"] = x.float().cpu().numpy()
    print("[case]", name, flush=True)
bf, f16, f32 = torch.bfloat16, torch.float16, torch.float32
q, k, v = t(1, 4, 1000, 128, bf, 1)
put("fwd_bf16_d128_causal", *A.fwd(q, k, v, scale=128 ** -0.5, causal=True, generic_loop=True))
put("fwd_bf16_d128_full_o1", *A.fwd(q, k, v, scale=128 ** -0.5, kv_order=1, generic_loop=True))
q, k, v = t(1, 16, 2048, 128, bf, 2)
put("fwd_bf16_d128_c5like", *A.fwd(q, k, v, scale=128 ** -0.5, causal=True, generic_loop=True))
# default options: the release build pipelines this call (bitwise equal to its
# generic loop), the poisoned build cannot
put("fwd_bf16_d128_default", *A.fwd(q, k, v, scale=128 ** -0.5, causal=True))
q, k, v = t(4, 2, 301, 64, f16, 3)
mask = torch.zeros(4, 301, dtype=torch.uint8)
mask[0, 150:] = 1; mask[1, :] = 1; mask[2, :200] = 1
mask = mask.to(dev)
put("fwd_f16_d64_causal_mask", *A.fwd(q, k, v, scale=0.125, causal=True, key_padding_mask=mask, out_fp32=True))
put("fwd_f16_d64_128x64_mask", *A.fwd(q, k, v, scale=0.125, key_padding_mask=mask, br=128, bc=64, out_fp32=True))
q, k, v = t(1, 2, 333, 64, f32, 4)
put("fwd_f32_d64_causal", *A.fwd(q, k, v, scale=0.125, causal=True))
m32 = (torch.arange(333, device=dev) % 7 == 3).to(torch.uint8)[None].contiguous()
put("fwd_f32_d64_causal_mask", *A.fwd(q, k, v, scale=0.125, causal=True, key_padding_mask=m32))
q, k, v = t(1, 2, 1000, 128, bf, 5)
nb = (1000 + 63) // 64
bm = torch.zeros(1, 2, nb, nb, dtype=torch.uint8)
for i in range(nb):
    for j in range(nb):
        bm[:, :, i, j] = 1 if abs(i - j) <= 2 or j == 0 else 0
put("fwd_sparse_bf16_d128", *A.fwd_sparse(q, k, v, bm.to(dev), block=64, scale=128 ** -0.5, causal=True))
q, k, v = t(2, 4, 1000, 128, bf, 6)
qd = q[:, :, :3].contiguous()
put("decode_bf16_d128", *A.decode_fwd(qd, k, v, scale=128 ** -0.5, causal=True))
dmask = (torch.arange(1000, device=dev) > 700).to(torch.uint8)[None].repeat(2, 1).contiguous()
put("decode_bf16_d128_mask", *A.decode_fwd(qd, k, v, scale=128 ** -0.5, causal=True, key_padding_mask=dmask))
# the release build's dK/dV and dQ kernels run their full tiles through their
# software pipelines at d = 128, the poisoned build through the C++ loops
for d, N, causal, dt, name in ((128, 500, True, bf, "bf16"), (64, 500, True, bf, "bf16"),
                               (128, 2048, False, f16, "f16"), (128, 1536, True, bf, "bf16")):
    q, k, v = t(1, 2, N, d, dt, 7 + d + N)
    o, lse = A.fwd(q, k, v, scale=d ** -0.5, causal=causal, generic_loop=True)
    g = torch.Generator(device="cpu").manual_seed(9)
    do = torch.randn(1, 2, N, d, generator=g).to(dt).to(dev)
    put(f"bwd_{name}_d{d}_N{N}_c{int(causal)}", *A.bwd(q, k, v, o, do, lse, scale=d ** -0.5, causal=causal))
np.savez(out, **res)
print("done", flush=True)
"""


def run_child(lib, out, trace=False):
    env = dict(os.environ)
    env.pop("ATTN_TRACE", None)
    if trace:
        env["ATTN_TRACE"] = "1"
    r = subprocess.run([sys.executable, "-u", "-c", CHILD, ROOT, lib, out], capture_output=True, text=True,
                       env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "done" in r.stdout
    return r


def test_poisoned_build_matches_release_bitwise(tmp_path):
    rel, poi = os.path.join(PKG, "libattn.so"), os.path.join(PKG, "libattn_poison.so")
    assert os.path.exists(poi), "libattn_poison.so not built (tiled_online_softmax_fwd_amd/build.py)"
    print("[case] release build", flush=True)
    run_child(rel, str(tmp_path / "rel.npz"))
    print("[case] poisoned build", flush=True)
    r = run_child(poi, str(tmp_path / "poi.npz"), trace=True)
    # the poisoned build runs the compiler-scheduled loop at the 256 x 64 tile
    # even for the call with default options, which the release build
    # pipelines: the switch was compiled in
    lines = [l for l in r.stderr.splitlines() if l.startswith("attn: attn_fwd kernel=fwd_m32_h16<bf16,d128,256x64>")]
    assert len(lines) >= 4 and all("loop=generic" in l for l in lines), "\n".join(lines)
    bl = [l for l in r.stderr.splitlines() if l.startswith("attn: attn_bwd ")]
    assert len(bl) == 4 and all("loops=generic" in l for l in bl), "\n".join(bl)
    a, b = np.load(tmp_path / "rel.npz"), np.load(tmp_path / "poi.npz")
    assert sorted(a.files) == sorted(b.files)
    for name in sorted(a.files):
        x, y = a[name], b[name]
        assert not np.isnan(y).any() or np.isnan(x).any(), f"{name}: NaN from the poisoned build"
        assert np.array_equal(x, y, equal_nan=True), \
            f"{name}: max |delta| {float(np.nanmax(np.abs(x.astype(np.float64) - y))):.3e}"
