"""GPU parity for every finite scale, not only the pages' 1/sqrt(d): negative
scales (run as |scale| on scores negated through Q) and scale 0 (every score 0:
the output is the mean of the visible value rows, lse = ln(count)), against the
fp64 oracle, which takes any scale as given.  Forward tiles (the pipelined
default, the 16x16 kernel, fp32, padding), the cache path, the block-sparse
forward, the gradient and the materialising baseline."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SCALES = [-0.125, 0.0, -1.5]


@pytest.fixture(scope="module")
def attn():
    import torch
    assert torch.cuda.is_available()
    import tiled_online_softmax_fwd_amd as A
    A.lib()
    return A


def say(*a):
    print("[case]", *a, flush=True)


def fp32_gate(p, scale):
    """fp32 gate for a scale of any size: scores of magnitude S carry an ulp of
    2^(floor(log2 S) - 23) and the output moves by at most 2 max|v| per unit of
    score error (d o / d s_j = p_j (v_j - o)); 4 ulps of score error on top of
    the 1e-5 of the N(0,1), 1/sqrt(d) workloads."""
    smax = abs(scale) * float(np.abs(np.einsum("bhid,bhjd->bhij", p.q64, p.k64)).max())
    ulp = 2.0 ** (np.floor(np.log2(max(smax, 1e-30))) - 23)
    return gu.TOL_F32 + 8 * ulp * float(np.abs(p.v64).max())


def mask_for(B, N, seed):
    rng = np.random.default_rng([seed, N, 99])
    m = (rng.random((B, N)) < 0.2).astype(np.uint8)
    m[0, :] = 0
    return m


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("dtype,d,br,bc", [("bf16", 128, 0, 0), ("f16", 64, 0, 0), ("bf16", 128, 64, 16),
                                           ("f32", 128, 0, 0), ("f32", 64, 16, 32)])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_any_scale(attn, scale, dtype, d, br, bc, causal):
    import torch
    B, H, N = 2, 2, 700
    p = synth.make_qkv(B, H, N, d, dtype, 90, variant=d)
    tol = gu.TOL_F32 if dtype == "f32" else gu.TOL_H16
    if dtype == "f32":
        tol = fp32_gate(p, scale)
    q, k, v = gu.upload(p)
    for masked in (False, True):
        mask = mask_for(B, N, 91) if masked else None
        say("forward", dtype, d, br, bc, "causal", causal, "scale", scale, "mask", masked)
        o, l = attn.fwd(q, k, v, scale=scale, causal=causal, key_padding_mask=gu.mask_to_torch(mask),
                        out_fp32=dtype != "f32", br=br or None, bc=bc or None)
        torch.cuda.synchronize()
        ro, rl = oracle.attn(p.q64, p.k64, p.v64, scale, causal, mask)
        gu.assert_close(gu.host(o), ro, tol, "O")
        gu.assert_lse(gu.host(l), rl, tol if dtype == "f32" else gu.TOL_LSE_H16, "lse")


@pytest.mark.parametrize("scale", SCALES)
def test_pipelined_and_persistent_paths_any_scale(attn, scale):
    """B1 H16 N8192 causal runs the persistent grid and the pipelined steady
    tiles; sampled rows against the oracle."""
    import torch
    p = synth.make_qkv(1, 16, 8192, 128, "bf16", 92)
    say("pipelined + persistent, scale", scale)
    q, k, v = gu.upload(p)
    o, l = attn.fwd(q, k, v, scale=scale, causal=True, out_fp32=True)
    torch.cuda.synchronize()
    rows = gu.sample_rows(1, 16, 8192, per_head=24, seed=93)
    ro, rl = oracle.attn_rows(p.q64, p.k64, p.v64, scale, rows, True)
    gu.assert_close(gu.host(o).reshape(-1, 128)[rows], ro, gu.TOL_H16, "O rows")
    gu.assert_lse(gu.host(l).reshape(-1)[rows], rl, gu.TOL_LSE_H16, "lse rows")


def test_zero_scale_is_the_mean_of_visible_values(attn):
    """scale 0: O is the plain mean of the visible V rows and lse = ln(count)
    (causal row i sees i + 1 keys), on the pipelined default path."""
    import torch
    p = synth.make_qkv(1, 2, 1024, 128, "bf16", 94)
    q, k, v = gu.upload(p)
    say("scale 0: mean of visible values")
    o, l = attn.fwd(q, k, v, scale=0.0, causal=True, out_fp32=True)
    torch.cuda.synchronize()
    cnt = np.arange(1, 1025, dtype=np.float64)
    mean = np.cumsum(p.v64, axis=2) / cnt[None, None, :, None]
    gu.assert_close(gu.host(o), mean, gu.TOL_H16, "mean")
    assert np.allclose(gu.host(l), np.log(cnt)[None, None, :], atol=1e-5)


@pytest.mark.parametrize("scale", SCALES)
def test_cache_path_any_scale(attn, scale):
    import torch
    kv = synth.make_qkv(2, 3, 1000, 128, "bf16", 95)
    qq = synth.make_qkv(2, 3, 5, 128, "bf16", 95, variant=1)
    tq, tk, tv = (synth.to_torch(x, "bf16") for x in (qq.q, kv.k, kv.v))
    for causal in (False, True):
        say("cache path scale", scale, "causal", causal)
        o, l = attn.decode_fwd(tq, tk, tv, scale=scale, causal=causal, out_fp32=True)
        torch.cuda.synchronize()
        ro, rl = oracle.attn_kv(qq.q64, kv.k64, kv.v64, scale, causal)
        gu.assert_close(gu.host(o), ro, gu.TOL_H16, "O")
        gu.assert_lse(gu.host(l), rl, gu.TOL_LSE_H16, "lse")


@pytest.mark.parametrize("scale", SCALES)
def test_block_sparse_any_scale(attn, scale):
    import torch
    B, H, N = 1, 2, 512
    p = synth.make_qkv(B, H, N, 128, "bf16", 96)
    nb = N // 64
    bm = synth.block_mask(B, H, N, 64, 96, pattern="random", density=0.5)
    q, k, v = gu.upload(p)
    say("block-sparse scale", scale)
    o, l = attn.fwd_sparse(q, k, v, torch.from_numpy(bm).cuda(), block=64, scale=scale, causal=True, out_fp32=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_blockmask(p.q64, p.k64, p.v64, scale, bm, 64, True)
    gu.assert_close(gu.host(o), ro, gu.TOL_H16, "O")
    gu.assert_lse(gu.host(l), rl, gu.TOL_LSE_H16, "lse")


@pytest.mark.parametrize("scale", SCALES)
def test_gradient_any_scale(attn, scale):
    import torch
    B, H, N, d = 1, 2, 256, 64
    p = synth.make_qkv(B, H, N, d, "bf16", 97)
    g = synth.make_qkv(B, H, N, d, "bf16", 97, variant=1)
    q, k, v = synth.upload(p)
    dout = synth.to_torch(g.q, "bf16")
    say("gradient scale", scale)
    o, lse = attn.fwd(q, k, v, scale=scale, causal=True)
    dq, dk, dv = attn.bwd(q, k, v, o, dout, lse, scale=scale, causal=True)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd(p.q64, p.k64, p.v64, g.q64, scale, True)
    for name, x, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        x = gu.host(x)
        err = gu.max_abs(x, r)
        ref = float(np.abs(r).max())
        assert not np.isnan(x).any()
        assert err <= max(2e-2 * ref, 1e-4), f"{name}: {err:.3e} vs max|ref| {ref:.3e}"


@pytest.mark.parametrize("scale", SCALES)
def test_naive_baseline_any_scale(attn, scale):
    import torch
    p = synth.make_qkv(1, 2, 300, 64, "f32", 98)
    q, k, v = gu.upload(p)
    say("naive scale", scale)
    o, l = attn.naive_fwd(q, k, v, scale=scale, causal=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attn(p.q64, p.k64, p.v64, scale, True)
    gu.assert_close(gu.host(o), ro, fp32_gate(p, scale), "O")
    gu.assert_lse(gu.host(l), rl, fp32_gate(p, scale), "lse")
