"""GPU parity of the backward (attn_bwd, through the C ABI) against the fp64
gradient of the plain definition (oracle.attn_bwd).

The 16-bit path rounds P and dS to the input type for the matrix cores (as the
forward rounds P), so the gate is relative to each gradient's own scale:
max |GPU - oracle| <= max(TOL_GRAD * max |oracle|, GRAD_FLOOR) per tensor; the
floor covers gradients that are exactly zero (one visible key gives dS = 0,
which the GPU reproduces only to rounding).
"""
import math

import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

TOL_GRAD = 2e-2
GRAD_FLOOR = 1e-4


@pytest.fixture(scope="module")
def attn():
    import torch
    assert torch.cuda.is_available()
    import tiled_online_softmax_fwd_amd as A
    A.lib()
    return A


def say(*a):
    print("[case]", *a, flush=True)


def run_bwd(A, B, H, N, d, dtype, causal, mask=None, seed=70):
    import torch
    p = synth.make_qkv(B, H, N, d, dtype, seed)
    g = synth.make_qkv(B, H, N, d, dtype, seed, variant=1)        # dO drawn from its own stream
    scale = float(np.float32(1 / math.sqrt(d)))
    q, k, v = synth.upload(p)
    dout = synth.to_torch(g.q, dtype)
    m = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask, np.uint8)).cuda()
    o, lse = A.fwd(q, k, v, scale=scale, causal=causal, key_padding_mask=m)
    dq, dk, dv = A.bwd(q, k, v, o, dout, lse, scale=scale, causal=causal, key_padding_mask=m)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd(p.q64, p.k64, p.v64, g.q64, scale, causal, mask)
    return (gu.host(dq), gu.host(dk), gu.host(dv)), (rq, rk, rv)


def check(got, ref, what):
    for name, x, r in zip(("dq", "dk", "dv"), got, ref):
        assert not np.isnan(x).any(), f"{what} {name}: NaN"
        err = gu.max_abs(x, r)
        scale = float(np.abs(r).max())
        say(what, name, f"max|d| {err:.3e} max|ref| {scale:.3e}")
        assert err <= max(TOL_GRAD * scale, GRAD_FLOOR), f"{what} {name}: {err:.3e} > {TOL_GRAD} * {scale:.3e}"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_shapes(attn, dtype, d, causal):
    for N in (1, 33, 200, 517):
        got, ref = run_bwd(attn, 2, 2, N, d, dtype, causal)
        check(got, ref, f"bwd {dtype} d{d} causal {causal} N{N}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_backward_padding(attn, dtype):
    """Key padding with random valid lengths and one fully padded sequence:
    its rows contribute nothing and its gradients are exactly zero."""
    B, N = 4, 300
    mask = synth.c2_mask(B, N)
    got, ref = run_bwd(attn, B, 2, N, 128, dtype, True, mask)
    check(got, ref, f"bwd padding {dtype}")
    for x in got:
        assert np.all(x[1] == 0)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_scattered_padding_unaligned_rows(attn, d, causal):
    """Key padding with odd N (mask rows of odd batches are not 4-byte
    aligned), scattered padded keys (key tiles with and without a padded key),
    a fully padded sequence and one whose first 200 keys are padded (wholly
    padded key tiles, and waves whose keys are all padded)."""
    B, N = 4, 301
    rng = np.random.default_rng([71, N, 99])
    mask = (rng.random((B, N)) < 0.01).astype(np.uint8)
    mask[1, :] = 1
    mask[2, :200] = 1
    got, ref = run_bwd(attn, B, 2, N, d, "bf16", causal, mask, seed=71)
    check(got, ref, f"bwd scattered padding d{d} causal {causal}")
    for x in got:
        assert np.all(x[1] == 0)


def test_backward_sum_rule_and_determinism(attn):
    """sum_j dV_j = sum_i dO_i (rows of P sum to one) holds on the GPU, and two
    calls give bitwise-identical gradients."""
    import torch
    p = synth.make_qkv(1, 2, 700, 64, "bf16", 71)
    g = synth.make_qkv(1, 2, 700, 64, "bf16", 71, variant=1)
    q, k, v = synth.upload(p)
    dout = synth.to_torch(g.q, "bf16")
    o, lse = attn.fwd(q, k, v)
    a = attn.bwd(q, k, v, o, dout, lse)
    b = attn.bwd(q, k, v, o, dout, lse)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    dv = gu.host(a[2])
    np.testing.assert_allclose(dv.sum(axis=2), g.q64.sum(axis=2), rtol=2e-2, atol=2e-2 * np.abs(g.q64).sum(axis=2).max() / 700)


def test_backward_long_sequence(attn):
    """B1 H8 N4096 d128 bf16 causal: every gradient against the oracle."""
    got, ref = run_bwd(attn, 1, 8, 4096, 128, "bf16", True, seed=72)
    check(got, ref, "bwd N4096")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [80, 768, 1091])
def test_backward_pipeline_ranges(attn, causal, N):
    """d = 128 sizes where the gradient kernels' pipelined blocks run several
    loop iterations and hand over to the compiler-scheduled loops at their
    range ends: N a multiple of the 256-key workgroup (every key workgroup
    pipelined), a ragged N (the last key workgroup and the last query tiles
    outside the blocks; at N = 1091 the last key workgroup's block has a
    single pair of steps) and N = 80 (the dQ block over two 32-key tiles,
    without loop iterations), with an odd number of heads."""
    got, ref = run_bwd(attn, 1, 3, N, 128, "bf16", causal, seed=73)
    check(got, ref, f"bwd pipeline ranges N{N} causal {causal}")


def test_backward_headline_shape_two_heads(attn):
    """B1 H32 N8192 d128 bf16 causal, the shape and launch the backward
    benchmark times (both gradient kernels' pipelined loops over their longest
    ranges): the first and the last head's gradients against the oracle."""
    import torch
    B, H, N, d = 1, 32, 8192, 128
    p = synth.make_qkv(B, H, N, d, "bf16", 74)
    g = synth.make_qkv(B, H, N, d, "bf16", 74, variant=1)
    scale = float(np.float32(1 / math.sqrt(d)))
    q, k, v = synth.upload(p)
    dout = synth.to_torch(g.q, "bf16")
    o, lse = attn.fwd(q, k, v, scale=scale, causal=True)
    dq, dk, dv = attn.bwd(q, k, v, o, dout, lse, scale=scale, causal=True)
    torch.cuda.synchronize()
    hs = [0, H - 1]
    ref = oracle.attn_bwd(p.q64[:, hs], p.k64[:, hs], p.v64[:, hs], g.q64[:, hs], scale, True)
    got = tuple(gu.host(x)[:, hs] for x in (dq, dk, dv))
    check(got, ref, "bwd B1 H32 N8192 heads 0, 31")
