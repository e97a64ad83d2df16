"""GPU: the software-pipelined steady state of the 16-bit d = 128 kernel (256 x
64 tiles) against the compiler-scheduled tile loop of the same kernel
(attn_opts.generic_loop = 1) and against the fp64 oracle.

Both loops do the same per-row operations in the same order, so O and lse must
be bitwise equal; the shapes below put the end of the pipelined range at every
kind of boundary (no tile after it, a full tile, a ragged tile, the causal
diagonal) and run the pipeline with zero, one and many iterations.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def attn():
    import torch
    assert torch.cuda.is_available()
    import tiled_online_softmax_fwd_amd as A
    A.lib()
    return A


def say(*a):
    print("[case]", *a, flush=True)


def both(A, p, scale, causal, out_fp32, ref_slack=0):
    import torch
    q, k, v = gu.upload(p)
    outs = []
    for generic in (False, True):
        o, l = A.fwd(q, k, v, scale=scale, causal=causal, out_fp32=out_fp32, generic_loop=generic,
                     ref_slack=ref_slack)
        outs.append((o, l))
    torch.cuda.synchronize()
    return outs


# N: 128 (two full tiles, nothing after), 150 / 130 (ragged tile right after the
# range), 192 (full tile after), 200 (full then ragged), 512, 1000, 1024, 2112
SHAPES = [(1, 2, 128), (1, 2, 130), (1, 2, 150), (2, 2, 192), (1, 3, 200), (2, 2, 512),
          (1, 4, 1000), (2, 3, 1024), (1, 2, 2112)]


@pytest.mark.parametrize("B,H,N", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_pipelined_equals_tile_loop_bitwise(attn, B, H, N, causal, dtype):
    import torch
    p = synth.make_qkv(B, H, N, 128, dtype, 70, variant=N)
    scale = float(np.float32(128 ** -0.5))
    for out_fp32 in (True, False):
        say("pipeline vs tile loop", dtype, B, H, N, "causal", causal, "out_fp32", out_fp32)
        (o1, l1), (o2, l2) = both(attn, p, scale, causal, out_fp32)
        assert torch.equal(o1, o2), f"O differs: max {float((o1.double() - o2.double()).abs().max()):.3e}"
        assert torch.equal(l1, l2), "lse differs"


@pytest.mark.parametrize("B,H,N", [(1, 2, 150), (2, 2, 512), (1, 4, 1000)])
@pytest.mark.parametrize("causal", [False, True])
def test_pipelined_against_oracle(attn, B, H, N, causal):
    import torch
    p = synth.make_qkv(B, H, N, 128, "bf16", 71, variant=N)
    scale = float(np.float32(128 ** -0.5))
    say("pipeline vs oracle bf16", B, H, N, "causal", causal)
    q, k, v = gu.upload(p)
    o, l = attn.fwd(q, k, v, scale=scale, causal=causal, out_fp32=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attn(p.q64, p.k64, p.v64, scale, causal)
    gu.assert_close(gu.host(o), ro, gu.TOL_H16, "pipelined O")
    gu.assert_lse(gu.host(l), rl, gu.TOL_LSE_H16, "pipelined lse")


def test_pipelined_headline_shape_bitwise(attn):
    """B1 H32 N8192 d128 bf16 causal, bf16 output: the benchmarked call."""
    import torch
    p = synth.make_qkv(1, 32, 8192, 128, "bf16", 5)
    scale = float(np.float32(128 ** -0.5))
    say("pipeline vs tile loop B1 H32 N8192 causal")
    (o1, l1), (o2, l2) = both(attn, p, scale, True, False)
    assert torch.equal(o1, o2)
    assert torch.equal(l1, l2)


def test_pipelined_peaked_rows_bitwise(attn):
    """Q and K x4 (score std about 16): the reference moves on few tiles, so
    most iterations take the no-rescale branch of the pipeline."""
    import torch
    p = synth.make_qkv(2, 4, 1024, 128, "bf16", 72, qk_factor=4.0)
    scale = float(np.float32(128 ** -0.5))
    for causal in (False, True):
        say("pipeline vs tile loop peaked rows causal", causal)
        (o1, l1), (o2, l2) = both(attn, p, scale, causal, True)
        assert torch.equal(o1, o2)
        assert torch.equal(l1, l2)


@pytest.mark.parametrize("slack", [1, 8])
@pytest.mark.parametrize("B,H,N,causal,dtype", [(1, 2, 200, True, "bf16"), (2, 2, 512, False, "f16"),
                                                (1, 4, 1000, True, "f16"), (1, 32, 4096, True, "bf16")])
def test_pipelined_lagging_reference_bitwise(attn, slack, B, H, N, causal, dtype):
    """With ref_slack the pipeline compares c (mt - m) against the slack
    instead of 0; both loops then move the reference on the same tiles."""
    import torch
    p = synth.make_qkv(B, H, N, 128, dtype, 76, variant=N + slack)
    scale = float(np.float32(128 ** -0.5))
    say("pipeline vs tile loop, ref_slack", slack, dtype, B, H, N, "causal", causal)
    (o1, l1), (o2, l2) = both(attn, p, scale, causal, False, ref_slack=slack)
    assert torch.equal(o1, o2), f"O differs: max {float((o1.double() - o2.double()).abs().max()):.3e}"
    assert torch.equal(l1, l2), "lse differs"
    if N <= 1000:
        ro, rl = oracle.attn(p.q64, p.k64, p.v64, scale, causal)
        gu.assert_close(gu.host(o1), ro, gu.TOL_H16, f"ref_slack {slack} O")
        gu.assert_lse(gu.host(l1), rl, gu.TOL_LSE_H16, f"ref_slack {slack} lse")


# Shapes whose work splits evenly over 256 compute units run on the persistent
# grid (one workgroup per compute unit walking a list of query tiles, or of
# causal pairs of query tiles); generic_loop = 1 runs one workgroup per query
# tile.  (B, H, N, causal): one pair per workgroup; two and four pairs per
# workgroup; query tiles without causal masking; a head count that is not a
# multiple of 8 (no XCD affinity).
PERSISTENT = [(1, 16, 8192, True), (1, 32, 4096, True), (2, 32, 8192, True), (2, 16, 4096, False),
              (1, 4, 32768, True)]


@pytest.mark.parametrize("B,H,N,causal", PERSISTENT)
def test_persistent_grid_bitwise(attn, B, H, N, causal):
    import torch
    p = synth.make_qkv(B, H, N, 128, "bf16", 73, variant=N)
    scale = float(np.float32(128 ** -0.5))
    say("persistent grid vs one workgroup per tile", B, H, N, "causal", causal)
    (o1, l1), (o2, l2) = both(attn, p, scale, causal, False)
    assert torch.equal(o1, o2), f"O differs: max {float((o1.double() - o2.double()).abs().max()):.3e}"
    assert torch.equal(l1, l2), "lse differs"


def test_persistent_grid_sampled_rows_against_oracle(attn):
    """B2 H32 N8192 causal (four causal pairs per workgroup): sampled rows
    against the fp64 oracle."""
    import torch
    p = synth.make_qkv(2, 32, 8192, 128, "bf16", 74)
    scale = float(np.float32(128 ** -0.5))
    say("persistent grid B2 H32 N8192 causal vs oracle rows")
    q, k, v = gu.upload(p)
    o, l = attn.fwd(q, k, v, scale=scale, causal=True, out_fp32=True)
    torch.cuda.synchronize()
    rows = gu.sample_rows(2, 32, 8192, per_head=40, seed=75)
    ro, rl = oracle.attn_rows(p.q64, p.k64, p.v64, scale, rows, True)
    gu.assert_close(gu.host(o).reshape(-1, 128)[rows], ro, gu.TOL_H16, "persistent O rows")
    gu.assert_lse(gu.host(l).reshape(-1)[rows], rl, gu.TOL_LSE_H16, "persistent lse rows")
