"""GPU parity of the block-sparse forward (attn_fwd_sparse) against the fp64
oracle with block-sparse visibility, on seeded inputs and seeded block flags.

Every case prints what it runs (flushed) before touching the GPU.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

TILES = [(64, 64), (128, 64), (128, 128), (256, 64)]


@pytest.fixture(scope="module")
def attn():
    import torch
    assert torch.cuda.is_available()
    import tiled_online_softmax_fwd_amd as A
    A.lib()
    return A


def say(*a):
    print("[case]", *a, flush=True)


def run(A, p, bm, block, scale, causal=False, mask=None, out_fp32=True, **kw):
    import torch
    q, k, v = gu.upload(p)
    bmt = torch.from_numpy(np.ascontiguousarray(bm, np.uint8)).cuda()
    o, l = A.fwd_sparse(q, k, v, bmt, block=block, scale=scale, causal=causal,
                        key_padding_mask=gu.mask_to_torch(mask), out_fp32=out_fp32, **kw)
    torch.cuda.synchronize()
    return gu.host(o), gu.host(l)


def check(A, p, bm, block, scale, causal=False, mask=None, what="", **kw):
    o, l = run(A, p, bm, block, scale, causal, mask, **kw)
    ro, rl = oracle.attn_blockmask(p.q64, p.k64, p.v64, scale, bm, block, causal, mask)
    gu.assert_close(o, ro, gu.TOL_H16, what)
    gu.assert_lse(l, rl, gu.TOL_LSE_H16, what)
    # rows with no visible key: exact zeros
    empty = np.isneginf(rl)
    assert np.all(o[empty] == 0.0), f"{what}: empty rows not zero"
    return o, l, ro, rl


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("tile", TILES)
def test_random_blocks_every_tile(attn, dtype, d, tile):
    """Random 50% block flags (block 64), ragged N = 700 (11 blocks, last one
    60 rows), plain and causal, two heads per batch with different flags."""
    br, bc = tile
    p = synth.make_qkv(2, 2, 700, d, dtype, 60)
    bm = synth.block_mask(2, 2, 700, 64, 60, "random", 0.5)
    for causal in (False, True):
        say("sparse random", dtype, d, tile, "causal", causal)
        check(attn, p, bm, 64, d ** -0.5, causal, what=f"{dtype} d{d} {tile} causal={causal}", br=br, bc=bc)


@pytest.mark.parametrize("block", [32, 96, 128, 192])
def test_other_block_sizes(attn, block):
    """Blocks of 32, 96 (not a power of two), 128 and 192 rows against every
    default-tile geometry: a tile may span several blocks and a block several
    tiles."""
    for d in (64, 128):
        p = synth.make_qkv(1, 3, 777, d, "bf16", 61)
        bm = synth.block_mask(1, 3, 777, block, 61, "random", 0.4)
        for causal in (False, True):
            say("sparse block", block, "d", d, "causal", causal)
            check(attn, p, bm, block, d ** -0.5, causal, what=f"block {block} d{d} causal={causal}")


def test_all_blocks_on_equals_dense_bitwise(attn):
    """All flags on: the block-sparse kernel visits the same tiles in the same
    order with the same arithmetic as the dense kernel, so o and lse are
    bitwise equal to attn_fwd_ex with the same tiles."""
    import torch
    for d, tile in ((128, (256, 64)), (64, (128, 128)), (128, (128, 64))):
        p = synth.make_qkv(1, 4, 1000, d, "bf16", 62)
        q, k, v = gu.upload(p)
        bm = torch.ones((1, 4, 16, 16), dtype=torch.uint8, device="cuda")
        for causal in (False, True):
            say("sparse all-on vs dense", d, tile, causal)
            o1, l1 = attn.fwd_sparse(q, k, v, bm, block=64, causal=causal, br=tile[0], bc=tile[1])
            o2, l2 = attn.fwd(q, k, v, causal=causal, br=tile[0], bc=tile[1])
            torch.cuda.synchronize()
            assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_no_blocks_and_empty_row_blocks(attn):
    """All flags off: every row is empty (zeros, lse = -inf).  One row block
    switched off entirely: its rows are empty, the others match the oracle."""
    p = synth.make_qkv(1, 2, 300, 64, "bf16", 63)
    bm = np.zeros((1, 2, 5, 5), np.uint8)
    say("sparse all off")
    o, l = run(attn, p, bm, 64, 0.125)
    assert np.all(o == 0.0) and np.all(np.isneginf(l))
    bm = synth.block_mask(1, 2, 300, 64, 63, "random", 0.7)
    bm[0, 0, 2, :] = 0
    bm[0, 1, :, 0] = 1
    say("sparse one row block off")
    o, l, ro, rl = check(attn, p, bm, 64, 0.125, what="row block off")
    assert np.all(o[0, 0, 128:192] == 0.0) and np.all(np.isneginf(l[0, 0, 128:192]))


def test_with_padding_and_causal(attn):
    """Block flags, key padding and causality together (the padding of the
    B4 H16 N1024 d64 causal workload: one partly padded and one fully padded
    sequence)."""
    p = synth.make_qkv(4, 2, 1024, 64, "f16", 64)
    mask = synth.c2_mask(4, 1024, 64)
    bm = synth.block_mask(4, 2, 1024, 64, 64, "local_global", band=2, n_global=1)
    for causal in (False, True):
        say("sparse padding causal", causal)
        check(attn, p, bm, 64, 0.125, causal, mask, what=f"padding causal={causal}")


def test_more_than_64_tiles(attn):
    """N = 5000 with 64-key tiles: 79 key tiles, so the flag scan crosses a
    64-tile word; sliding window of 3 blocks plus one global block, and a
    random pattern."""
    p = synth.make_qkv(1, 2, 5000, 64, "bf16", 65)
    for pat in ("local_global", "random"):
        bm = synth.block_mask(1, 2, 5000, 64, 65, pat, 0.1, band=1, n_global=1)
        say("sparse N5000", pat)
        check(attn, p, bm, 64, 0.125, False, what=f"N5000 {pat}", br=128, bc=64)
        check(attn, p, bm, 64, 0.125, True, what=f"N5000 {pat} causal", br=256, bc=64)


def test_bf16_output_within_half_ulp_band(attn):
    """16-bit output flavour: the stored o differs from the fp32-output run by
    at most half an ulp of the storage type (the only extra step is the final
    rounding)."""
    import torch
    p = synth.make_qkv(1, 2, 513, 128, "bf16", 66)
    bm = synth.block_mask(1, 2, 513, 64, 66, "random", 0.5)
    say("sparse bf16 out")
    o16, l16 = run(attn, p, bm, 64, 128 ** -0.5, out_fp32=False)
    o32, l32 = run(attn, p, bm, 64, 128 ** -0.5, out_fp32=True)
    assert np.array_equal(l16, l32, equal_nan=True)
    assert np.all(np.abs(o16 - o32) <= gu.half_ulp(o32, "bf16"))


def test_large_sampled_rows(attn):
    """B1 H32 N8192 d128 causal with a sliding window of 4 blocks plus one
    global block (block 64), on the default tiles; sampled rows against the
    oracle evaluated on those rows only (the flags turn into a key-padding
    pattern per row)."""
    import torch
    B, H, N, d = 1, 32, 8192, 128
    p = synth.make_qkv(B, H, N, d, "bf16", 5)
    bm = synth.block_mask(B, H, N, 64, 5, "local_global", band=4, n_global=1)
    say("sparse C5 sampled")
    o, l = run(attn, p, bm, 64, d ** -0.5, True)
    rows = synth.sample_rows(B, H, N, 8, 7)
    for r in rows:
        bh, i = divmod(int(r), N)
        vis = np.repeat(bm[0, bh, i // 64], 64)[:N].astype(bool) & (np.arange(N) <= i)
        ro, rl = oracle.attn_rows(p.q64[:, bh:bh + 1], p.k64[:, bh:bh + 1], p.v64[:, bh:bh + 1], d ** -0.5,
                                  np.array([i]), False, (~vis).astype(np.uint8)[None, :])
        assert np.max(np.abs(o[0, bh, i] - ro[0])) <= gu.TOL_H16, f"row {r}"
        assert abs(l[0, bh, i] - rl[0]) <= gu.TOL_LSE_H16


def test_degenerate_sizes(attn):
    """One block covering everything (N <= block), N = 1, a block far larger
    than N, and empty sizes: flags on give the dense result bitwise, flags off
    give zeros and -inf, and B*H*N = 0 is a no-op."""
    import torch
    for N, block in ((1, 64), (50, 64), (64, 64), (65, 64), (200, 4096), (33, 32)):
        p = synth.make_qkv(1, 2, N, 64, "bf16", 67)
        q, k, v = gu.upload(p)
        nb = (N + block - 1) // block
        for causal in (False, True):
            say("sparse degenerate", N, block, causal)
            on = torch.ones((1, 2, nb, nb), dtype=torch.uint8, device="cuda")
            o1, l1 = attn.fwd_sparse(q, k, v, on, block=block, causal=causal, br=128, bc=64)
            o2, l2 = attn.fwd(q, k, v, causal=causal, br=128, bc=64)
            torch.cuda.synchronize()
            assert torch.equal(o1, o2) and torch.equal(l1, l2), (N, block, causal)
            off = torch.zeros_like(on)
            o3, l3 = attn.fwd_sparse(q, k, v, off, block=block, causal=causal)
            torch.cuda.synchronize()
            assert bool((o3 == 0).all()) and bool(torch.isneginf(l3).all())
    for shape in ((0, 2, 64, 64), (1, 0, 64, 64), (1, 2, 0, 64)):
        say("sparse empty", shape)
        z = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        nb = (shape[2] + 63) // 64
        bm = torch.ones((shape[0], shape[1], nb, nb), dtype=torch.uint8, device="cuda")
        o, l = attn.fwd_sparse(z, z, z, bm, block=64)
        torch.cuda.synchronize()
        assert o.shape == z.shape


def test_benchmark_window_at_full_size(attn):
    """The block-sparse benchmark's workload: B1 H32 N8192 d128 bf16 causal,
    blocks of 64, a window of +-4 blocks plus one global block, default tiles
    (the launch the benchmark times); every row of every head against the
    oracle."""
    import math
    p = synth.make_qkv(1, 32, 8192, 128, "bf16", 5)
    bm = synth.block_mask(1, 32, 8192, 64, 5, "local_global", 0.5, 4, 1)
    scale = float(np.float32(1 / math.sqrt(128)))
    say("sparse benchmark window B1 H32 N8192 d128 causal")
    check(attn, p, bm, 64, scale, True, what="sparse window +-4 + global, B1 H32 N8192")
