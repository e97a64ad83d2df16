"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on
the same seeded inputs, element by element.

Every case prints what it runs (flushed) before touching the GPU.
"""
import math

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


def run(A, p: synth.QKV, scale, causal=False, mask=None, **kw):
    import torch
    q, k, v = gu.upload(p)
    out, lse = A.fwd(q, k, v, scale=scale, causal=causal, key_padding_mask=gu.mask_to_torch(mask), **kw)
    torch.cuda.synchronize()
    return gu.host(out), gu.host(lse)


def gate(dtype):
    return (gu.TOL_F32, gu.TOL_LSE_F32) if dtype == "f32" else (gu.TOL_H16, gu.TOL_LSE_H16)


def check_full(A, p, scale, causal=False, mask=None, what="", **kw):
    out_f32 = p.dtype != "f32"
    o, l = run(A, p, scale, causal, mask, out_fp32=out_f32, **kw)
    ro, rl = oracle.attn(p.q64, p.k64, p.v64, scale, causal, mask)
    tol, tl = gate(p.dtype)
    e = gu.assert_close(o, ro, tol, what)
    gu.assert_lse(l, rl, tl, what)
    return e, o, l, ro, rl


# ------------------------------------------------------------------ C1
def test_c1_single_head_fp32_no_mask_and_causal(attn):
    """B1 H1 N128 d64 fp32, scale 1/8; plain and causal (row 0 of the causal run
    has one visible key and must return v_0 bit for bit)."""
    p = synth.make_qkv(1, 1, 128, 64, "f32", 1)
    for causal in (False, True):
        say("C1 fp32 N128 d64 causal", causal)
        e, o, l, ro, rl = check_full(attn, p, 0.125, causal, what=f"C1 causal={causal}")
        if causal:
            assert np.array_equal(o[0, 0, 0], p.v64[0, 0, 0])


def test_c1_score_shift_of_1000(attn):
    """Every score shifted by +1000 (q[:, d-1] = 8000, k[:, d-1] = 1 with scale
    1/8): nothing overflows and the result matches the oracle.  fp32 scores near
    1000 carry an ulp of 6.1e-5, so the gate is 1e-5 + 4 ulp(1000) * max|v|
    (|d o| <= 2 max|v| max|d s| since d o / d s_j = p_j (v_j - o))."""
    base = synth.make_qkv(1, 1, 128, 64, "f32", 1, variant=1)
    q = base.q64.copy(); k = base.k64.copy()
    q[..., -1] = 8000.0
    k[..., -1] = 1.0
    p = synth.qkv_from_f64(q, k, base.v64, "f32")
    tol = 1e-5 + 4 * 2.0 ** -14 * np.abs(p.v64).max()
    for causal in (False, True):
        say("C1b shift 1000 causal", causal)
        o, l = run(attn, p, 0.125, causal)
        ro, rl = oracle.attn(p.q64, p.k64, p.v64, 0.125, causal)
        assert np.isfinite(o).all() and np.isfinite(l).all()
        gu.assert_close(o, ro, tol, "C1b")
        gu.assert_lse(l, rl, 1e-3, "C1b")


def embed_scores(scores, values, d=64):
    """fp32 tensors whose scaled scores (scale 1/8) are exactly `scores` for
    query row i = len-1 ... and whose value rows are `values` padded with zeros."""
    n = len(scores)
    q = np.zeros((1, 1, n, d)); k = np.zeros((1, 1, n, d)); v = np.zeros((1, 1, n, d))
    q[0, 0, :, 0] = 1.0
    k[0, 0, :, 0] = 8.0 * np.asarray(scores, np.float64)
    vals = np.asarray(values, np.float64)
    v[0, 0, :, :vals.shape[1]] = vals
    return synth.qkv_from_f64(q, k, v, "f32")


def test_tutorial_worked_example_on_the_gpu(attn):
    """The tutorial's self-check, embedded exactly in fp32: scores
    [1000, 1001, 999, 1004, 997] for every query row, causal, so row i sees the
    prefix of length i+1.  Rows 0 and 1 have closed forms."""
    s = [1000.0, 1001.0, 999.0, 1004.0, 997.0]
    vals = [[2.0, -1.0], [0.0, 3.0], [4.0, 1.0], [-2.0, 2.0], [1.0, -4.0]]
    p = embed_scores(s, vals)
    for order in (0, 1):
        for bc in (32, 64, 128):
            say("tutorial example order", order, "bc", bc)
            o, l = run(attn, p, 0.125, causal=True, bc=bc, kv_order=order)
            assert o[0, 0, 0, 0] == 2.0 and o[0, 0, 0, 1] == -1.0
            e = math.e
            assert abs(o[0, 0, 1, 0] - 2 / (1 + e)) <= 1e-5 and abs(o[0, 0, 1, 1] - (3 * e - 1) / (1 + e)) <= 1e-5
            ro, rl = oracle.attn(p.q64, p.k64, p.v64, 0.125, True)
            gu.assert_close(o, ro, 1e-5, "tutorial example")
            gu.assert_lse(l, rl, 1e-4, "tutorial example")


def test_averaging_counterexample_on_the_gpu(attn):
    """Scores [0, 0, 100, 100] with values [0, 0, 1, 1]: the last row's output is
    1/(1+e^-100) (> 0.999), not the 0.5 that averaging block softmaxes gives."""
    p = embed_scores([0.0, 0.0, 100.0, 100.0], [[0.0], [0.0], [1.0], [1.0]])
    for bc in (32, 64):
        say("averaging example bc", bc)
        o, l = run(attn, p, 0.125, causal=False, bc=bc)
        assert np.all(np.abs(o[0, 0, :, 0] - 1.0) <= 1e-5)
        assert np.all(np.abs(l[0, 0] - (100 + math.log(2))) <= 1e-4)


# ------------------------------------------------------------------ C2
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_c2_causal_with_key_padding(attn, dtype):
    """B4 H16 N1024 d64, causal, key padding: batch 0 has a random valid length,
    batch 1 is fully padded (every row outputs exact zeros and lse = -inf),
    batches 2 and 3 are unpadded."""
    import torch
    p = synth.make_qkv(4, 16, 1024, 64, dtype, 2)
    mask = synth.c2_mask(4, 1024)
    say("C2", dtype, "fp32-out flavour")
    e, o, l, ro, rl = check_full(attn, p, 0.125, True, mask, what=f"C2 {dtype}")
    assert np.all(o[1] == 0) and np.all(np.signbit(o[1]) == False)
    assert np.all(np.isneginf(l[1]))
    say("C2", dtype, "16-bit output flavour")
    o16, l16 = run(attn, p, 0.125, True, mask)
    tol = gu.TOL_H16 + gu.half_ulp(ro, dtype)
    assert not np.isnan(o16).any()
    assert np.all(np.abs(o16 - ro) <= tol), f"max|d| {np.abs(o16 - ro).max():.3e}"
    assert np.all(o16[1] == 0) and np.all(np.isneginf(l16[1]))


def test_key_zero_padded_under_causal_masks_exactly_row_zero(attn):
    """Padding only key 0 under causal leaves query row 0 with nothing visible."""
    p = synth.make_qkv(2, 2, 70, 64, "bf16", 5)
    mask = np.zeros((2, 70), np.uint8); mask[:, 0] = 1
    for order in (0, 1):
        say("key0 padded causal, order", order)
        e, o, l, ro, rl = check_full(attn, p, 0.125, True, mask, what="key0", kv_order=order)
        assert np.all(o[:, :, 0] == 0) and np.all(np.isneginf(l[:, :, 0]))
        assert np.isfinite(l[:, :, 1:]).all()


@pytest.mark.parametrize("slack", [0, 8])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_reference_moves_and_stays(attn, dtype, causal, slack):
    """Rows whose scores rise slowly along the keys (the merge reference moves
    only every few tiles), steeply (it moves at every tile) or fall (it moves
    once), plus a random head: the result must equal the plain definition.
    Scores are exact: q[:, 0] = 1, k[j, 0] = a * j, scale 1.  fp32 gate as for
    the +1000 shift: 1e-5 + 2 max|v| * 4 ulp(max|s|)."""
    N, d, H = 1000, 64, 4
    rng = np.random.default_rng([7, N, 1])
    q = np.zeros((1, H, N, d)); k = np.zeros((1, H, N, d))
    v = rng.standard_normal((1, H, N, d))
    j = np.arange(N)
    q[0, :3, :, 0] = 1.0
    for h, a in enumerate((0.01, 0.1, -0.01)):
        k[0, h, :, 0] = a * j
    q[0, 3] = rng.standard_normal((N, d)) * 0.2
    k[0, 3] = rng.standard_normal((N, d))
    p = synth.qkv_from_f64(q, k, v, dtype)
    smax = float(np.abs(p.k64[0, :3, :, 0]).max())
    tol = gu.TOL_H16 if dtype == "bf16" else 1e-5 + 2 * np.abs(p.v64).max() * 4 * 2.0 ** (np.floor(np.log2(smax)) - 23)
    for bc in (32, 64):
        say("reference paths", dtype, "causal", causal, "bc", bc, "slack", slack)
        o, l = run(attn, p, 1.0, causal, out_fp32=dtype != "f32", bc=bc, ref_slack=slack)
        ro, rl = oracle.attn(p.q64, p.k64, p.v64, 1.0, causal)
        gu.assert_close(o, ro, tol, f"reference paths {dtype} bc{bc}")
        gu.assert_lse(l, rl, 1e-3 if dtype == "f32" else gu.TOL_LSE_H16, "reference paths")


# ------------------------------------------------------------------ tiles
TILES = [(br, bc) for br in (16, 32, 64, 128) for bc in (16, 32, 64, 128)]
WIDE_TILES = [(256, 32), (256, 64), (256, 128)]      # eight-wave tiles, 16-bit inputs only


@pytest.mark.parametrize("br,bc", TILES + WIDE_TILES)
def test_tile_shapes_and_orders_bf16(attn, br, bc):
    """Every tile shape and both fold orders, on a ragged length (1000, not a
    multiple of any tile) with peaked rows (Q, K scaled by 4), d = 128."""
    p = synth.make_qkv(1, 2, 1000, 128, "bf16", 3, qk_factor=4.0)
    scale = float(np.float32(1 / math.sqrt(128)))
    ro, rl = oracle.attn(p.q64, p.k64, p.v64, scale)
    for order in (0, 1):
        say("tiles bf16 d128 N1000", br, bc, "order", order)
        o, l = run(attn, p, scale, br=br, bc=bc, kv_order=order, out_fp32=True)
        gu.assert_close(o, ro, gu.TOL_H16, f"tile {br}x{bc} order {order}")
        gu.assert_lse(l, rl, gu.TOL_LSE_H16, "tile")


@pytest.mark.parametrize("br,bc", TILES)
@pytest.mark.parametrize("d", [64, 128])
def test_tile_shapes_fp32_causal(attn, br, bc, d):
    """fp32 arithmetic at every tile shape, causal, ragged length."""
    p = synth.make_qkv(1, 2, 333, d, "f32", 4)
    scale = float(np.float32(1 / math.sqrt(d)))
    ro, rl = oracle.attn(p.q64, p.k64, p.v64, scale, True)
    for order in (0, 1):
        say("tiles fp32", d, br, bc, "order", order)
        o, l = run(attn, p, scale, True, br=br, bc=bc, kv_order=order)
        gu.assert_close(o, ro, gu.TOL_F32, f"fp32 tile {br}x{bc}")
        gu.assert_lse(l, rl, gu.TOL_LSE_F32, "fp32 tile")


@pytest.mark.parametrize("br,bc", [(16, 16), (16, 64), (64, 16), (128, 16), (32, 32), (256, 64)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_tiles_16bit_causal_with_padding(attn, br, bc, dtype, d):
    """Causal + key padding (one sequence with a random valid length, one fully
    padded) through the 16-row/16-key kernel and the 32-row kernel, ragged N."""
    N = 300
    p = synth.make_qkv(4, 2, N, d, dtype, 2)
    mask = synth.c2_mask(4, N)
    scale = float(np.float32(1 / math.sqrt(d)))
    for order in (0, 1):
        say("tiles causal+padding", dtype, d, br, bc, "order", order)
        e, o, l, ro, rl = check_full(attn, p, scale, True, mask, f"{dtype} d{d} {br}x{bc} o{order}",
                                     br=br, bc=bc, kv_order=order)
        assert np.all(o[1] == 0) and np.all(np.isneginf(l[1]))


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_scattered_padding_with_unaligned_mask_rows(attn, dtype, d, causal):
    """Key padding with odd N (mask rows of odd batches are not 4-byte
    aligned, so flags are read byte by byte there), scattered padded keys (key
    tiles with and without a padded key), a fully padded sequence (its key
    tiles are skipped) and a sequence whose first 200 keys are padded (its
    first key tiles are wholly padded), at the default tiles in both orders."""
    N = 301
    p = synth.make_qkv(4, 2, N, d, dtype, 7)
    rng = np.random.default_rng([7, N, 99])
    mask = (rng.random((4, N)) < 0.01).astype(np.uint8)
    mask[1, :] = 1
    mask[2, :200] = 1
    scale = float(np.float32(1 / math.sqrt(d)))
    for order in (0, 1):
        say("scattered padding", dtype, d, "causal", causal, "order", order)
        e, o, l, ro, rl = check_full(attn, p, scale, causal, mask, f"{dtype} d{d} causal={causal} o{order}",
                                     kv_order=order)
        assert np.all(o[1] == 0) and np.all(np.isneginf(l[1]))


@pytest.mark.parametrize("dtype,d,br,bc", [("f32", 128, 128, 128), ("f32", 64, 32, 128), ("f32", 128, 16, 64),
                                            ("f32", 64, 64, 16), ("bf16", 128, 16, 32), ("f16", 64, 128, 16)])
def test_scattered_padding_fp32_and_16_row_tiles(attn, dtype, d, br, bc):
    """The padding cases above through the fp32 single-buffer kernel (128-key
    tiles at d = 128), the fp32 double-buffered kernel at 128-key tiles and the
    16-row/16-key kernel: tiles without a padded key take the unmasked path,
    wholly padded tiles are skipped, the rest read the flags as words (or
    bytes, where the mask row is not 4-byte aligned)."""
    N = 301
    p = synth.make_qkv(4, 2, N, d, dtype, 8)
    rng = np.random.default_rng([8, N, 99])
    mask = (rng.random((4, N)) < 0.01).astype(np.uint8)
    mask[1, :] = 1
    mask[2, :200] = 1
    scale = float(np.float32(1 / math.sqrt(d)))
    for causal in (False, True):
        for order in (0, 1):
            say("scattered padding tiles", dtype, d, br, bc, "causal", causal, "order", order)
            e, o, l, ro, rl = check_full(attn, p, scale, causal, mask,
                                         f"{dtype} d{d} {br}x{bc} causal={causal} o{order}",
                                         br=br, bc=bc, kv_order=order)
            assert np.all(o[1] == 0) and np.all(np.isneginf(l[1]))


# ------------------------------------------------------------------ edges
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 2, 31, 33, 129])
def test_small_and_ragged_lengths(attn, dtype, d, N):
    p = synth.make_qkv(2, 3, N, d, dtype, 6)
    scale = float(np.float32(1 / math.sqrt(d)))
    for causal in (False, True):
        say("ragged", dtype, d, N, causal)
        check_full(attn, p, scale, causal, what=f"ragged {dtype} d{d} N{N}")


def test_empty_sizes_are_noops(attn):
    import torch
    for shape in [(0, 2, 8, 64), (1, 0, 8, 64), (1, 2, 0, 64)]:
        say("empty", shape)
        q = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
        out = torch.full(shape, 7.0, dtype=torch.bfloat16, device="cuda")
        attn.fwd(q, q, q, out=out, scale=0.125)
        torch.cuda.synchronize()


def test_equal_scores_give_mean_of_v_and_constant_v(attn):
    """Q = 0: all scores equal, causal row i is the mean of v_0..v_i.
    V = 1: every visible row outputs 1 (a convex combination)."""
    base = synth.make_qkv(1, 2, 200, 64, "bf16", 7)
    p = synth.qkv_from_f64(np.zeros_like(base.q64), base.k64, base.v64, "bf16")
    say("Q=0 mean of V")
    o, l = run(attn, p, 0.125, True, out_fp32=True)
    want = np.cumsum(p.v64, axis=2) / np.arange(1, 201)[None, None, :, None]
    gu.assert_close(o, want, gu.TOL_H16, "mean of V")
    np.testing.assert_allclose(l[0, 0], np.log(np.arange(1, 201)), atol=1e-4)
    p1 = synth.qkv_from_f64(base.q64, base.k64, np.ones_like(base.v64), "bf16")
    say("V=1")
    o1, _ = run(attn, p1, 0.125, True, out_fp32=True)
    assert np.abs(o1 - 1.0).max() <= 1e-5


def test_sentinel_trap_scores_below_minus_50000(attn):
    """Valid scores near -60,000 with some keys padded: the result is the
    softmax over the valid keys only (a -50,000 sentinel would hand the padded
    keys all the weight)."""
    N, d = 96, 64
    rng = np.random.default_rng([31, 0])
    q = np.zeros((1, 1, N, d)); k = np.zeros((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    q[..., 0] = 1.0
    k[0, 0, :, 0] = 8.0 * (-60000.0 + rng.standard_normal(N) * 2)
    mask = (rng.random((1, N)) < 0.3).astype(np.uint8)
    k[0, 0, mask[0] == 1, 0] = 8.0 * (-50000.0 + 5.0)
    p = synth.qkv_from_f64(q, k, v, "f32")
    say("sentinel trap")
    o, l = run(attn, p, 0.125, False, mask)
    ro, rl = oracle.attn(p.q64, p.k64, p.v64, 0.125, False, mask)
    gu.assert_close(o, ro, 1e-5, "sentinel")
    gu.assert_lse(l, rl, 1e-2, "sentinel")


def test_deterministic_bitwise(attn):
    import torch
    p = synth.make_qkv(2, 4, 777, 128, "bf16", 8)
    q, k, v = gu.upload(p)
    say("determinism")
    a = attn.fwd(q, k, v, scale=0.088, causal=True)
    b = attn.fwd(q, k, v, scale=0.088, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


# ------------------------------------------------------------------ full size, sampled rows
def sampled_check(A, B, H, N, d, dtype, causal, cfg, qk_factor=1.0, per_head=12, **kw):
    import torch
    p = synth.make_qkv(B, H, N, d, dtype, cfg, qk_factor=qk_factor)
    scale = float(np.float32(1 / math.sqrt(d)))
    say("full size", B, H, N, d, dtype, "causal", causal, kw)
    o, l = run(A, p, scale, causal, out_fp32=dtype != "f32", **kw)
    rows = gu.sample_rows(B, H, N, per_head)
    ro, rl = oracle.attn_rows(p.q64, p.k64, p.v64, scale, rows, causal)
    tol, tl = gate(dtype)
    e = gu.assert_close(o.reshape(-1, d)[rows], ro, tol, f"sampled {B}x{H}x{N}x{d}")
    gu.assert_lse(l.reshape(-1)[rows], rl, tl, "sampled")
    assert np.isfinite(o).all() and np.isfinite(l).all()
    return e


def test_c5_headline_shape_sampled_rows(attn):
    """B1 H32 N8192 d128 bf16 causal, default tiles (the launch the benchmark
    times); every head's first, last and spread rows against the oracle."""
    sampled_check(attn, 1, 32, 8192, 128, "bf16", True, 5)


def test_c5_with_lagging_reference(attn):
    """The headline shape with the merge reference allowed to lag by 2^8."""
    sampled_check(attn, 1, 32, 8192, 128, "bf16", True, 5, per_head=6, ref_slack=8)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_c2_with_lagging_reference(attn, dtype):
    """Causal + key padding with the lagging reference, several tiles."""
    p = synth.make_qkv(4, 4, 1024, 64, dtype, 2)
    mask = synth.c2_mask(4, 1024)
    for br, bc in ((256, 64) if dtype != "f32" else (128, 64), (64, 32), (16, 16)):
        say("C2 lagging reference", dtype, br, bc)
        e, o, l, ro, rl = check_full(attn, p, 0.125, True, mask, f"C2 slack {dtype} {br}x{bc}",
                                     br=br, bc=bc, ref_slack=8)
        assert np.all(o[1] == 0) and np.all(np.isneginf(l[1]))


def test_c3_shape_sampled_rows(attn):
    """B2 H16 N4096 d128 bf16, Q and K scaled by 4 (peaked rows), non-causal."""
    for order in (0, 1):
        sampled_check(attn, 2, 16, 4096, 128, "bf16", False, 3, qk_factor=4.0, kv_order=order)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_c4_sequence_sweep(attn, dtype):
    """B1 H8 d64, N from 512 to 16384: full oracle up to 2048, sampled rows above."""
    for N in (512, 1024, 2048, 4096, 8192, 16384):
        if N <= 2048:
            p = synth.make_qkv(1, 8, N, 64, dtype, 4)
            say("C4 full", dtype, N)
            check_full(attn, p, 0.125, what=f"C4 {dtype} N{N}")
        else:
            sampled_check(attn, 1, 8, N, 64, dtype, False, 4, per_head=6)


def test_c3_tile_and_order_sweep_at_its_shape(attn):
    """The C3 sweep itself: B2 H16 N4096 d128 bf16, Q and K scaled by 4 (peaked
    rows), non-causal, every Br x Bc in {16, 32, 64, 128}^2 in both fold orders
    (32 runs), sampled rows of each run against the fp64 oracle at the 16-bit
    gate on the fp32-output flavour."""
    import torch
    B, H, N, d = 2, 16, 4096, 128
    p = synth.make_qkv(B, H, N, d, "bf16", 3, qk_factor=4.0)
    scale = float(np.float32(1 / math.sqrt(d)))
    rows = gu.sample_rows(B, H, N, 8)
    ro, rl = oracle.attn_rows(p.q64, p.k64, p.v64, scale, rows, False)
    q, k, v = gu.upload(p)
    worst = 0.0
    for br, bc in TILES:
        for order in (0, 1):
            say("C3 sweep", br, bc, "order", order)
            o, l = attn.fwd(q, k, v, scale=scale, out_fp32=True, br=br, bc=bc, kv_order=order)
            torch.cuda.synchronize()
            oh = gu.host(o).reshape(-1, d)[rows]
            lh = gu.host(l).reshape(-1)[rows]
            worst = max(worst, gu.assert_close(oh, ro, gu.TOL_H16, f"C3 {br}x{bc} order {order}"))
            gu.assert_lse(lh, rl, gu.TOL_LSE_H16, f"C3 {br}x{bc} order {order}")
    say(f"C3 sweep: worst max|d| {worst:.3e}")
