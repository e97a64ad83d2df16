"""GPU parity of the key/value-cache decode path (attn_decode_fwd) against the
fp64 oracle's query-block definition (oracle.attn_kv), through the C ABI."""
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


# fp32(0.1): the library receives the scale as a float and the oracle widens
# the same value
S01 = float(np.float32(0.1))


def say(*a):
    print("[case]", *a, flush=True)


def make(B, H, Nq, Nk, d, dtype, seed):
    """Seeded Q [B,H,Nq,d] and K, V [B,H,Nk,d] rounded to dtype (Q drawn after K, V)."""
    kv = synth.make_qkv(B, H, Nk, d, dtype, seed)
    qq = synth.make_qkv(B, H, Nq, d, dtype, seed, variant=1)
    return qq.q, qq.q64, kv.k, kv.k64, kv.v, kv.v64


def run(A, q, k, v, dtype, scale, causal, mask=None, splits=0, out_fp32=True):
    import torch
    tq, tk, tv = (synth.to_torch(x, dtype) for x in (q, k, v))
    m = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask, np.uint8)).cuda()
    o, l = A.decode_fwd(tq, tk, tv, scale=scale, causal=causal, key_padding_mask=m, out_fp32=out_fp32,
                        num_splits=splits)
    torch.cuda.synchronize()
    return gu.host(o), gu.host(l)


SHAPES = [(2, 3, 1, 1000), (1, 4, 5, 333), (2, 2, 16, 64), (1, 2, 17, 2000), (1, 1, 64, 64), (1, 2, 1, 1), (1, 1, 3, 31)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_decode_shapes(attn, dtype, d, causal):
    for si, (B, H, Nq, Nk) in enumerate(SHAPES):
        q, q64, k, k64, v, v64 = make(B, H, Nq, Nk, d, dtype, 50 + si)
        scale = float(np.float32(1 / math.sqrt(d)))
        ro, rl = oracle.attn_kv(q64, k64, v64, scale, causal)
        for splits in (0, 1, 7):
            say("decode", dtype, d, causal, (B, H, Nq, Nk), "splits", splits)
            o, l = run(attn, q, k, v, dtype, scale, causal, splits=splits)
            gu.assert_close(o, ro, gu.TOL_H16, f"decode {B}x{H}x{Nq}x{Nk} splits {splits}")
            gu.assert_lse(l, rl, gu.TOL_LSE_H16, "decode")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_decode_padding_and_empty_rows(attn, dtype):
    """Key padding (random valid lengths, one cache fully padded) and causal rows
    that precede the cache (Nq > Nk) give exact zeros and -inf."""
    B, H, Nq, Nk, d = 4, 2, 8, 700, 128
    q, q64, k, k64, v, v64 = make(B, H, Nq, Nk, d, dtype, 60)
    mask = synth.c2_mask(B, Nk)
    ro, rl = oracle.attn_kv(q64, k64, v64, S01, False, mask)
    for splits in (0, 3):
        say("decode padding", dtype, splits)
        o, l = run(attn, q, k, v, dtype, S01, False, mask, splits)
        gu.assert_close(o, ro, gu.TOL_H16, "decode padding")
        gu.assert_lse(l, rl, gu.TOL_LSE_H16, "decode padding")
        assert np.all(o[1] == 0) and np.all(np.isneginf(l[1]))
    q, q64, k, k64, v, v64 = make(1, 2, 20, 12, 64, dtype, 61)
    ro, rl = oracle.attn_kv(q64, k64, v64, S01, True)
    say("decode Nq > Nk causal", dtype)
    o, l = run(attn, q, k, v, dtype, S01, True, splits=2)
    gu.assert_close(o, ro, gu.TOL_H16, "decode Nq > Nk")
    gu.assert_lse(l, rl, gu.TOL_LSE_H16, "decode Nq > Nk")
    assert np.all(o[:, :, :8] == 0) and np.all(np.isneginf(l[:, :, :8]))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_decode_scattered_padding_unaligned_rows(attn, d, causal):
    """Key padding with an odd cache length (mask rows of odd batches are not
    4-byte aligned, so flags are read byte by byte there), scattered padded
    keys (tiles with and without a padded key), a fully padded cache (every
    tile skipped) and a cache whose first 600 keys are padded (its first
    tiles are wholly padded), with several query rows and key splits."""
    B, H, Nq, Nk = 4, 2, 5, 1001
    q, q64, k, k64, v, v64 = make(B, H, Nq, Nk, d, "bf16", 62)
    rng = np.random.default_rng([62, Nk, 99])
    mask = (rng.random((B, Nk)) < 0.01).astype(np.uint8)
    mask[1, :] = 1
    mask[2, :600] = 1
    ro, rl = oracle.attn_kv(q64, k64, v64, S01, causal, mask)
    for splits in (0, 3):
        say("decode scattered padding", d, causal, splits)
        o, l = run(attn, q, k, v, "bf16", S01, causal, mask, splits)
        gu.assert_close(o, ro, gu.TOL_H16, f"decode scattered padding d{d} causal={causal} splits {splits}")
        gu.assert_lse(l, rl, gu.TOL_LSE_H16, "decode scattered padding")
        assert np.all(o[1] == 0) and np.all(np.isneginf(l[1]))


def test_decode_empty_cache_and_sizes(attn):
    import torch
    q = torch.zeros((1, 2, 3, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    say("decode Nk = 0")
    o, l = attn.decode_fwd(q, k, k.clone(), out_fp32=True)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(l))
    q0 = torch.zeros((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    k1 = torch.zeros((1, 2, 5, 64), dtype=torch.bfloat16, device="cuda")
    attn.decode_fwd(q0, k1, k1.clone())


def test_decode_equals_tail_of_causal_forward(attn):
    """The last rows of the causal forward (attn_fwd) and the same rows decoded
    against the whole cache agree to the 16-bit gate."""
    import torch
    p = synth.make_qkv(1, 4, 1500, 128, "bf16", 62)
    q, k, v = synth.upload(p)
    of, lf = attn.fwd(q, k, v, causal=True, out_fp32=True)
    od, ld = attn.decode_fwd(q[:, :, -9:].contiguous(), k, v, causal=True, out_fp32=True)
    torch.cuda.synchronize()
    assert gu.max_abs(gu.host(od), gu.host(of)[:, :, -9:]) <= gu.TOL_H16
    assert gu.max_abs(gu.host(ld), gu.host(lf)[:, :, -9:]) <= gu.TOL_LSE_H16


def test_decode_benchmark_shape(attn):
    """B8 H32, one query row per head against an 8192-key cache, d128 bf16
    (the decode benchmark's launch), every row against the oracle."""
    B, H, Nq, Nk, d = 8, 32, 1, 8192, 128
    q, q64, k, k64, v, v64 = make(B, H, Nq, Nk, d, "bf16", 7)
    scale = float(np.float32(1 / math.sqrt(d)))
    say("decode benchmark shape")
    ro, rl = oracle.attn_kv(q64, k64, v64, scale, False)
    o, l = run(attn, q, k, v, "bf16", scale, False)
    gu.assert_close(o, ro, gu.TOL_H16, "decode bench shape")
    gu.assert_lse(l, rl, gu.TOL_LSE_H16, "decode bench shape")
    ob, _ = run(attn, q, k, v, "bf16", scale, False, out_fp32=False)
    err = np.abs(ob - ro) - gu.half_ulp(ro, "bf16")
    assert err.max() <= gu.TOL_H16
