"""GPU parity at long sequence lengths (the largest single-head shapes the
tests run): the forward, the block-sparse forward and the key/value-cache path
on sampled rows against the fp64 oracle evaluated on those rows only.

Every case prints what it runs (flushed) before touching the GPU.
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


def check_rows(o, l, p, rows, scale, causal, tol, tl, what, key_mask_of=None):
    """Sampled rows against oracle.attn_rows; key_mask_of(bh, i) gives the extra
    per-row key mask ([N] bytes, 1 = excluded) of a block-sparse case."""
    B, H, N, d = p.q64.shape
    if key_mask_of is None:
        ro, rl = oracle.attn_rows(p.q64, p.k64, p.v64, scale, rows, causal)
        got = o.reshape(-1, d)[rows]
        gu.assert_close(got, ro, tol, what)
        gu.assert_lse(l.reshape(-1)[rows], rl, tl, what)
        return
    for r in rows:
        bh, i = divmod(int(r), N)
        sl = slice(bh, bh + 1)
        ro, rl = oracle.attn_rows(p.q64[:, sl], p.k64[:, sl], p.v64[:, sl], scale, np.array([i]), causal,
                                  key_mask_of(bh, i)[None, :])
        gu.assert_close(o[0, bh, i][None], ro, tol, f"{what} row {r}")
        gu.assert_lse(l[0, bh, i][None], rl, tl, f"{what} row {r}")


@pytest.mark.parametrize("N, d, H", [(262144, 64, 1), (131072, 128, 2)])
def test_long_causal_forward_bf16(attn, N, d, H):
    """Causal bf16 forward at N = 262144 (d 64) and 131072 (d 128), default
    tiles, fp32 output; 64-bit offsets and the causal tile bound at length."""
    import torch
    p = synth.make_qkv(1, H, N, d, "bf16", 70)
    q, k, v = gu.upload(p)
    say("long forward", N, d, H)
    o, l = attn.fwd(q, k, v, scale=float(np.float32(d ** -0.5)), causal=True, out_fp32=True)
    torch.cuda.synchronize()
    rows = synth.sample_rows(1, H, N, 12, 1)
    check_rows(gu.host(o), gu.host(l), p, rows, float(np.float32(d ** -0.5)), True, gu.TOL_H16, gu.TOL_LSE_H16, f"long N{N} d{d}")


def test_long_forward_fp32(attn):
    """fp32 inputs at N = 131072, d 64, causal, within 1e-5 on sampled rows."""
    import torch
    N, d = 131072, 64
    p = synth.make_qkv(1, 1, N, d, "f32", 71)
    q, k, v = gu.upload(p)
    say("long forward fp32", N)
    o, l = attn.fwd(q, k, v, scale=0.125, causal=True)
    torch.cuda.synchronize()
    rows = synth.sample_rows(1, 1, N, 12, 2)
    check_rows(gu.host(o), gu.host(l), p, rows, 0.125, True, gu.TOL_F32, gu.TOL_LSE_F32, "long fp32")


def test_long_block_sparse(attn):
    """Block-sparse at N = 262144 (4096 blocks of 64 per side, so 64 words of
    the flag scan per workgroup): sliding window of 2 blocks plus one global
    block, causal."""
    import torch
    N, d = 262144, 64
    p = synth.make_qkv(1, 1, N, d, "bf16", 72)
    q, k, v = gu.upload(p)
    bm = synth.block_mask(1, 1, N, 64, 72, "local_global", band=2, n_global=1)
    say("long block-sparse", N)
    o, l = attn.fwd_sparse(q, k, v, torch.from_numpy(bm).cuda(), block=64, scale=0.125, causal=True, out_fp32=True)
    torch.cuda.synchronize()
    rows = synth.sample_rows(1, 1, N, 12, 3)

    def key_mask_of(bh, i):
        return (np.repeat(bm[0, bh, i // 64], 64)[:N] == 0).astype(np.uint8)

    check_rows(gu.host(o), gu.host(l), p, rows, 0.125, True, gu.TOL_H16, gu.TOL_LSE_H16, "long sparse", key_mask_of)


def test_long_key_value_cache(attn):
    """Decode against a cache of 2^19 keys (d 128, four query rows, causal
    aligned to the end of the cache), default key split, against the oracle's
    query-block definition."""
    import torch
    Nk, Nq, d = 1 << 19, 4, 128
    kv = synth.make_qkv(1, 1, Nk, d, "bf16", 73)
    qp = synth.make_qkv(1, 1, Nq, d, "bf16", 73, variant=1)
    q = synth.to_torch(qp.q, "bf16")
    k = synth.to_torch(kv.k, "bf16")
    v = synth.to_torch(kv.v, "bf16")
    say("long decode", Nk)
    o, l = attn.decode_fwd(q, k, v, scale=float(np.float32(d ** -0.5)), causal=True, out_fp32=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_kv(qp.q64, kv.k64, kv.v64, float(np.float32(d ** -0.5)), True)
    gu.assert_close(gu.host(o), ro, gu.TOL_H16, "long decode")
    gu.assert_lse(gu.host(l), rl, gu.TOL_LSE_H16, "long decode")


def _big_head_problem(H, N, d, config_id):
    """[1, H, N, d] bf16 q, k, v on the device with seeded data in heads 0 and
    H - 1 and zeros elsewhere; returns the tensors and the two heads' problems."""
    import torch
    heads = {0: synth.make_qkv(1, 1, N, d, "bf16", config_id, 0),
             H - 1: synth.make_qkv(1, 1, N, d, "bf16", config_id, 1)}
    q, k, v = (torch.zeros((1, H, N, d), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    for h, p in heads.items():
        hq, hk, hv = gu.upload(p)
        q[0, h].copy_(hq[0, 0])
        k[0, h].copy_(hk[0, 0])
        v[0, h].copy_(hv[0, 0])
    torch.cuda.synchronize()
    return q, k, v, heads


def test_forward_beyond_2_31_elements(attn):
    """Each of q, k, v and o holds more than 2^31 elements (B1 H136 N131072
    d128: 2.28e9, the last heads past 4 GiB of bf16 and 8 GiB of fp32 output).
    Sampled rows of the first and last heads against the oracle: every element
    and byte offset is formed in 64 bits."""
    import torch
    H, N, d = 136, 131072, 128
    assert H * N * d > 2 ** 31 and (H - 1) * N * d * 2 >= 2 ** 32
    say("forward beyond 2^31 elements", H, N, d)
    q, k, v, heads = _big_head_problem(H, N, d, 72)
    o, l = attn.fwd(q, k, v, scale=float(np.float32(d ** -0.5)), causal=True, out_fp32=True)
    torch.cuda.synchronize()
    rows = synth.sample_rows(1, 1, N, 10, 2)
    for h, p in heads.items():
        check_rows(gu.host(o[0, h][None, None]), gu.host(l[0, h][None, None]), p, rows, float(np.float32(d ** -0.5)), True,
                   gu.TOL_H16, gu.TOL_LSE_H16, f"big head {h}")
    # a head in between holds zeros: every score is 0, so o = mean of zero rows = 0
    mid = gu.host(o[0, H // 2, ::4096])
    assert np.all(mid == 0.0)
    del q, k, v, o, l
    torch.cuda.empty_cache()


def test_decode_beyond_2_31_elements(attn):
    """Key/value cache of more than 2^31 elements per tensor (B1 H136 Nk131072
    d128), one query row per head; the first and last heads against the oracle."""
    import torch
    H, Nk, d = 136, 131072, 128
    say("decode beyond 2^31 elements", H, Nk, d)
    _, k, v, heads = _big_head_problem(H, Nk, d, 73)
    qp = synth.make_qkv(1, H, 1, d, "bf16", 73, 2)
    q = gu.upload(qp)[0]
    o, l = attn.decode_fwd(q, k, v, scale=float(np.float32(d ** -0.5)), out_fp32=True)
    torch.cuda.synchronize()
    for h, p in heads.items():
        ro, rl = oracle.attn_kv(qp.q64[:, h:h + 1], p.k64, p.v64, float(np.float32(d ** -0.5)))
        gu.assert_close(gu.host(o[0, h]), ro[0, 0], gu.TOL_H16, f"decode big head {h}")
        gu.assert_lse(gu.host(l[0, h]), rl[0, 0], gu.TOL_LSE_H16, f"decode big head {h}")
    del q, k, v, o, l
    torch.cuda.empty_cache()
