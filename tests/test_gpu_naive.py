"""GPU: the materialising baseline (attn_naive_fwd: S = scale Q K^T stored in
the input type, row softmax in fp32 with P stored back in the input type, then
P V with fp32 accumulation), the pages' "baseline attention", against the fp64
oracle.  fp32 runs at the fp32 gate.  In 16-bit modes the gate follows from the
two stores: each score carries at most half an ulp of the input type at its
magnitude, each weight half an ulp relative, and the output moves by at most
2 max|v| per unit of score error (d o / d s_j = p_j (v_j - o)); the fp32-output
flavour removes the output rounding.  Fully masked rows must still come out as
exact zeros with lse = -inf."""
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


def gate16(p, scale, dtype):
    """Bound on |naive - oracle| from the stores of S and P in the input type."""
    mant = 7 if dtype == "bf16" else 10
    smax = abs(scale) * float(np.abs(np.einsum("bhid,bhjd->bhij", p.q64, p.k64)).max())
    half_ulp_s = 0.5 * 2.0 ** (math.floor(math.log2(max(smax, 1e-30))) - mant)
    half_ulp_p = 2.0 ** -(mant + 1)
    vmax = float(np.abs(p.v64).max())
    return 2 * vmax * (half_ulp_s + half_ulp_p) + 1e-5, half_ulp_s + 2 * half_ulp_p + 1e-5


def run(A, p, scale, causal, mask, out_fp32):
    import torch
    q, k, v = gu.upload(p)
    o, l = A.naive_fwd(q, k, v, scale=scale, causal=causal, key_padding_mask=gu.mask_to_torch(mask), out_fp32=out_fp32)
    torch.cuda.synchronize()
    return gu.host(o), gu.host(l)


@pytest.mark.parametrize("causal", [False, True])
def test_naive_c1_fp32(attn, causal):
    """B1 H1 N128 d64 fp32, scale 1/8: everything in fp32, the fp32 gate."""
    p = synth.make_qkv(1, 1, 128, 64, "f32", 1)
    say("naive C1 fp32 causal", causal)
    o, l = run(attn, p, 0.125, causal, None, False)
    ro, rl = oracle.attn(p.q64, p.k64, p.v64, 0.125, causal)
    gu.assert_close(o, ro, gu.TOL_F32, "naive C1 O")
    gu.assert_lse(l, rl, gu.TOL_LSE_F32, "naive C1 lse")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_naive_c2_causal_padding_and_empty_rows(attn, dtype):
    """B4 H16 N1024 d64 causal with the C2 key-padding mask (batch 1 fully
    padded): the storage-derived gate, exact (+0, -inf) on the empty rows."""
    B, H, N, d = 4, 16, 1024, 64
    p = synth.make_qkv(B, H, N, d, dtype, 2)
    mask = synth.c2_mask(B, N)
    say("naive C2", dtype)
    o, l = run(attn, p, 0.125, True, mask, True)
    ro, rl = oracle.attn(p.q64, p.k64, p.v64, 0.125, True, mask)
    tol, tl = gate16(p, 0.125, dtype)
    err = gu.assert_close(o, ro, tol, "naive C2 O")
    gu.assert_lse(l, rl, tl, "naive C2 lse")
    empty = ~np.isfinite(rl)
    assert empty[1].all()
    assert np.all(o[empty] == 0) and not np.signbit(o[empty]).any() and np.all(np.isneginf(l[empty]))
    say(f"naive C2 {dtype}: max|d| {err:.3e} (gate {tol:.3e}), mean {np.abs(o - ro)[~empty].mean():.2e}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_naive_ragged_length(attn, dtype):
    """N = 1000 (not a multiple of the baseline's 64 x 64 tiles), d = 128."""
    p = synth.make_qkv(1, 3, 1000, 128, dtype, 3, variant=7)
    scale = float(np.float32(128 ** -0.5))
    say("naive ragged", dtype)
    o, l = run(attn, p, scale, False, None, dtype != "f32")
    ro, rl = oracle.attn(p.q64, p.k64, p.v64, scale, False)
    tol, tl = (gu.TOL_F32, gu.TOL_LSE_F32) if dtype == "f32" else gate16(p, scale, dtype)
    gu.assert_close(o, ro, tol, "naive ragged O")
    gu.assert_lse(l, rl, tl, "naive ragged lse")
