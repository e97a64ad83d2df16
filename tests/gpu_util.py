"""Shared helpers of the GPU parity tests: device upload of the seeded inputs,
tolerances, and row sampling for sizes the oracle cannot do in full."""
import numpy as np

import synth

# Tolerances on max |GPU - oracle|, stated by the target of this library:
# fp32 inputs with fp32 arithmetic 1e-5; 16-bit inputs (fp32 accumulation,
# P rounded to the input type) 1.5e-2, measured on the fp32-output flavour.
TOL_F32 = 1e-5
TOL_H16 = 1.5e-2
# lse is a natural-log value of the same arithmetic.
TOL_LSE_F32 = 1e-5
TOL_LSE_H16 = 1.5e-2


def half_ulp(x, dtype):
    """Half a unit in the last place of |x| in the 16-bit storage type."""
    mant = 7 if dtype == "bf16" else 10
    ax = np.maximum(np.abs(x), 2.0 ** -14)
    return 0.5 * 2.0 ** (np.floor(np.log2(ax)) - mant)


def to_torch(arr, dtype, device="cuda"):
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, np.float32)).to(device)
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(arr, np.float16)).to(device)
    bits = np.ascontiguousarray(arr, np.uint16).view(np.int16)
    return torch.from_numpy(bits).to(device).view(torch.bfloat16)


def upload(p: synth.QKV):
    return to_torch(p.q, p.dtype), to_torch(p.k, p.dtype), to_torch(p.v, p.dtype)


def mask_to_torch(mask):
    import torch
    return None if mask is None else torch.from_numpy(np.ascontiguousarray(mask, np.uint8)).cuda()


def host(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def sample_rows(B, H, N, per_head=24, seed=0):
    """Flat row indices (b*H+h)*N + i: for every (b, h) the first and last rows,
    plus rows spread over the sequence (including every query-tile boundary
    region), for the checks at full size."""
    rng = np.random.default_rng([4242, B, H, N, seed])
    rows = []
    for bh in range(B * H):
        pick = {0, 1, min(31, N - 1), min(32, N - 1), N // 2, N - 2 if N > 1 else 0, N - 1}
        pick.update(int(x) for x in rng.integers(0, N, size=per_head))
        rows.extend(bh * N + i for i in sorted(pick) if 0 <= i < N)
    return np.array(rows, np.int64)


def max_abs(a, b):
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def assert_close(o_gpu, o_ref, tol, what=""):
    assert not np.isnan(o_gpu).any(), f"{what}: NaN in GPU output"
    err = max_abs(o_gpu, o_ref)
    assert err <= tol, f"{what}: max|d| = {err:.3e} > {tol:.1e}"
    return err


def assert_lse(lse_gpu, lse_ref, tol, what=""):
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), np.isneginf(lse_ref)), f"{what}: -inf pattern differs"
    assert not np.isnan(lse_gpu).any(), f"{what}: NaN in lse"
    err = max_abs(lse_gpu[fin], lse_ref[fin])
    assert err <= tol, f"{what}: lse max|d| = {err:.3e} > {tol:.1e}"
    return err
