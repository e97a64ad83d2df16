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


to_torch = synth.to_torch
upload = synth.upload
sample_rows = synth.sample_rows


def mask_to_torch(mask):
    import torch
    return None if mask is None else torch.from_numpy(np.ascontiguousarray(mask, np.uint8)).cuda()


def host(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


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
