"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerances (stated once, used by every parity test):
* bf16 inputs, fp32 accumulation, bf16 output: max |O_gpu - O_ref| <= 2e-2
* fp32 path: max |O_gpu - O_ref| <= 1e-5
* LSE: both -inf, or |LSE_gpu - LSE_ref| <= 1e-3 * max(1, |LSE_ref|)
* no NaN anywhere; rows without a valid key have O = 0 exactly and LSE = -inf.
"""
import numpy as np

O_TOL = {"bf16": 2e-2, "fp32": 1e-5}
LSE_RTOL = 1e-3


def check(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    """Assert the GPU rows match the oracle rows; return (max O err, max LSE err)."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    assert not np.isnan(o_gpu).any(), f"{what}: NaN in O"
    assert not np.isnan(lse_gpu).any(), f"{what}: NaN in LSE"
    empty_ref = np.isneginf(lse_ref)
    empty_gpu = np.isneginf(lse_gpu)
    assert np.array_equal(empty_ref, empty_gpu), (
        f"{what}: -inf LSE placement differs at {np.argwhere(empty_ref != empty_gpu)[:5]}")
    assert np.all(o_gpu[empty_ref] == 0.0), f"{what}: rows without valid keys are not 0"
    assert np.all(np.isfinite(lse_gpu[~empty_ref])), f"{what}: non-finite LSE"
    o_err = float(np.max(np.abs(o_gpu - o_ref))) if o_ref.size else 0.0
    fin = ~empty_ref
    lse_err = 0.0
    if fin.any():
        rel = np.abs(lse_gpu[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))
        lse_err = float(rel.max())
    assert o_err <= O_TOL[dtype], f"{what}: max |dO| = {o_err:.3e} > {O_TOL[dtype]}"
    assert lse_err <= LSE_RTOL, f"{what}: LSE rel err {lse_err:.3e} > {LSE_RTOL}"
    return o_err, lse_err
