"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerances (stated once, used by every parity test):
* bf16 inputs, fp32 accumulation, bf16 output: max |O_gpu - O_ref| <= 2e-2
* fp32 path: max |O_gpu - O_ref| <= 1e-5
* LSE: both -inf, or |LSE_gpu - LSE_ref| <= 1e-3 * max(1, |LSE_ref|)
* no NaN anywhere; rows without a valid key have O = 0 exactly and LSE = -inf.
* FP8 path (E4M3 inputs, P rounded to E4M3 before P.V): an element-wise bound
  derived from that rounding, ``fp8_o_bound`` below; LSE and the -inf rules as above.
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


def fp8_o_bound(P, v_deq, o_ref):
    """Largest |O_gpu - O_ref| the FP8 kernel's arithmetic allows, element by element.

    P [..., Nq, Nk]: the oracle's probabilities; v_deq [..., Nk, D]: the dequantised
    values; o_ref [..., Nq, D].  The kernel rounds each weight p' = 2^6 exp2(s c - m)
    (m <= the row maximum) to E4M3.  Where P_j >= 2^-12 max_k P_k, p' is at least
    2^-6 (E4M3's smallest normal) and its relative rounding error is at most 2^-4;
    below that the error is at most the weight itself.  The normaliser uses the
    unrounded weights, so O changes by sum_j (error_j / l) v_j.  On top: fp32
    accumulation and exponentials (1e-3 of sum_j P_j |v_j|, far above their
    rounding) and the final bf16 rounding (2^-8 relative).
    """
    P = np.asarray(P, dtype=np.float64)
    av = np.abs(np.asarray(v_deq, dtype=np.float64))
    pmax = P.max(axis=-1, keepdims=True)
    w = np.where(P >= pmax * 2.0 ** -12, 2.0 ** -4 * P, P)
    rounding = w @ av
    arith = 1e-3 * (P @ av)
    return rounding + arith + 2.0 ** -8 * (np.abs(o_ref) + rounding + arith) + 1e-6


def check_fp8(o_gpu, lse_gpu, o_ref, lse_ref, bound, what=""):
    """FP8 parity: the element-wise bound on O, the common LSE / -inf / NaN rules.

    Returns (max |dO|, max |dO| / bound, rms |dO|, max LSE err)."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    assert not np.isnan(o_gpu).any(), f"{what}: NaN in O"
    assert not np.isnan(lse_gpu).any(), f"{what}: NaN in LSE"
    empty_ref = np.isneginf(lse_ref)
    assert np.array_equal(empty_ref, np.isneginf(lse_gpu)), f"{what}: -inf LSE placement differs"
    assert np.all(o_gpu[empty_ref] == 0.0), f"{what}: rows without valid keys are not 0"
    err = np.abs(o_gpu - o_ref)
    ratio = float((err / bound).max()) if err.size else 0.0
    fin = ~empty_ref
    lse_err = 0.0
    if fin.any():
        rel = np.abs(lse_gpu[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))
        lse_err = float(rel.max())
    worst = np.unravel_index(int(np.argmax(err / bound)), err.shape) if err.size else ()
    assert ratio <= 1.0, (f"{what}: |dO| exceeds the FP8 bound by x{ratio:.3f} at {worst} "
                          f"(|dO| {err[worst]:.3e}, bound {bound[worst]:.3e})")
    assert lse_err <= LSE_RTOL, f"{what}: LSE rel err {lse_err:.3e} > {LSE_RTOL}"
    o_max = float(err.max()) if err.size else 0.0
    rms = float(np.sqrt((err ** 2).mean())) if err.size else 0.0
    return o_max, ratio, rms, lse_err
