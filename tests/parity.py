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


U32 = 2.0 ** -24                  # unit roundoff of fp32


def gamma(n):
    """Bound on the relative error of an fp32 sum of n terms in any order, n u / (1 - n u)."""
    return n * U32 / (1.0 - n * U32)


def fp8_score_abs(q_deq, k_deq, scale):
    """Per query row, max over keys of |scale log2 e| sum_d |q_d k_d| (log2 units): the size
    the fp32 score sums work at, which bounds their rounding."""
    q = np.abs(np.asarray(q_deq, dtype=np.float64))
    k = np.abs(np.asarray(k_deq, dtype=np.float64))
    return abs(scale) * 1.4426950408889634 * (q @ np.swapaxes(k, -1, -2)).max(axis=-1)


def fp8_o_bound(P, v_deq, o_ref, score_abs=None):
    """Largest |O_gpu - O_ref| the FP8 kernel's arithmetic allows, element by element.

    P [..., Nq, Nk]: the oracle's probabilities; v_deq [..., Nk, D]: the dequantised
    values; o_ref [..., Nq, D]; score_abs [..., Nq] (``fp8_score_abs``; None: 64).

    Rounding of the weights.  The kernel rounds each weight p' = 2^6 exp2(x), x = s c - m
    (m, the exponent reference at the time, <= the row maximum), to E4M3.  Where
    P_j >= 2^-12 max_k P_k, p' >= 2^-6 (E4M3's smallest normal), so its relative rounding
    error is at most 2^-4; below that the error is at most the weight itself (a weight
    under half the smallest subnormal becomes 0).  The normaliser sums the unrounded
    weights, so O moves by sum_j (error_j / l) v_j: the first term.

    Arithmetic in fp32 (u = 2^-24, round to nearest; gamma_n as in ``gamma``), from the
    operations the kernel performs, for the weights at or above 2^-12 of the largest (the
    error of the smaller ones is already counted whole in the first term):
      * P.V: a product of two E4M3 values is exact in fp32; each product passes through
        at most Nk additions, in whatever order the matrix instructions take them, and
        at most R rescalings of the accumulator by the correction factor, so the sum
        errs by at most gamma_(Nk + R) sum_j p'_j |v_j|;
      * the normaliser: 32 weights to a lane in a tree of depth 10 per 64-key tile, one
        term per tile into the running sum, R rescalings, and the two halves of the row:
        gamma_(12 + Nk/64 + R) relative, below the P.V term's;
      * a weight's exponent x: the score is a sum of D exact products, off by at most
        gamma_D sum_d |q_d k_d|; the combined factor c = scale * q_descale * k_descale is
        two fp32 products (2 u relative); the fused multiply-add rounds once (u |x|); so
        x is off by at most (gamma_D + 2 u) score_abs + u |x|, and exp2 multiplies the
        weight by 2 to that power, plus the hardware exp2's own error (within 2 ulp,
        4 u relative); |x| <= 8 for these weights (2^-6 <= p' <= 2^8: the reference
        lags the maximum by at most 2);
      * the correction factor exp2(m_old - m_new) of each rescaling multiplies the old
        weights' share of both the accumulator and the normaliser, so only its own
        error, at most ln 2 u 2 score_abs + 4 u, enters, once per rescaling;
      * O = v_descale acc / l: two more roundings, 2 u.
    R, the number of rescalings: the reference moves only when the maximum exceeds it by
    more than 2 (log2 units) and stays within [-score_abs, score_abs], so R <=
    score_abs + 1.  The sum of these relative errors, times (1 + 2^-4) sum_j P_j
    |v_j| (the rounded weights exceed P by at most 2^-4), bounds their effect on O.
    On top, the final bf16 rounding: 2^-8 relative.
    """
    P = np.asarray(P, dtype=np.float64)
    av = np.abs(np.asarray(v_deq, dtype=np.float64))
    nk, d = P.shape[-1], av.shape[-1]
    pmax = P.max(axis=-1, keepdims=True)
    w = np.where(P >= pmax * 2.0 ** -12, 2.0 ** -4 * P, P)
    rounding = w @ av
    sa = 64.0 if score_abs is None else np.asarray(score_abs, dtype=np.float64)[..., None]
    ln2 = np.log(2.0)
    n_rescale = np.floor(sa) + 1.0
    exponent = ln2 * ((gamma(d) + 2 * U32) * sa + 8 * U32) + 4 * U32
    correction = n_rescale * (ln2 * 2 * U32 * sa + 4 * U32)
    rel = (gamma(nk + n_rescale) + gamma(12 + -(-nk // 64) + n_rescale) + exponent
           + correction + 2 * U32)
    arith = rel * (1.0 + 2.0 ** -4) * (P @ av)
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
