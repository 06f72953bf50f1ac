"""Pins of the FP8 oracle to facts that do not come from the oracle itself.

Sources: the OCP E4M3 format (closed-form codes, ordering, sign symmetry), torch's
float8_e4m3fn cast on the CPU (a library special case covering every code), and
invariants of attention under the per-tensor dequantisation factors (page "Fused
Multi-Head Attention", quantization item of the section on how fused attention
combines with other techniques).  ``DECODE_PINS`` take a decoder as an argument so
that ``test_planted_decode_mistakes_are_caught`` shows each planted mistake fails one.
No test here touches a GPU.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8_oracle as F8
from exact_attention_89_amd.workloads import quantize_e4m3, random_fp8_case

CODES = np.arange(256, dtype=np.uint8)


def pin_torch_cast(dec):
    """Every code against torch's float8_e4m3fn -> float64 cast (NaN where torch has NaN)."""
    ref = torch.from_numpy(CODES.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = dec(CODES)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def pin_closed_forms(dec):
    """Codes whose values the format fixes: 1, the extremes, the subnormal steps, NaN."""
    table = {0x00: 0.0, 0x38: 1.0, 0x40: 2.0, 0x30: 0.5, 0x3C: 1.5, 0x7E: 448.0,
             0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 1.875 * 2.0 ** -6,
             0xB8: -1.0, 0xFE: -448.0, 0x81: -(2.0 ** -9)}
    got = dec(np.array(list(table), dtype=np.uint8))
    assert np.array_equal(got, np.array(list(table.values())))
    assert np.isnan(dec(np.array([0x7F, 0xFF], dtype=np.uint8))).all()
    assert math.copysign(1.0, float(dec(np.array([0x80], dtype=np.uint8))[0])) == -1.0


def pin_order_and_sign(dec):
    """Positive codes 0x00..0x7E increase strictly; setting bit 7 negates every value."""
    pos = dec(CODES[:0x7F])
    assert np.all(np.diff(pos) > 0)
    neg = dec(CODES[0x80:0xFF])
    assert np.array_equal(neg, -pos)
    # 8 codes per binade above the subnormals: code + 8 doubles the value
    assert np.array_equal(dec(CODES[0x10:0x77]), 2.0 * dec(CODES[0x08:0x6F]))


DECODE_PINS = [pin_torch_cast, pin_closed_forms, pin_order_and_sign]


@pytest.mark.parametrize("pin", DECODE_PINS, ids=lambda p: p.__name__)
def test_decode_pin(pin):
    pin(F8.e4m3_decode)


def _mut_bias8(c):
    c = np.asarray(c).astype(np.int64)
    v = F8.e4m3_decode(c)
    return np.where((c & 0x78) != 0, v / 2.0, v)


def _mut_no_subnormal(c):
    c = np.asarray(c).astype(np.int64)
    v = F8.e4m3_decode(c)
    return np.where(((c & 0x78) == 0) & ((c & 7) != 0), np.sign(v) * 2.0 ** -6, v)


def _mut_fnuz_nan(c):
    c = np.asarray(c).astype(np.int64)
    v = F8.e4m3_decode(c)
    return np.where(c == 0x80, np.nan, v)


def _mut_inf_top(c):
    c = np.asarray(c).astype(np.int64)
    v = F8.e4m3_decode(c)
    return np.where((c & 0x7F) == 0x7E, np.sign(v) * np.inf, v)


def _mut_fraction_16(c):
    c = np.asarray(c).astype(np.int64)
    e = (c >> 3) & 0xF
    f = c & 7
    v = F8.e4m3_decode(c)
    alt = np.where(c & 0x80, -1.0, 1.0) * (1.0 + f / 16.0) * np.exp2(e - 7.0)
    return np.where((e > 0) & ~np.isnan(v), alt, v)


MUTANTS = [_mut_bias8, _mut_no_subnormal, _mut_fnuz_nan, _mut_inf_top, _mut_fraction_16]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_planted_decode_mistakes_are_caught(mutant):
    failed = 0
    for pin in DECODE_PINS:
        try:
            pin(mutant)
        except AssertionError:
            failed += 1
    assert failed >= 1, f"no pin catches {mutant.__name__}"


def _case(seed=3, B=2, H=2, Nq=19, Nk=23, D=16):
    return random_fp8_case(seed, B, H, Nq, Nk, D)


@pytest.mark.parametrize("causal", [False, True])
def test_descale_moves_between_q_and_k(causal):
    """Doubling q_descale and halving k_descale (exact in fp32) changes no score."""
    q8, k8, v8, (qd, kd, vd) = _case()
    lens = np.array([23, 9], dtype=np.int32)
    o1, l1 = oracle.attention_fp8_oracle(q8, k8, v8, 0.25, qd, kd, vd, causal, lens)
    o2, l2 = oracle.attention_fp8_oracle(q8, k8, v8, 0.25, 2 * qd, kd / 2, vd, causal, lens)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_descale_of_q_equals_scale():
    """Scores depend on scale * q_descale * k_descale only (powers of two: exact)."""
    q8, k8, v8, (qd, kd, vd) = _case()
    o1, l1 = oracle.attention_fp8_oracle(q8, k8, v8, 0.5, qd, kd, vd)
    o2, l2 = oracle.attention_fp8_oracle(q8, k8, v8, 0.25, 2 * qd, kd, vd)
    assert np.allclose(o1, o2, rtol=0, atol=1e-14) and np.allclose(l1, l2, rtol=0, atol=1e-12)


def test_v_descale_is_linear():
    """O is linear in v_descale; LSE does not depend on it."""
    q8, k8, v8, (qd, kd, vd) = _case()
    o1, l1 = oracle.attention_fp8_oracle(q8, k8, v8, 0.3, qd, kd, 1.0)
    o2, l2 = oracle.attention_fp8_oracle(q8, k8, v8, 0.3, qd, kd, 0.75)
    assert np.allclose(o2, 0.75 * o1, rtol=1e-14, atol=1e-12) and np.array_equal(l1, l2)


def test_single_key_and_zero_query_closed_forms():
    """Nk = 1: O = the dequantised value row, LSE = the one score.  Q = 0: O = mean of
    the dequantised values, LSE = ln(number of keys)."""
    q8, k8, v8, (qd, kd, vd) = _case(Nk=1)
    o, lse = oracle.attention_fp8_oracle(q8, k8, v8, 0.2, qd, kd, vd)
    vv = vd * F8.e4m3_decode(v8)
    assert np.array_equal(o, np.broadcast_to(vv, o.shape))
    sigma = float(np.float32(0.2))   # the scale reaches the kernel as a C float
    s = sigma * np.einsum("bhqd,bhkd->bhqk", qd * F8.e4m3_decode(q8), kd * F8.e4m3_decode(k8))
    assert np.allclose(lse, s[..., 0], rtol=1e-13, atol=1e-13)
    q8, k8, v8, (qd, kd, vd) = _case(Nk=11)
    z = np.zeros_like(q8)
    o, lse = oracle.attention_fp8_oracle(z, k8, v8, 0.2, qd, kd, vd)
    mean = (vd * F8.e4m3_decode(v8)).mean(axis=2, keepdims=True)
    assert np.allclose(o, np.broadcast_to(mean, o.shape), rtol=0, atol=1e-12)
    assert np.allclose(lse, math.log(11), rtol=0, atol=1e-12)


def test_fully_masked_rows():
    q8, k8, v8, (qd, kd, vd) = _case()
    o, lse = oracle.attention_fp8_oracle(q8, k8, v8, 0.2, qd, kd, vd, True,
                                         np.array([0, 5], dtype=np.int32))
    assert np.all(o[0] == 0) and np.all(lse[0] == -np.inf)
    assert np.isfinite(lse[1]).all() and not np.isnan(o).any()


def test_rejects_bad_descale():
    q8, k8, v8, (qd, kd, vd) = _case()
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(ValueError):
            oracle.attention_fp8_oracle(q8, k8, v8, 0.2, bad, kd, vd)


def test_rows_variant_matches_whole():
    q8, k8, v8, (qd, kd, vd) = _case()
    o, lse = oracle.attention_fp8_oracle(q8, k8, v8, 0.2, qd, kd, vd, True)
    samples = [(0, 0, 0), (1, 1, 18), (0, 1, 7)]
    ro, rl = oracle.attention_fp8_oracle_rows(q8, k8, v8, 0.2, qd, kd, vd, True, None, samples)
    for n, (b, h, i) in enumerate(samples):
        # the same definition on one row; a matrix product of one row may round differently
        assert np.allclose(ro[n], o[b, h, i], rtol=0, atol=1e-13)
        assert abs(rl[n] - lse[b, h, i]) <= 1e-13


def test_quantizer_round_trip():
    """The input generator's codes decode to within half an E4M3 step of x / descale."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal(4096).astype(np.float32)
    codes, d = quantize_e4m3(x)
    y = F8.e4m3_decode(codes)
    t = x.astype(np.float64) / d
    step = np.exp2(np.maximum(np.floor(np.log2(np.maximum(np.abs(t), 2.0 ** -9))), -6) - 3)
    assert np.all(np.abs(y - t) <= step / 2 + 1e-12)
    assert np.max(np.abs(y)) == 448.0


def _kernel_model(q8, k8, v8, ds, scale, causal):
    """A float32 model of the FP8 kernel's arithmetic for one (batch, head), on the CPU:
    fp32 scores of the decoded codes, 64-key tiles, an exponent reference that moves only
    when the tile maximum exceeds it by more than 2 (log2 units), weights 2^6 exp2(x)
    rounded to E4M3 by torch's cast before the value product, the normaliser over the
    unrounded weights, O = v_descale acc / l."""
    f32 = np.float32
    q = oracle.e4m3_decode(q8).astype(f32)
    k = oracle.e4m3_decode(k8).astype(f32)
    v = oracle.e4m3_decode(v8).astype(f32)
    c = f32(f32(f32(scale) * f32(ds[0])) * f32(ds[1])) * f32(1.4426950408889634)
    s = (q @ k.T).astype(f32)
    nq, nk = s.shape
    if causal:
        s = np.where(np.arange(nk)[None, :] <= np.arange(nq)[:, None], s, f32(-np.inf))
    m = np.full(nq, -np.inf, f32)
    l = np.zeros(nq, f32)
    acc = np.zeros((nq, v.shape[1]), f32)
    for lo in range(0, nk, 64):
        blk = s[:, lo:lo + 64] * c
        mx = blk.max(axis=1)
        move = mx > m + f32(2)
        m_new = np.where(move, mx, m)
        m_use = np.where(m_new == -np.inf, f32(0), m_new)
        alpha = np.where(move, np.exp2(m - m_use), f32(1)).astype(f32)
        l *= alpha
        acc *= alpha[:, None]
        m = m_new
        w = np.exp2(blk - (m_use - f32(6))[:, None]).astype(f32)
        l += w.sum(axis=1, dtype=f32)
        wr = torch.from_numpy(w).to(torch.float8_e4m3fn).to(torch.float32).numpy()
        acc += wr @ v[lo:lo + 64]
    return (f32(ds[2]) * acc / l[:, None]).astype(np.float64)


@pytest.mark.parametrize("nq,nk,d,causal,std", [(64, 4096, 128, False, 1.0),
                                                (96, 1000, 64, True, 1.0),
                                                (32, 2048, 128, False, 3.0)])
def test_o_bound_covers_a_model_of_the_kernel_arithmetic(nq, nk, d, causal, std):
    """The element-wise FP8 bound of the parity tests holds for a float32 model of the
    kernel's steps (the rounding of the weights to E4M3 dominates), and is not loose: the
    model's error reaches a visible fraction of it."""
    from tests.parity import fp8_o_bound, fp8_score_abs

    q8, k8, v8, ds = random_fp8_case(11, 1, 1, nq, nk, d, std=std)
    scale = 1.0 / math.sqrt(d)
    o_ref, _, P = oracle.attention_fp8_oracle(q8, k8, v8, scale, *ds, causal=causal,
                                              return_probs=True)
    o_model = _kernel_model(q8[0, 0], k8[0, 0], v8[0, 0], ds, scale, causal)
    sa = fp8_score_abs(oracle.dequantize(q8, ds[0]), oracle.dequantize(k8, ds[1]), scale)
    bound = fp8_o_bound(P, oracle.dequantize(v8, ds[2]), o_ref, sa)[0, 0]
    ratio = np.abs(o_model - o_ref[0, 0]) / bound
    assert ratio.max() <= 1.0
    assert ratio.max() >= 0.02
