"""Plain fp64 CPU oracle for attention on FP8 (e4m3) inputs.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The product
path never does, and shares no code with it: this file imports numpy and the
definition oracle of this package, nothing else.

What it computes
----------------
The page "Fused Multi-Head Attention" (section on how fused attention combines with
other inference techniques, the quantization item) says a fused kernel can take
FP8 data for its two matrix products.  The method stays exact attention: the result
it approximates is attention on the values the FP8 codes stand for.  With one
dequantisation factor per tensor (q_descale, k_descale, v_descale),

    Q = q_descale * decode(q8),  K = k_descale * decode(k8),  V = v_descale * decode(v8)
    O, LSE = attention(Q, K, V, scale, mask)

where ``attention`` is the definition in ``attn_oracle`` (scaled scores, additive
mask, stable softmax, contraction with V; LSE the natural-log log-sum-exp of the
masked scores).  A kernel that also rounds the probabilities to FP8 before the
second product approximates this result; how far it may be from it is a property
of that rounding and is stated where the kernel is tested, not here.

``decode`` follows the OCP 8-bit floating point format E4M3 (the "fn" variant:
finite values and NaN, no infinities): bit 7 is the sign, bits 6..3 a biased
exponent (bias 7), bits 2..0 the fraction.  Exponent field 0 encodes subnormals
fraction/8 * 2^-6; exponent field 15 with fraction 7 encodes NaN; every other code
is (1 + fraction/8) * 2^(exponent - 7).  The largest finite magnitude is 448.

Readings (listed in the design notes as well): the pages name FP8 but no format,
scaling granularity or output type.  E4M3 with one float32 descale per tensor is
the plainest choice; the descales are rounded to float32 before use (the kernel
receives C floats) and must be positive and finite.
"""

from __future__ import annotations

import numpy as np

from .attn_oracle import attention_oracle, attention_oracle_rows

__all__ = ["e4m3_decode", "attention_fp8_oracle", "attention_fp8_oracle_rows",
           "dequantize"]


def e4m3_decode(codes) -> np.ndarray:
    """fp64 values of OCP E4M3 codes (any integer array of bytes); NaN for the NaN codes."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    f = (c & 0x7).astype(np.float64)
    normal = (1.0 + f / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (f / 8.0) * 2.0 ** -6
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where((e == 15) & ((c & 0x7) == 7), np.nan, mag)
    return sign * mag


def _descale(x: float) -> float:
    d = float(np.float32(x))
    if not (np.isfinite(d) and d > 0.0):
        raise ValueError("descale factors must be positive and finite")
    return d


def dequantize(codes, descale: float) -> np.ndarray:
    """descale * decode(codes) in fp64 (the descale rounded to float32 first)."""
    return _descale(descale) * e4m3_decode(codes)


def attention_fp8_oracle(q8, k8, v8, scale: float, q_descale: float, k_descale: float,
                         v_descale: float, causal: bool = False, kv_lens=None,
                         return_probs: bool = False):
    """Exact attention of the dequantised FP8 tensors, in fp64.

    q8 [B,H,Nq,D], k8 [B,H,Nk,D], v8 [B,H,Nk,Dv]: E4M3 codes (uint8).  Returns O and
    LSE (and P if ``return_probs``) as ``attn_oracle.attention_oracle`` does.
    """
    return attention_oracle(dequantize(q8, q_descale), dequantize(k8, k_descale),
                            dequantize(v8, v_descale), scale, causal=causal, kv_lens=kv_lens,
                            return_probs=return_probs)


def attention_fp8_oracle_rows(q8, k8, v8, scale: float, q_descale: float, k_descale: float,
                              v_descale: float, causal: bool, kv_lens, samples):
    """``attention_fp8_oracle`` on selected rows (b, h, i) only."""
    return attention_oracle_rows(dequantize(q8, q_descale), dequantize(k8, k_descale),
                                 dequantize(v8, v_descale), scale, causal, kv_lens, samples)
