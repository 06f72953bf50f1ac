"""Seeded synthetic inputs for exact attention.

This module only draws and rounds numbers.  It holds none of attention's
arithmetic, so both the HIP path's tests and the CPU oracle's tests may use it.

Recipe (numpy ``default_rng(seed)``; draw order as listed):

* Q, K, V are iid N(0, 1), drawn as float32 with ``standard_normal``.
* bf16 workloads round every value once to bfloat16 with round-to-nearest-even
  and keep the rounded values (as float32, exactly representable), so the GPU
  and the oracle consume identical numbers.
* The padded workload draws ``kv_lens`` as integers uniform in [1, Nk] after
  Q, K, V, then sets ``kv_lens[0] = 0`` (every row of sequence 0 is fully
  masked).
* The drifting-key workload draws g ~ N(0, I_D) first, sets u = g / |g|, draws
  Q, K0, V, and forms K = K0 + 0.002 * j * u in float32 (j the 0-based key
  index, one u for all heads) before rounding to bf16.  Later keys then keep
  raising the running maximum for queries with q.u > 0.
* FP8 inputs: Q, K, V drawn as above (float32), then each tensor is quantised to
  OCP E4M3 codes with one factor per tensor: descale = fp32(amax / 448), codes =
  E4M3(x / descale) rounded to nearest even (torch's float8_e4m3fn cast, after
  clipping to +-448).  Both sides consume the codes and the descales.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(x.shape)


E4M3_MAX = 448.0


def quantize_e4m3(x: np.ndarray):
    """(codes uint8, descale float) of a float32 tensor, one descale for the tensor."""
    import torch

    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    descale = float(np.float32(amax / E4M3_MAX)) if amax > 0 else 1.0
    y = np.clip(x / np.float32(descale), -E4M3_MAX, E4M3_MAX).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return np.ascontiguousarray(codes), descale


def random_fp8_case(seed: int, B: int, H: int, Nq: int, Nk: int, D: int, std: float = 1.0):
    """A seeded FP8 case: N(0, std^2) Q and K, N(0, 1) V, each quantised to E4M3.

    Returns (q8, k8, v8, (q_descale, k_descale, v_descale)).
    """
    rng = np.random.default_rng(seed)
    q = (std * rng.standard_normal((B, H, Nq, D), dtype=np.float32)).astype(np.float32)
    k = (std * rng.standard_normal((B, H, Nk, D), dtype=np.float32)).astype(np.float32)
    v = rng.standard_normal((B, H, Nk, D), dtype=np.float32)
    (q8, qd), (k8, kd), (v8, vd) = (quantize_e4m3(t) for t in (q, k, v))
    return q8, k8, v8, (qd, kd, vd)


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str            # "bf16" or "fp32"
    B: int
    H: int
    Nq: int
    Nk: int
    D: int
    causal: bool
    scale: float
    seed: int
    padded: bool = False  # kv_lens drawn as described above
    drift: float = 0.0    # key drift coefficient (0: none)

    def metric_flops(self) -> float:
        """4*B*H*Nq*Nk*D, halved when causal (the attention-throughput convention)."""
        f = 4.0 * self.B * self.H * self.Nq * self.Nk * self.D
        return f / 2.0 if self.causal else f


# The five workloads, smallest first.  The fourth is the throughput headline.
WORKLOADS = {
    "fp32_b1h1_n128_d64": Workload("fp32_b1h1_n128_d64", "fp32", 1, 1, 128, 128, 64,
                                   False, 1.0 / 8.0, 1),
    "bf16_causal_b4h8_n1024_d64": Workload("bf16_causal_b4h8_n1024_d64", "bf16", 4, 8, 1024,
                                           1024, 64, True, 1.0 / 8.0, 2),
    "bf16_padded_b8h16_n2048_d128": Workload("bf16_padded_b8h16_n2048_d128", "bf16", 8, 16,
                                             2048, 2048, 128, False, 1.0 / math.sqrt(128), 3,
                                             padded=True),
    "bf16_causal_b1h32_n8192_d128": Workload("bf16_causal_b1h32_n8192_d128", "bf16", 1, 32,
                                             8192, 8192, 128, True, 1.0 / math.sqrt(128), 4),
    "bf16_causal_drift_b1h8_n32768_d128": Workload("bf16_causal_drift_b1h8_n32768_d128", "bf16",
                                                   1, 8, 32768, 32768, 128, True,
                                                   1.0 / math.sqrt(128), 5, drift=0.002),
}
WORKLOAD_ORDER = list(WORKLOADS)
HEADLINE = "bf16_causal_b1h32_n8192_d128"


def generate(w: Workload, heads: Optional[int] = None):
    """Draw (q, k, v, kv_lens) as float32 numpy arrays [B,H,N,D] (kv_lens int32 or None).

    ``heads`` keeps only the first ``heads`` heads of the draw (the draw itself is
    unchanged, so the kept heads equal those of the full workload).
    """
    rng = np.random.default_rng(w.seed)
    u = None
    if w.drift:
        g = rng.standard_normal(w.D, dtype=np.float32)
        u = (g / np.float32(np.linalg.norm(g.astype(np.float64)))).astype(np.float32)
    q = rng.standard_normal((w.B, w.H, w.Nq, w.D), dtype=np.float32)
    k = rng.standard_normal((w.B, w.H, w.Nk, w.D), dtype=np.float32)
    v = rng.standard_normal((w.B, w.H, w.Nk, w.D), dtype=np.float32)
    kv_lens = None
    if w.padded:
        kv_lens = rng.integers(1, w.Nk + 1, size=w.B).astype(np.int32)
        kv_lens[0] = 0
    if u is not None:
        j = np.arange(w.Nk, dtype=np.float32)[:, None]
        k = (k + np.float32(w.drift) * j * u[None, :]).astype(np.float32)
    if heads is not None:
        q, k, v = q[:, :heads], k[:, :heads], v[:, :heads]
    if w.dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return (np.ascontiguousarray(q), np.ascontiguousarray(k), np.ascontiguousarray(v),
            kv_lens)


def random_case(seed: int, B: int, H: int, Nq: int, Nk: int, D: int, dtype: str = "bf16",
                kv_lens=None, std: float = 1.0):
    """A small seeded case with the same value distribution (N(0, std^2), bf16-rounded)."""
    rng = np.random.default_rng(seed)
    q = (std * rng.standard_normal((B, H, Nq, D), dtype=np.float32)).astype(np.float32)
    k = (std * rng.standard_normal((B, H, Nk, D), dtype=np.float32)).astype(np.float32)
    v = rng.standard_normal((B, H, Nk, D), dtype=np.float32)
    if dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    if kv_lens is not None:
        kv_lens = np.asarray(kv_lens, dtype=np.int32)
    return q, k, v, kv_lens


def generate_fp8(w: Workload, heads: Optional[int] = None):
    """The draws of ``generate`` quantised per tensor to E4M3 instead of rounded to bf16.

    Returns (q8, k8, v8, (q_descale, k_descale, v_descale), kv_lens).
    """
    rng = np.random.default_rng(w.seed)
    if w.drift:
        rng.standard_normal(w.D, dtype=np.float32)   # keep the draw order of generate
    q = rng.standard_normal((w.B, w.H, w.Nq, w.D), dtype=np.float32)
    k = rng.standard_normal((w.B, w.H, w.Nk, w.D), dtype=np.float32)
    v = rng.standard_normal((w.B, w.H, w.Nk, w.D), dtype=np.float32)
    kv_lens = None
    if w.padded:
        kv_lens = rng.integers(1, w.Nk + 1, size=w.B).astype(np.int32)
        kv_lens[0] = 0
    if w.drift:
        raise ValueError("the drifting-key workload has no FP8 variant")
    if heads is not None:
        q, k, v = q[:, :heads], k[:, :heads], v[:, :heads]
    (q8, qd), (k8, kd), (v8, vd) = (quantize_e4m3(t) for t in (q, k, v))
    return q8, k8, v8, (qd, kd, vd), kv_lens
