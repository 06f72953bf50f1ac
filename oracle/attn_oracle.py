"""Plain fp64 CPU oracle for exact (non-approximated) attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The product
path (the HIP library and its Python binding) never does, and shares no code with
it: this file imports numpy and nothing else.

What it computes
----------------
For every batch b, head h and query row i

    s_ij  = sigma * <q_i, k_j>                          (scaled scores)
    s_ij  = -inf   where key j is not valid for row i   (additive mask)
    O_i   = sum_j softmax(s_i)_j * v_j
    LSE_i = log sum_j exp(s_ij)                         (natural log)

with softmax taken in its numerically stable form, i.e. after subtracting the
row maximum (page "Kernel Fusion and the Memory Wall", section "Softmax needs a
global row statistic": the denominator covers the whole row).  The attention
function itself is the one in section "FlashAttention: avoid the full score
matrix" of the same page (softmax(Q K^T / sqrt(d)) V; the scale is an argument
here).  A key is valid for query i when j < kv_len[b] and, if causal, j <= i
(the causal mask and the rows without valid keys are named in section "A small
executable reference"; the page "Attention softmax fusion", section "Things
that break", names the fully masked case).  A row with no valid key returns
O_i = 0 and LSE_i = -inf: this is a convention, not a consequence of the
mathematics, because softmax over an empty set is undefined.

Two functions compute this:

* ``attention_oracle`` is the plain definition: it materialises the whole score
  row, masks it, and applies the stable softmax and the value contraction.
* ``attention_online_oracle`` follows the online recurrence that the pages give
  (page "Attention softmax fusion", section "The tile loop"; page "Kernel
  Fusion and the Memory Wall", sections "FlashAttention: avoid the full score
  matrix" and "A small executable reference"): keys are visited tile by tile,
  a running maximum m, normaliser l and unnormalised numerator a are kept, and
  on every tile the old accumulators are multiplied by exp(m - m').  After the
  last tile the result is a / l.  It exists so that tests can show the
  recurrence reaches the same result as the definition.

Readings where the pages are silent (each one is listed in the design notes):

* The pages never define LSE.  It is the natural-log log-sum-exp of the scaled,
  masked scores: LSE_i = m_i + ln(l_i).
* The scale is applied after rounding it to fp32 (``sigma = fp64(fp32(scale))``)
  because the GPU receives a C ``float``.
* kv_len values are clamped into [0, Nk]; ``None`` means every key is valid.
* Causal masking is top-left aligned: key j is visible to query i iff j <= i,
  also when Nq != Nk.
* Causal and kv_len masks combine by logical AND.
* In the online recurrence, when every score seen so far is -inf the running
  maximum is -inf and exp(m - m') would be exp(-inf + inf) = NaN.  Both
  exponent references are taken as 0 in that case (the guard the page
  "Attention softmax fusion" asks for in "Things that break").

Every input is upcast to float64 before any arithmetic.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "effective_scale",
    "kv_length",
    "valid_keys",
    "attention_oracle",
    "attention_online_oracle",
    "attention_rows",
    "attention_oracle_rows",
]


def effective_scale(scale: float) -> float:
    """The score scale as the kernel sees it: rounded to fp32, then widened."""
    return float(np.float32(scale))


def kv_length(kv_lens, b: int, nk: int) -> int:
    """Number of valid keys of sequence b, clamped into [0, nk]."""
    if kv_lens is None:
        return nk
    n = int(np.asarray(kv_lens).reshape(-1)[b])
    return min(max(n, 0), nk)


def valid_keys(row_lo: int, row_hi: int, nk: int, causal: bool, kv_len: int) -> np.ndarray:
    """Boolean [row_hi-row_lo, nk] mask: True where key j may be attended by query i.

    Valid iff j < kv_len and (not causal or j <= i); see the module docstring.
    """
    i = np.arange(row_lo, row_hi)[:, None]
    j = np.arange(nk)[None, :]
    valid = np.broadcast_to(j < kv_len, (row_hi - row_lo, nk))
    if causal:
        valid = valid & (j <= i)
    return np.array(valid)


def attention_rows(q_rows, k, v, sigma: float, valid: np.ndarray, return_probs: bool = False):
    """Attention of a block of query rows against one head's keys and values.

    q_rows [r, D], k [Nk, D], v [Nk, Dv] in float64; ``valid`` [r, Nk] bool.
    Returns (O [r, Dv], LSE [r]) and, if asked, the probability rows P [r, Nk].

    Steps, in the order of the definition:
      1. s = sigma * q k^T
      2. s = -inf where the key is not valid
      3. m = row max of s; rows whose max is -inf have no valid key
      4. e = exp(s - m), l = row sum of e, P = e / l
      5. O = P v, LSE = m + ln l
    """
    s = sigma * (q_rows @ k.T)                              # step 1
    s = np.where(valid, s, -np.inf)                         # step 2
    m = s.max(axis=1) if s.shape[1] > 0 else np.full(s.shape[0], -np.inf)  # step 3
    has_key = m > -np.inf
    m_ref = np.where(has_key, m, 0.0)
    e = np.exp(s - m_ref[:, None])                          # step 4 (exp(-inf) = 0)
    l = e.sum(axis=1)
    p = np.zeros_like(e)
    p[has_key] = e[has_key] / l[has_key, None]
    o = p @ v                                               # step 5
    lse = np.full(s.shape[0], -np.inf)
    lse[has_key] = m[has_key] + np.log(l[has_key])
    o[~has_key] = 0.0
    if return_probs:
        return o, lse, p
    return o, lse


def attention_oracle(q, k, v, scale: float, causal: bool = False, kv_lens=None,
                     row_chunk: int = 1024, return_probs: bool = False):
    """Exact attention by its definition, materialised, in float64.

    q [B,H,Nq,D], k [B,H,Nk,D], v [B,H,Nk,Dv] (any real dtype; upcast to fp64),
    kv_lens [B] integers or None.  Returns O [B,H,Nq,Dv] fp64 and LSE [B,H,Nq]
    fp64 (and P [B,H,Nq,Nk] if ``return_probs``; keep such calls small).

    Query rows are processed in chunks of ``row_chunk``; softmax is row-local,
    so chunking changes no value.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    Dv = v.shape[3]
    assert k.shape == (B, H, Nk, D) and v.shape[:3] == (B, H, Nk)
    sigma = effective_scale(scale)
    o = np.zeros((B, H, Nq, Dv))
    lse = np.full((B, H, Nq), -np.inf)
    probs = np.zeros((B, H, Nq, Nk)) if return_probs else None
    for b in range(B):
        L = kv_length(kv_lens, b, Nk)
        for h in range(H):
            for r0 in range(0, Nq, row_chunk):
                r1 = min(Nq, r0 + row_chunk)
                valid = valid_keys(r0, r1, Nk, causal, L)
                res = attention_rows(q[b, h, r0:r1], k[b, h], v[b, h], sigma, valid,
                                     return_probs=return_probs)
                o[b, h, r0:r1] = res[0]
                lse[b, h, r0:r1] = res[1]
                if return_probs:
                    probs[b, h, r0:r1] = res[2]
    if return_probs:
        return o, lse, probs
    return o, lse


def attention_online_oracle(q, k, v, scale: float, causal: bool = False, kv_lens=None,
                            tile: int = 64):
    """The online (tile-by-tile) recurrence, in float64, one query row at a time.

    For each query row, keys are visited in tiles of ``tile``.  With the running
    maximum m, normaliser l and numerator a of the keys seen so far, and the
    scores s_t of the next tile:

        m'   = max(m, max s_t)
        c    = exp(m - m')            (the correction of the old accumulators)
        l    = c * l + sum exp(s_t - m')
        a    = c * a + exp(s_t - m') @ v_t
        m    = m'

    and after the last tile O = a / l, LSE = m + ln l.  Masked scores are -inf.
    While every score seen is -inf, m and m' are -inf; the exponent references
    are then taken as 0 (the guard), so c = exp(-inf) = 0 and no NaN appears.
    A row whose l is 0 at the end has no valid key: O = 0, LSE = -inf.

    Slow (pure-Python loop over rows): for small shapes only.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    Dv = v.shape[3]
    sigma = effective_scale(scale)
    o = np.zeros((B, H, Nq, Dv))
    lse = np.full((B, H, Nq), -np.inf)
    for b in range(B):
        L = kv_length(kv_lens, b, Nk)
        for h in range(H):
            valid_all = valid_keys(0, Nq, Nk, causal, L)
            for i in range(Nq):
                scores = sigma * (k[b, h] @ q[b, h, i])
                scores = np.where(valid_all[i], scores, -np.inf)
                maximum = -np.inf
                normalizer = 0.0
                numerator = np.zeros(Dv)
                for start in range(0, Nk, tile):
                    s_t = scores[start:start + tile]
                    new_maximum = max(maximum, float(s_t.max()))
                    ref_new = 0.0 if new_maximum == -np.inf else new_maximum
                    ref_old = 0.0 if maximum == -np.inf else maximum
                    correction = math.exp(ref_old - ref_new) if maximum > -np.inf else 0.0
                    tile_exp = np.exp(s_t - ref_new)
                    normalizer = correction * normalizer + tile_exp.sum()
                    numerator = correction * numerator + tile_exp @ v[b, h, start:start + tile]
                    maximum = new_maximum
                if normalizer > 0.0:
                    o[b, h, i] = numerator / normalizer
                    lse[b, h, i] = maximum + math.log(normalizer)
    return o, lse


def attention_oracle_rows(q, k, v, scale: float, causal: bool, kv_lens, samples):
    """The definition evaluated on selected rows only: ``samples`` lists (b, h, i).

    Returns O [n, Dv] and LSE [n] (fp64) for those rows, each computed exactly as
    ``attention_oracle`` computes it, so large problems can be checked row by row.
    """
    Nk = k.shape[2]
    sigma = effective_scale(scale)
    samples = list(samples)
    o = np.zeros((len(samples), v.shape[3]))
    lse = np.full(len(samples), -np.inf)
    for n, (b, h, i) in enumerate(samples):
        L = kv_length(kv_lens, b, Nk)
        valid = valid_keys(i, i + 1, Nk, causal, L)
        res = attention_rows(np.asarray(q[b, h, i:i + 1], dtype=np.float64),
                             np.asarray(k[b, h], dtype=np.float64),
                             np.asarray(v[b, h], dtype=np.float64), sigma, valid)
        o[n] = res[0][0]
        lse[n] = res[1][0]
    return o, lse
