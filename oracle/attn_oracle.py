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
* ``attention_online_oracle`` is the online recurrence the pages describe (page
  "Attention softmax fusion", section "The tile loop"; page "Kernel Fusion and
  the Memory Wall", sections "FlashAttention: avoid the full score matrix" and
  "A small executable reference"), restated block by block over all rows of a
  head: a running maximum, a running sum of exponentials and a running weighted
  sum of values, with the old sums rescaled by exp(old max - new max) whenever
  the maximum moves, and one division at the end.  It exists so that tests can
  show the recurrence reaches the same result as the definition.

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
    """The online (block-by-block) form of the same function, in float64.

    For each (b, h) the keys are cut into consecutive blocks of ``tile`` and visited in
    order; all query rows of the head advance together.  Per row, three running values
    summarise the keys seen so far:

        top   the largest masked score so far (-inf while none is valid),
        den   the sum of exp(score - ref) over them,
        num   the sum of exp(score - ref) * v_j over them (a row vector),

    where the exponent reference ``ref`` is ``top``, or 0 while ``top`` is -inf (the
    guard: the reference never takes the value -inf, so -inf - (-inf) never occurs).
    A new block raises ``top`` to ``max(top, block row max)``; the sums kept so far
    were taken against the old reference, so both are first multiplied by
    exp(old ref - new ref), the correction the pages apply whenever the maximum moves
    (0 for rows that had no valid key yet, whose sums are empty); then the block's
    weights exp(score - new ref), exactly 0 at masked keys, are added.  After the last
    block, a row with den > 0 gets O = num / den and LSE = top + ln(den); a row with
    den = 0 has no valid key: O = 0, LSE = -inf.

    It exists so that tests can show this recurrence reaches the definition's result
    for every block size.
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
        allowed = valid_keys(0, Nq, Nk, causal, kv_length(kv_lens, b, Nk))
        for h in range(H):
            scores = np.where(allowed, sigma * (q[b, h] @ k[b, h].T), -np.inf)
            top = np.full(Nq, -np.inf)
            den = np.zeros(Nq)
            num = np.zeros((Nq, Dv))
            for lo in range(0, Nk, tile):
                blk = scores[:, lo:lo + tile]
                seen = top > -np.inf
                raised = np.maximum(top, blk.max(axis=1))
                ref_old = np.where(seen, top, 0.0)
                ref_new = np.where(raised > -np.inf, raised, 0.0)
                keep = np.exp(np.where(seen, ref_old - ref_new, -np.inf))
                weights = np.exp(blk - ref_new[:, None])
                den = keep * den + weights.sum(axis=1)
                num = keep[:, None] * num + weights @ v[b, h, lo:lo + tile]
                top = raised
            has_key = den > 0.0
            o[b, h, has_key] = num[has_key] / den[has_key, None]
            lse[b, h, has_key] = top[has_key] + np.log(den[has_key])
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
