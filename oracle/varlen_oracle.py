"""Plain fp64 CPU oracle for attention over a packed batch of variable-length sequences.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The product
path never does, and shares no code with it: this file imports numpy and the
definition oracle of this package, nothing else.

What it computes
----------------
The page "Fused Multi-Head Attention" (section on how fused attention combines with
other inference techniques, the continuous-batching item) names the ragged tensors
that batching sequences of different lengths creates.  Packed, the B sequences are
concatenated along the token axis: q [total_q, H, D], k and v [total_k, H, D]; the
cumulative offsets cu_q, cu_k (B + 1 entries) say that sequence b owns query tokens
[cu_q[b], cu_q[b+1]) and key tokens [cu_k[b], cu_k[b+1]).  Each sequence is an
independent attention problem: its queries see only its own keys (causal masking,
when asked, is top-left within the sequence).  So

    O[cu_q[b] + i, h] = attention(q_b[h], k_b[h], v_b[h])[i]
    LSE[h, cu_q[b] + i] likewise,

evaluated by ``attn_oracle.attention_oracle`` on every sequence sliced out of the
pack.  Query tokens that no sequence owns are left as NaN (nothing is defined there).

Readings (listed in the design notes as well): the offsets are clamped the way the
kernel clamps them -- each entry into [0, total], an end below its start to the start,
a length above max_seqlen to max_seqlen -- so that inconsistent offsets still have
one defined meaning; LSE is laid out [H, total_q].
"""

from __future__ import annotations

import numpy as np

from .attn_oracle import attention_oracle

__all__ = ["seq_spans", "attention_varlen_oracle"]


def seq_spans(cu, total: int, max_len: int):
    """[(start, length)] of every sequence after clamping (see the module docstring)."""
    cu = [int(x) for x in np.asarray(cu).reshape(-1)]
    spans = []
    for b in range(len(cu) - 1):
        s = min(max(cu[b], 0), total)
        e = min(max(cu[b + 1], s), total)
        spans.append((s, min(e - s, max_len)))
    return spans


def attention_varlen_oracle(q, k, v, cu_q, cu_k, scale: float, causal: bool = False,
                            max_seqlen_q=None, max_seqlen_k=None):
    """Exact attention of every packed sequence, in fp64.

    q [total_q, H, D], k [total_k, H, D], v [total_k, H, Dv] (any real dtype); cu_q,
    cu_k: B + 1 integers.  Returns O [total_q, H, Dv] and LSE [H, total_q] (NaN on
    query tokens no sequence owns).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    total_q, H, _ = q.shape
    total_k = k.shape[0]
    mq = total_q if max_seqlen_q is None else int(max_seqlen_q)
    mk = total_k if max_seqlen_k is None else int(max_seqlen_k)
    sq, sk = seq_spans(cu_q, total_q, mq), seq_spans(cu_k, total_k, mk)
    assert len(sq) == len(sk), "cu_q and cu_k must describe the same number of sequences"
    o = np.full((total_q, H, v.shape[2]), np.nan)
    lse = np.full((H, total_q), np.nan)
    for (qs, nq), (ks, nk) in zip(sq, sk):
        if nq == 0:
            continue
        qb = q[qs:qs + nq].transpose(1, 0, 2)[None]           # [1, H, nq, D]
        if nk == 0:
            o[qs:qs + nq] = 0.0
            lse[:, qs:qs + nq] = -np.inf
            continue
        kb = k[ks:ks + nk].transpose(1, 0, 2)[None]
        vb = v[ks:ks + nk].transpose(1, 0, 2)[None]
        ob, lb = attention_oracle(qb, kb, vb, scale, causal=causal)
        o[qs:qs + nq] = ob[0].transpose(1, 0, 2)
        lse[:, qs:qs + nq] = lb[0]
    return o, lse
