"""Plain fp64 CPU oracle for the row softmax.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` legs of the measurement scripts may import or call this module.
The product path (the HIP library and its Python binding) never does, and shares
no code with it: this file imports numpy and nothing else.

What it computes
----------------
For every row x of a matrix, the numerically stable softmax (page "Kernel Fusion
and the Memory Wall", section "Softmax needs a global row statistic"):

    m   = max_j x_j
    e_j = exp(x_j - m)
    y_j = e_j / sum_k e_k

The denominator covers the whole row, so a row cannot be normalised tile by tile
(same section).  Entries equal to -inf are masked entries: their exponential is
exactly 0.  A row whose entries are all -inf has no valid entry; it returns all
zeros.  This is a convention (softmax over an empty set is undefined), the same
one the attention oracle uses for a query with no valid key.

Two functions compute this:

* ``softmax_rows`` is the plain definition above.
* ``softmax_rows_four_pass`` takes the unfused steps in the page's order: a pass
  over the row for its maximum, a pass that stores the exponentials, a pass that
  sums them, and a pass that divides them by the sum.  It
  exists so tests can show that the step order gives the same function (the HIP
  unfused baseline follows the same four steps).

Every input is upcast to float64 before any arithmetic.
"""

from __future__ import annotations

import numpy as np


def softmax_rows(x: np.ndarray) -> np.ndarray:
    """Stable softmax along the last axis, fp64; all -inf rows give zeros."""
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=-1, keepdims=True)
    empty = np.isneginf(m)                   # every entry masked
    m_use = np.where(empty, 0.0, m)          # keeps exp(-inf - m_use) = 0, never NaN
    e = np.exp(x - m_use)
    s = np.sum(e, axis=-1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        y = np.where(empty, 0.0, e / np.where(empty, 1.0, s))
    return y


def softmax_rows_four_pass(x: np.ndarray) -> np.ndarray:
    """The unfused step order: max, exponentials, sum, normalise (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    for idx in np.ndindex(x.shape[:-1]):
        row = x[idx]
        m = -np.inf
        for v in row:                          # pass 1: read for the maximum
            m = max(m, v)
        m_use = 0.0 if m == -np.inf else m
        e = np.exp(row - m_use)                # pass 2: read, write exponentials
        s = 0.0
        for v in e:                            # pass 3: read exponentials for the sum
            s += v
        out[idx] = e / s if s > 0.0 else 0.0   # pass 4: read again, write output
    return out
