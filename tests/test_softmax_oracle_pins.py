"""Pins of the row-softmax oracle to facts that do not come from the oracle itself.

Sources: the definition of the stable softmax (page "Kernel Fusion and the Memory
Wall", section "Softmax needs a global row statistic"), closed forms, invariants,
brute force on tiny rows, and torch's softmax in float64 on rows that have at least
one finite entry.  ``PINS`` take a softmax implementation as an argument so that
``test_planted_mistakes_are_caught`` can show every planted mistake fails one.
No test here touches a GPU.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

import oracle.softmax_oracle as SO

NEG_INF = -np.inf


def _brute(row):
    """Textbook definition, no max subtraction, Python floats (math.exp / fsum)."""
    finite = [v for v in row if v != NEG_INF]
    if not finite:
        return [0.0] * len(row)
    e = [math.exp(v) if v != NEG_INF else 0.0 for v in row]
    s = math.fsum(e)
    return [x / s for x in e]


def pin_brute_force(fn):
    rng = np.random.default_rng(3)
    for cols in (1, 2, 3, 7, 16, 33):
        x = rng.standard_normal((4, cols)) * 3.0
        if cols > 2:
            x[1, rng.integers(0, cols, size=cols // 2)] = NEG_INF
        x[3, :] = NEG_INF if cols == 1 else x[3, :]
        y = fn(x)
        for r in range(x.shape[0]):
            np.testing.assert_allclose(y[r], _brute(list(x[r])), rtol=1e-13, atol=1e-300)


def pin_two_entry_closed_form(fn):
    # scores differing by g: weights 1/(1+e^g) and e^g/(1+e^g); g = ln 3 gives 1/4, 3/4.
    # Far from 0 (+-1000) the max subtraction is what keeps exp finite; there the gap
    # actually stored is (base + ln 3) - base, exact in fp64.
    for base in (0.0, 1000.0, -1000.0):
        hi = base + math.log(3.0)
        g = hi - base
        y = fn(np.array([[base, hi]]))
        np.testing.assert_allclose(y, [[1 / (1 + math.exp(g)), math.exp(g) / (1 + math.exp(g))]],
                                   rtol=1e-14)
        if base == 0.0:
            np.testing.assert_allclose(y, [[0.25, 0.75]], rtol=1e-14)


def pin_special_rows(fn):
    x = np.array([[5.0, NEG_INF, NEG_INF],        # one valid entry: one-hot
                  [NEG_INF, NEG_INF, NEG_INF],    # no valid entry: zeros by convention
                  [2.0, 2.0, 2.0]])               # equal entries: uniform
    y = fn(x)
    np.testing.assert_array_equal(y[0], [1.0, 0.0, 0.0])
    np.testing.assert_array_equal(y[1], [0.0, 0.0, 0.0])
    np.testing.assert_allclose(y[2], [1 / 3] * 3, rtol=1e-15)
    assert not np.isnan(y).any()


def pin_distribution_and_shift(fn):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 50)) * 4.0
    y = fn(x)
    np.testing.assert_allclose(y.sum(axis=1), 1.0, rtol=1e-14)
    assert (y >= 0).all() and (y <= 1).all()
    np.testing.assert_allclose(fn(x + 37.5), y, rtol=1e-12, atol=1e-300)
    perm = rng.permutation(50)
    np.testing.assert_allclose(fn(x[:, perm]), y[:, perm], rtol=1e-14, atol=1e-300)


PINS = [pin_brute_force, pin_two_entry_closed_form, pin_special_rows,
        pin_distribution_and_shift]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_softmax_oracle_pin(pin):
    pin(SO.softmax_rows)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_four_pass_oracle_pin(pin):
    pin(SO.softmax_rows_four_pass)


def test_four_pass_equals_definition():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((5, 300)) * 5.0
    x[2, ::3] = NEG_INF
    x[4, :] = NEG_INF
    np.testing.assert_allclose(SO.softmax_rows_four_pass(x), SO.softmax_rows(x), rtol=1e-14,
                               atol=1e-300)


def test_torch_softmax_special_case():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    x = rng.standard_normal((8, 129)) * 6.0
    x[3, 10:] = NEG_INF
    ref = torch.softmax(torch.from_numpy(x), dim=-1).numpy()
    np.testing.assert_allclose(SO.softmax_rows(x), ref, rtol=1e-13, atol=1e-300)


def test_higher_rank_rows():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((2, 3, 17))
    y = SO.softmax_rows(x)
    np.testing.assert_allclose(y.reshape(6, 17), SO.softmax_rows(x.reshape(6, 17)))


# ---------------------------------------------------------------------------
# planted mistakes: each deliberately wrong copy must fail at least one pin
# ---------------------------------------------------------------------------

def _no_max_subtraction(x):
    x = np.asarray(x, np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(x)
        y = e / e.sum(-1, keepdims=True)
    return np.nan_to_num(y, nan=0.0)


def _no_empty_guard(x):
    x = np.asarray(x, np.float64)
    m = x.max(-1, keepdims=True)
    with np.errstate(invalid="ignore"):
        e = np.exp(x - m)
        return e / e.sum(-1, keepdims=True)


def _wrong_axis(x):
    x = np.asarray(x, np.float64)
    m = x.max(0, keepdims=True)
    m = np.where(np.isneginf(m), 0.0, m)
    e = np.exp(x - m)
    s = e.sum(0, keepdims=True)
    return np.where(s > 0, e / np.where(s > 0, s, 1.0), 0.0)


def _missing_division(x):
    x = np.asarray(x, np.float64)
    m = x.max(-1, keepdims=True)
    m = np.where(np.isneginf(m), 0.0, m)
    return np.exp(x - m)


def _sum_over_tile_only(x):
    """Normalises each block of 16 entries by its own sum (the mistake the page names)."""
    x = np.asarray(x, np.float64)
    out = np.empty_like(x)
    for c0 in range(0, x.shape[-1], 16):
        out[..., c0:c0 + 16] = SO.softmax_rows(x[..., c0:c0 + 16])
    return out


MUTANTS = [_no_max_subtraction, _no_empty_guard, _wrong_axis, _missing_division,
           _sum_over_tile_only]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_planted_mistakes_are_caught(mutant):
    failed = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mutant)
        except AssertionError:
            failed += 1
    assert failed >= 1, f"no pin catches {mutant.__name__}"
