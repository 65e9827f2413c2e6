"""The long-table oracle (oracle/tables.py) against pins of its own (CPU only).

Pins, each independent of the oracle's code:
* a hand-written example (a 2 x 3 matrix and its six rows) whose shape is not
  square, so swapping t and d, or T and D, fails it;
* the row order written out by a double loop over (t, d);
* bit-exact round trips, including -0.0, infinities and subnormals;
* the pivot does not depend on the order of the rows (any permutation);
* holes become NaN exactly where no row names a cell;
* a cell named twice, and every kind of out-of-range coordinate, raise.
"""
from __future__ import annotations

import os
import types

import numpy as np
import pytest

from oracle import tables

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def check_hand_example(tables):
    a = np.array([[1.0, 2.0, 3.0], [4.0, 5.0, 6.0]])
    t, d, x = tables.table(a)
    assert t.tolist() == [0, 0, 0, 1, 1, 1]
    assert d.tolist() == [0, 1, 2, 0, 1, 2]
    assert x.tolist() == [1.0, 2.0, 3.0, 4.0, 5.0, 6.0]
    back = tables.matrix([1, 0, 1], [2, 0, 0], [6.0, 1.0, 4.0], 2, 3)
    want = np.array([[1.0, np.nan, np.nan], [4.0, np.nan, 6.0]])
    assert np.array_equal(back, want, equal_nan=True)


def check_row_order_is_t_then_d(tables):
    rng = np.random.default_rng(11)
    a = rng.normal(size=(7, 5))
    t, d, x = tables.table(a)
    rows = [(i, j, a[i, j]) for i in range(7) for j in range(5)]
    assert list(zip(t.tolist(), d.tolist(), x.tolist())) == rows


def check_round_trip_bit_exact(tables):
    for shape in [(1, 1), (3, 64), (64, 64), (256, 64), (5, 7)]:
        rng = np.random.default_rng(sum(shape))
        a = rng.normal(size=shape)
        flat = a.reshape(-1)
        specials = [-0.0, np.inf, -np.inf, 5e-324, -2.2250738585072014e-308]
        flat[: min(len(specials), flat.size)] = specials[: flat.size]
        back = tables.matrix(*tables.table(a), *shape)
        assert back.dtype == a.dtype
        assert np.array_equal(back.view(np.uint64), a.view(np.uint64))


def check_pivot_ignores_row_order(tables):
    rng = np.random.default_rng(12)
    a = rng.normal(size=(9, 6)).astype(np.float32)
    t, d, x = tables.table(a)
    perm = rng.permutation(t.size)
    back = tables.matrix(t[perm], d[perm], x[perm], 9, 6)
    assert back.dtype == np.float32
    assert np.array_equal(back, a)


def check_holes_are_nan(tables):
    rng = np.random.default_rng(13)
    a = rng.normal(size=(4, 3))
    t, d, x = tables.table(a)
    keep = np.ones(t.size, dtype=bool)
    keep[[0, 5, 11]] = False  # cells (0,0), (1,2), (3,2)
    back = tables.matrix(t[keep], d[keep], x[keep], 4, 3)
    holes = np.isnan(back)
    assert sorted(zip(*np.nonzero(holes))) == [(0, 0), (1, 2), (3, 2)]
    assert np.array_equal(back[~holes], a[~holes])


def check_duplicate_cell_raises(tables):
    with pytest.raises(ValueError):
        tables.matrix([0, 1, 0], [1, 1, 1], [1.0, 2.0, 3.0], 2, 2)


def check_out_of_range_raises(tables):
    for t, d in [(-1, 0), (2, 0), (0, -1), (0, 3), (5, 5)]:
        with pytest.raises(ValueError):
            tables.matrix([t], [d], [1.0], 2, 3)


CHECKS = [check_hand_example, check_row_order_is_t_then_d, check_round_trip_bit_exact,
          check_pivot_ignores_row_order, check_holes_are_nan, check_duplicate_cell_raises,
          check_out_of_range_raises]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(tables)


# plausible mistakes planted in a copy of the oracle; each must fail a pin
MUTANTS = {
    "t and d swapped": ("t = np.repeat(np.arange(T, dtype=np.int64), D)",
                        "t = np.tile(np.arange(T, dtype=np.int64), D)"),
    "pivot mirrored": ("out[ti, di] = x[r]", "out[ti, D - 1 - di] = x[r]"),
    "duplicates accepted": ("if seen[ti, di]:", "if False:"),
    "holes zero": ("out = np.full((T, D), np.nan,", "out = np.full((T, D), 0.0,"),
    "last row accepted": ("0 <= ti < T and", "0 <= ti <= T and"),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    src = open(os.path.join(ROOT, "oracle", "tables.py")).read()
    assert old in src
    mod = types.ModuleType("tables_mutant")
    exec(compile(src.replace(old, new, 1), "tables.py", "exec"), mod.__dict__)
    caught = []
    for check in CHECKS:
        try:
            check(mod)
        except (Exception, pytest.fail.Exception) as e:  # noqa: BLE001 - any rejection counts
            caught.append((check.__name__, type(e).__name__))
    assert caught, f"mutant {name!r} passed every pin"
