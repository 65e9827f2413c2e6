"""Oracle for the long-table <-> matrix adapter: float64 / integer NumPy, CPU.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares
no code with the GPU library and never imports it.

What it computes follows the demo script of "Show HN: automatic deduction of
FlashAttention kernel from 25 lines of SQL" (neshdevtech.com), its helpers
``table()`` and ``matrix()``: a (t, d) matrix is registered with the SQL
engines as the long table ``(t, d, x)`` whose coordinates are the row and
column positions (``np.arange``), and a ``(t, d, ...)`` query result is turned
back into a (t, d) matrix by pivoting on those two columns.

* ``table(values)``: the rows (t, d, x) of a T x D matrix, one per cell, in
  (t, d) order (the order the forward query asks for with ``ORDER BY t, d``);
* ``matrix(t, d, x, T, D)``: the pivot.  Cell (t, d) of the result holds the x
  of the row with those coordinates.  Readings where the pages are silent:
  a cell no row names is NaN (the pivot of a sparse table fills the holes with
  NaN); two rows naming one cell, or a coordinate outside [0, T) x [0, D),
  is an error (``ValueError``), since a matrix cell has one value.

Parity pins live in ``tests/test_oracle_tables.py``.
"""
from __future__ import annotations

import numpy as np


def table(values: np.ndarray):
    """The long table (t, d, x) of a 2-D array, rows in (t, d) order."""
    values = np.asarray(values)
    if values.ndim != 2:
        raise ValueError("table() takes a (t, d) matrix")
    T, D = values.shape
    t = np.repeat(np.arange(T, dtype=np.int64), D)
    d = np.tile(np.arange(D, dtype=np.int64), T)
    return t, d, values.reshape(-1).copy()


def matrix(t, d, x, T: int, D: int):
    """Pivot rows (t, d, x) into a T x D matrix (NaN where no row names a cell).

    Raises ValueError for a coordinate out of range or a cell named twice."""
    t = np.asarray(t, dtype=np.int64)
    d = np.asarray(d, dtype=np.int64)
    x = np.asarray(x)
    if not (t.shape == d.shape == x.shape) or t.ndim != 1:
        raise ValueError("t, d, x must be 1-D and of one length")
    out = np.full((T, D), np.nan, dtype=x.dtype if x.dtype.kind == "f" else np.float64)
    seen = np.zeros((T, D), dtype=bool)
    for r in range(t.size):
        ti, di = int(t[r]), int(d[r])
        if not (0 <= ti < T and 0 <= di < D):
            raise ValueError(f"row {r}: coordinate ({ti}, {di}) outside {T} x {D}")
        if seen[ti, di]:
            raise ValueError(f"row {r}: cell ({ti}, {di}) named twice")
        seen[ti, di] = True
        out[ti, di] = x[r]
    return out
