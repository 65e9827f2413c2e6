"""The parity error metric used by every comparison in the tests.

The pages print no tolerance (their ``assert_close`` helper is not on them), so
the measure is: per output tensor, max |got - want| / max |want| over the
entries where ``want`` is finite (an infinity-norm relative error).  Entries
where ``want`` is not finite must match it exactly in class and sign.
Elementwise relative error is not used: outputs cross zero.
"""
from __future__ import annotations

import numpy as np

TOL = {"f64": 1e-12, "f32": 1e-5, "bf16": 2e-2}


def rel_err(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    fin = np.isfinite(want)
    if not np.array_equal(np.isfinite(got), fin):
        return float("inf")
    nf = ~fin
    if nf.any() and not np.array_equal(got[nf], want[nf], equal_nan=True):
        return float("inf")
    if not fin.any():
        return 0.0
    scale = np.max(np.abs(want[fin]))
    diff = np.max(np.abs(got[fin] - want[fin]))
    if scale == 0.0:
        return float(diff)
    return float(diff / scale)


def assert_close(name: str, got, want, tol: float) -> float:
    e = rel_err(got, want)
    assert e <= tol, f"{name}: relative error {e:.3e} > {tol:.1e}"
    return e
