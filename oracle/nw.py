"""Oracle for the Nadaraya-Watson control, in float64, on the CPU.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares
no code with the GPU library and never imports it.

Follows the ``NADARAYA_WATSON`` query and ``check_nadaraya_watson()`` on "Show
HN: automatic deduction of FlashAttention kernel from 25 lines of SQL"
(neshdevtech.com): every target is paired with every source (CROSS JOIN), the
weight is exp(-((tx - sx)^2 + (ty - sy)^2) / 0.25), and the estimate at a
target is sum(w * v) / sum(w).  The comment there calls the bandwidth h = 0.5;
the divisor it writes is 0.25 = h^2, and that divisor is what is computed.

``shift=True`` (the default) subtracts each target's largest exponent before
exp, which changes nothing in exact arithmetic (it cancels from the ratio) and
keeps a target far from every source from giving 0 / 0.  ``shift=False`` is the
query exactly as written.
"""
from __future__ import annotations

import numpy as np


def nw_average(tx, ty, sx, sy, sv, denom: float = 0.25, shift: bool = True,
               block: int = 512) -> np.ndarray:
    """Per-target Gaussian-weighted average of the source values, float64."""
    tx, ty, sx, sy, sv = (np.asarray(a, dtype=np.float64) for a in (tx, ty, sx, sy, sv))
    out = np.empty(tx.shape[0])
    for r0 in range(0, tx.shape[0], block):
        r1 = min(tx.shape[0], r0 + block)
        e = -((tx[r0:r1, None] - sx[None, :]) ** 2 + (ty[r0:r1, None] - sy[None, :]) ** 2) / denom
        if shift:
            e = e - e.max(axis=1, keepdims=True)
        w = np.exp(e)
        out[r0:r1] = (w @ sv) / w.sum(axis=1)
    return out
