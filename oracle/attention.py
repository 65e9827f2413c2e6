"""Oracle for causal softmax attention: the naive plan, in float64, on the CPU.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares
no code with the GPU library and never imports it.

What it computes follows "Show HN: automatic deduction of FlashAttention kernel
from 25 lines of SQL" (neshdevtech.com), the view ``attention`` in its two SQL
spellings (``ATTENTION_WINDOW`` and ``ATTENTION_GROUP_BY``), the loss of the
``GRADIENT`` statement and the JAX ``attention()``/``loss()`` functions:

* scores   s_ij = (sum_d q_id k_jd) / 8   for every pair with i >= j (the join
  predicate ``q.t >= k.t``; pairs with j > i do not exist);
* m_i      = max_j s_ij over the pairs that exist (a window, or a GROUP BY);
* w_ij     = exp(s_ij - m_i);   z_i = sum_j w_ij;
* o_id     = sum_j (w_ij / z_i) v_jd, summed over existing pairs only, so an
  absent pair never contributes 0 * v (an infinity in V reaches only rows
  i >= j);
* loss     = sum(o^2) / 2, so the upstream gradient is dO = O;
* lse_i    = m_i + ln z_i (natural log of the scaled scores).  The pages do not
  name this quantity; it is the per-row value a streamed backward needs.

Masks.  The join predicate decides which pairs exist; the page's central claim
is that the same fused plan follows for any softmax-weighted average over a
join.  ``mask`` selects the predicate (every function defaults to the page's
causal one):

* ``"causal"``: q.t >= k.t, the view ``attention``;
* ``"full"``:   no predicate, every pair exists (the plain join, as in the
  attention query on the Show HN post's shorter page, which has no WHERE);
* ``"window"``: q.t >= k.t AND q.t - k.t < window, a causal band of ``window``
  keys per query (window >= 1).

``seg`` (one integer per token, or None) adds an equality to any of these
join conditions: the pair (i, j) exists only when seg[i] == seg[j], as when
the join also matches a segment column (packed documents that must not see
one another are the usual case).  Ids need not be sorted or contiguous.

The scale is an argument; the pages fix it at 1/8 (= 1/sqrt(64)).  Dividing by
8 and multiplying by 0.125 give the same float64 result, since 0.125 is a power
of two.

The backward pages use ddx and ``jax.grad`` and do not print an algorithm.  The
oracle takes the closed-form chain rule through the same definitions:

* P = w / z,  dV_j = sum_{i>=j} P_ij dO_i,  dP_ij = dO_i . v_j,
* delta_i = sum_j P_ij dP_ij,  dS_ij = P_ij (dP_ij - delta_i),
* dQ_i = scale * sum_{j<=i} dS_ij k_j,  dK_j = scale * sum_{i>=j} dS_ij q_i.

Adding one constant to every score of a row leaves every ratio w / z of that
row unchanged, so the loss does not depend on m_i and the derivative through
it is zero; the oracle treats m_i as a constant (the demo script says as much
beside its window spelling).  With ``route_max=True`` the backward also adds
the term that reaches the argmax pair through m_i, as a mechanical
differentiation of the window would, which must change nothing beyond
rounding.

``forward`` and ``backward`` apply the per-head functions to every (b, h)
head of [B, H, N, D] arrays, optionally on a thread pool over heads (NumPy
releases the interpreter lock inside its kernels).

Rows are processed in blocks of ``block`` queries only to bound memory: every
row's whole score vector is materialised and reduced exactly (two passes: max,
then exp and sum).  No running (online) softmax appears here.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

DEFAULT_SCALE = 0.125


MASKS = ("causal", "full", "window")


def _check_mask(mask: str, window: int) -> None:
    if mask not in MASKS:
        raise ValueError(f"unknown mask {mask!r}")
    if mask == "window" and window < 1:
        raise ValueError("window must be >= 1")


def _present(r0: int, r1: int, ncols: int, mask: str = "causal", window: int = 0,
             seg=None) -> np.ndarray:
    """Boolean (r1-r0, ncols) table of the pairs that exist for queries
    r0 .. r1-1 and keys 0 .. ncols-1 under the mask's join predicate, and,
    with segment ids, only between tokens of one segment."""
    i = np.arange(r0, r1)[:, None]
    j = np.arange(ncols)[None, :]
    if mask == "causal":
        p = j <= i
    elif mask == "full":
        p = np.ones((r1 - r0, ncols), dtype=bool)
    else:
        p = (j <= i) & (i - j < window)
    if seg is not None:
        p = p & (seg[r0:r1, None] == seg[None, :ncols])
    return p


def _check_seg(seg, n: int):
    if seg is None:
        return None
    seg = np.asarray(seg)
    if seg.shape != (n,) or not np.issubdtype(seg.dtype, np.integer):
        raise ValueError("seg must hold one integer per token")
    return seg


def _key_cols(r1: int, n: int, mask: str) -> int:
    """Keys a block of queries ending at r1 can pair with: all n for the full
    mask, keys below r1 otherwise."""
    return n if mask == "full" else r1


def _sum_present(weights: np.ndarray, present: np.ndarray, values: np.ndarray) -> np.ndarray:
    """sum_j weights[i, j] * values[j, :] over the pairs that exist.

    An absent pair contributes nothing (not 0 * v): finite values go through
    one product with absent weights set to 0, and each non-finite value is
    added only to the rows whose pair with it exists.  A present pair whose
    weight underflowed to 0 still multiplies, as the SQL engine would."""
    finite = np.isfinite(values)
    out = np.where(present, weights, 0.0) @ np.where(finite, values, 0.0)
    for j, d in zip(*np.nonzero(~finite)):
        with np.errstate(invalid="ignore"):
            term = weights[:, j] * values[j, d]
        out[:, d] += np.where(present[:, j], term, 0.0)
    return out


def forward_head(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                 scale: float = DEFAULT_SCALE, block: int = 256, mask: str = "causal",
                 window: int = 0, seg=None):
    """Window spelling, matrix form.  q, k, v: (N, D) float64; seg: (N,) ints or None.

    Returns (o, lse, m, z): o (N, D), and per-row lse, max m, denominator z."""
    _check_mask(mask, window)
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    n = q.shape[0]
    seg = _check_seg(seg, n)
    o = np.empty_like(q)
    lse = np.empty(n)
    m_all = np.empty(n)
    z_all = np.empty(n)
    for r0 in range(0, n, block):
        r1 = min(n, r0 + block)
        nc = _key_cols(r1, n, mask)
        present = _present(r0, r1, nc, mask, window, seg)
        s = (q[r0:r1] @ k[:nc].T) * scale                       # s_ij for every (i, j) of the block
        m = np.max(np.where(present, s, -np.inf), axis=1)       # m_i over present pairs only
        with np.errstate(invalid="ignore", over="ignore"):
            w = np.where(present, np.exp(s - m[:, None]), 0.0)  # w_ij, 0 where no pair exists
        z = w.sum(axis=1)                                       # z_i
        o[r0:r1] = _sum_present(w / z[:, None], present, v[:nc])  # o_i = sum_j (w_ij / z_i) v_j
        lse[r0:r1] = m + np.log(z)
        m_all[r0:r1] = m
        z_all[r0:r1] = z
    return o, lse, m_all, z_all


def forward_head_relational(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                            scale: float = DEFAULT_SCALE, spelling: str = "group by",
                            mask: str = "causal", window: int = 0, seg=None):
    """The same attention computed over an explicit list of the pairs that
    exist, the way the demo script's two views (``ATTENTION_WINDOW`` and
    ``ATTENTION_GROUP_BY``) treat their join: one record per pair (i, j), and
    every per-row quantity an aggregate over the records of row i.

    The two spellings differ only in how the row maximum reaches each record:
    ``"group by"`` reduces the records to one maximum per row and looks it up
    again by the record's row; ``"window"`` sorts the records by row and takes
    the maximum inside each row's run.  Records exist only for present pairs,
    so an absent pair is never touched.  Memory is quadratic: small N only.
    Returns (o, lse)."""
    _check_mask(mask, window)
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    n, d = q.shape
    rows, cols = np.nonzero(_present(0, n, n, mask, window, _check_seg(seg, n)))  # pair records
    s = np.einsum("pd,pd->p", q[rows], k[cols]) * scale      # one score per record
    if spelling == "group by":
        best = np.full(n, -np.inf)
        np.maximum.at(best, rows, s)                           # largest score of each row
        m = best[rows]                                         # ... handed back to its records
    elif spelling == "window":
        order = np.lexsort((cols, rows))                       # records grouped by row
        starts = np.searchsorted(rows[order], np.arange(n + 1))
        m = np.empty_like(s)
        for i in range(n):
            run = order[starts[i]:starts[i + 1]]
            m[run] = s[run].max()
    else:
        raise ValueError(spelling)
    w = np.exp(s - m)                                          # record weights
    z = np.zeros(n)
    np.add.at(z, rows, w)                                      # z_i: sum of row i's weights
    o = np.zeros((n, d))
    np.add.at(o, rows, (w / z[rows])[:, None] * v[cols])       # o_i: weighted sum of its values
    best = np.full(n, -np.inf)
    np.maximum.at(best, rows, s)
    return o, best + np.log(z)


def loss(o: np.ndarray) -> float:
    """Half the sum of the squares of every output value (the loss of the
    demo script's gradient statement and of its JAX ``loss()``), so that the
    loss's gradient with respect to o is o itself."""
    o = np.asarray(o, dtype=np.float64)
    return float(np.sum(o * o) / 2)


def backward_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray | None = None,
                  scale: float = DEFAULT_SCALE, block: int = 256, route_max: bool = False,
                  mask: str = "causal", window: int = 0, seg=None):
    """Gradients (dq, dk, dv) of sum_{i,d} dout_id * o_id; with dout = o (the
    default) that is the gradient of loss = sum(o^2) / 2.  Closed-form chain
    rule over the naive plan, recomputing each block's full score rows."""
    _check_mask(mask, window)
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    n = q.shape[0]
    seg = _check_seg(seg, n)
    if dout is None:
        dout = forward_head(q, k, v, scale, block, mask, window, seg)[0]
    dout = np.asarray(dout, dtype=np.float64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, n, block):
        r1 = min(n, r0 + block)
        nc = _key_cols(r1, n, mask)
        present = _present(r0, r1, nc, mask, window, seg)
        s = (q[r0:r1] @ k[:nc].T) * scale
        masked = np.where(present, s, -np.inf)
        m = masked.max(axis=1)
        with np.errstate(invalid="ignore", over="ignore"):
            w = np.where(present, np.exp(s - m[:, None]), 0.0)
        z = w.sum(axis=1)
        p = w / z[:, None]
        dp = np.where(present, dout[r0:r1] @ v[:nc].T, 0.0)      # dL/dP_ij = dO_i . v_j
        delta = np.sum(p * dp, axis=1)
        ds = p * (dp - delta[:, None])                           # dL/ds_ij through w_ij
        if route_max:
            # m_i is itself max_j s_ij: dL/dm_i = -sum_j dS_ij goes to the argmax pair.
            arg = np.argmax(masked, axis=1)
            ds[np.arange(r1 - r0), arg] += -ds.sum(axis=1)
        dq[r0:r1] = (ds @ k[:nc]) * scale
        dk[:nc] += (ds.T @ q[r0:r1]) * scale
        dv[:nc] += p.T @ dout[r0:r1]
    return dq, dk, dv


def _map_heads(fn, arrays, workers):
    """fn(per-head arrays..., batch index) over every (b, h) head."""
    b, h = arrays[0].shape[:2]
    jobs = [(bi, hi) for bi in range(b) for hi in range(h)]
    if workers is None or workers <= 1:
        return jobs, [fn(*(a[bi, hi] for a in arrays), bi) for bi, hi in jobs]
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return jobs, list(ex.map(lambda j: fn(*(a[j[0], j[1]] for a in arrays), j[0]), jobs))


def _seg_of(seg, b):
    return None if seg is None else np.asarray(seg)[b]


def forward(q, k, v, scale: float = DEFAULT_SCALE, workers: int | None = None, block: int = 256,
            mask: str = "causal", window: int = 0, seg=None):
    """[B, H, N, D] float64 -> (o [B, H, N, D], lse [B, H, N]); heads are
    independent; seg, if given, is [B, N] (every head of a batch shares it)."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    o = np.empty_like(q)
    lse = np.empty(q.shape[:3])
    jobs, res = _map_heads(lambda a, b_, c, bi: forward_head(a, b_, c, scale, block, mask, window,
                                                              _seg_of(seg, bi)),
                           (q, k, v), workers)
    for (bi, hi), (oh, lh, _, _) in zip(jobs, res):
        o[bi, hi] = oh
        lse[bi, hi] = lh
    return o, lse


def backward(q, k, v, dout=None, scale: float = DEFAULT_SCALE, workers: int | None = None,
             block: int = 256, mask: str = "causal", window: int = 0, seg=None):
    """[B, H, N, D] float64 -> (dq, dk, dv); dout defaults to the oracle's own o."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    if dout is None:
        arrays = (q, k, v)
        fn = lambda a, b_, c, bi: backward_head(a, b_, c, None, scale, block, mask=mask,
                                                window=window, seg=_seg_of(seg, bi))
    else:
        arrays = (q, k, v, np.asarray(dout, dtype=np.float64))
        fn = lambda a, b_, c, d_, bi: backward_head(a, b_, c, d_, scale, block, mask=mask,
                                                    window=window, seg=_seg_of(seg, bi))
    out = [np.empty_like(q) for _ in range(3)]
    jobs, res = _map_heads(fn, arrays, workers)
    for (bi, hi), grads in zip(jobs, res):
        for dst, g in zip(out, grads):
            dst[bi, hi] = g
    return tuple(out)
