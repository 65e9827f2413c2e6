"""Oracle for the Q / K / V input projections: float64 NumPy, CPU.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares
no code with the GPU library and never imports it.

What it computes follows the "Wiki notes" page (brainpick-2k7.pages.dev), its
MLIR functions ``@attention_head`` and ``@mini_attention``: from the token
embeddings x (seq x d_model) and three weight matrices (d_model x d_k), the
queries, keys and values are the products Q = x Wq, K = x Wk, V = x Wv (one
``linalg.matmul`` each), and the attention then works on Q, K, V.

Readings where the pages are silent (the listing is one head, no batch):

* several heads: the weight matrices are d_model x (H d_k) and head h takes
  columns h d_k .. h d_k + d_k - 1 of each product (the usual packing of
  per-head weights side by side);
* batch: x is B x N x d_model and every batch entry is projected with the
  same weights;
* the result is laid out as the attention takes it, [B, H, N, d_k];
* no bias and no scale: the listing has neither.

Each product is one float64 matmul (a library primitive), then a reshape.
Parity pins live in ``tests/test_oracle_projection.py``.
"""
from __future__ import annotations

import numpy as np


def project(x: np.ndarray, w: np.ndarray, heads: int) -> np.ndarray:
    """x [B, N, Dm] times w [Dm, heads * dk] -> [B, heads, N, dk] in float64."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if x.ndim != 3 or w.ndim != 2 or w.shape[0] != x.shape[2] or w.shape[1] % heads:
        raise ValueError("shapes: x [B, N, Dm], w [Dm, heads * dk]")
    B, N, _ = x.shape
    dk = w.shape[1] // heads
    y = x @ w                                   # [B, N, heads * dk]
    return y.reshape(B, N, heads, dk).transpose(0, 2, 1, 3).copy()


def project_qkv(x, wq, wk, wv, heads: int):
    """(Q, K, V), each [B, heads, N, dk], from one embedding x."""
    return project(x, wq, heads), project(x, wk, heads), project(x, wv, heads)
