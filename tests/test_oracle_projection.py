"""The projection oracle (oracle/projection.py) against pins of its own (CPU only).

Pins, each independent of the oracle's code:
* a triple loop written from the definition q[b, h, n, j] =
  sum_c x[b, n, c] w[c, h dk + j], on integer-valued inputs (exact in float64,
  so equality is exact), including the pages' sizes seq 4, d_model 8, d_k 4;
* identity weights return the embedding split into heads;
* a weight column that belongs to head h moves only head h's output;
* a swap of two heads' weight blocks swaps the heads of the result.
"""
from __future__ import annotations

import os
import types

import numpy as np
import pytest

from oracle import projection

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _loops(x, w, heads):
    B, N, Dm = x.shape
    dk = w.shape[1] // heads
    out = np.zeros((B, heads, N, dk))
    for b in range(B):
        for h in range(heads):
            for n in range(N):
                for j in range(dk):
                    acc = 0.0
                    for c in range(Dm):
                        acc += float(x[b, n, c]) * float(w[c, h * dk + j])
                    out[b, h, n, j] = acc
    return out


def check_against_loops(projection):
    for B, N, Dm, heads, dk in [(1, 4, 8, 1, 4), (2, 3, 5, 2, 3), (1, 5, 64, 1, 64)]:
        rng = np.random.default_rng(B * 100 + N * 10 + Dm)
        x = rng.integers(-8, 9, size=(B, N, Dm)).astype(np.float64)
        ws = [rng.integers(-8, 9, size=(Dm, heads * dk)).astype(np.float64) for _ in range(3)]
        got = projection.project_qkv(x, *ws, heads)
        for g, w in zip(got, ws):
            assert g.shape == (B, heads, N, dk)
            assert np.array_equal(g, _loops(x, w, heads))


def check_identity_weights_split_heads(projection):
    rng = np.random.default_rng(21)
    x = rng.normal(size=(2, 6, 128))
    q = projection.project(x, np.eye(128), 2)
    assert np.array_equal(q[:, 0], x[:, :, :64])
    assert np.array_equal(q[:, 1], x[:, :, 64:])


def check_head_columns_are_separate(projection):
    rng = np.random.default_rng(22)
    x = rng.normal(size=(1, 5, 16))
    w = rng.normal(size=(16, 3 * 4))
    base = projection.project(x, w, 3)
    w2 = w.copy()
    w2[:, 4 + 1] += 1.0   # head 1, column 1
    moved = projection.project(x, w2, 3)
    assert np.array_equal(moved[:, 0], base[:, 0])
    assert np.array_equal(moved[:, 2], base[:, 2])
    assert not np.array_equal(moved[:, 1, :, 1], base[:, 1, :, 1])
    assert np.array_equal(moved[:, 1, :, [0, 2, 3]], base[:, 1, :, [0, 2, 3]])


def check_swapping_head_blocks_swaps_heads(projection):
    rng = np.random.default_rng(23)
    x = rng.normal(size=(2, 4, 10))
    w = rng.normal(size=(10, 2 * 5))
    ws = np.concatenate([w[:, 5:], w[:, :5]], axis=1)
    a, b = projection.project(x, w, 2), projection.project(x, ws, 2)
    assert np.array_equal(a[:, 0], b[:, 1]) and np.array_equal(a[:, 1], b[:, 0])


CHECKS = [check_against_loops, check_identity_weights_split_heads, check_head_columns_are_separate,
          check_swapping_head_blocks_swaps_heads]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(projection)


# plausible mistakes planted in a copy of the oracle; each must fail a pin
MUTANTS = {
    "weight rows reversed": ("y = x @ w ", "y = x @ w[::-1] "),
    "heads interleaved": ("y.reshape(B, N, heads, dk).transpose(0, 2, 1, 3)",
                          "y.reshape(B, N, dk, heads).transpose(0, 3, 1, 2)"),
    "tokens and heads not transposed": (".transpose(0, 2, 1, 3)", ".transpose(0, 1, 2, 3)"),
    "one weight for all three": ("project(x, wk, heads), project(x, wv, heads)",
                                 "project(x, wq, heads), project(x, wq, heads)"),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    src = open(os.path.join(ROOT, "oracle", "projection.py")).read()
    assert old in src
    mod = types.ModuleType("projection_mutant")
    exec(compile(src.replace(old, new, 1), "projection.py", "exec"), mod.__dict__)
    caught = []
    for check in CHECKS:
        try:
            check(mod)
        except (Exception, pytest.fail.Exception) as e:  # noqa: BLE001 - any rejection counts
            caught.append((check.__name__, type(e).__name__))
    assert caught, f"mutant {name!r} passed every pin"
