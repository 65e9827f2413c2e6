"""GPU parity for the other join predicates: attn_fwd / attn_bwd with the full
predicate (every pair) and a causal window of w keys, against the float64
oracle under the same predicate.  Error measure and tolerances as in
test_gpu_attention.py (metrics.py): 1e-12 float64, 1e-5 float32, 2e-2 bf16."""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import causal_softmax_attention_amd.inputs as inp  # noqa: E402
import oracle  # noqa: E402
from gpu_util import note, run_bwd, run_fwd, to_dev, to_host  # noqa: E402
from metrics import TOL, assert_close, rel_err  # noqa: E402

S = 0.125
DTYPES = ["f64", "f32", "bf16"]
# window 1: each query sees only itself; 5000 > every N here: the causal mask;
# 400: a key block's walk has interior stages between its diagonal and the
# window's far edge (plain body) as well as edge stages (masked body)
MASKS = [("full", 0), ("window", 1), ("window", 37), ("window", 200), ("window", 400),
         ("window", 5000)]
SHAPES = [(1, 1, 1), (1, 2, 65), (2, 1, 300), (1, 1, 777)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_softmax_attention_amd as csa
    csa.lib()


def _check(a, o, lse, grads, mask, window, sel=None):
    tol = TOL[a.dtype]
    q, k, v = (a.as_f64(x) for x in "qkv")
    B, H = q.shape[:2]
    sel = sel if sel is not None else [(b, h) for b in range(B) for h in range(H)]
    oh, lh = to_host(o), to_host(lse)
    gh = [to_host(g) for g in grads] if grads is not None else None
    for b, h in sel:
        wo, wl = oracle.forward_head(q[b, h], k[b, h], v[b, h], S, mask=mask, window=window)[:2]
        assert_close(f"o[{b},{h}] {mask} {window}", oh[b, h], wo, tol)
        assert_close(f"lse[{b},{h}] {mask} {window}", lh[b, h], wl, tol)
        if gh is None:
            continue
        want = oracle.backward_head(q[b, h], k[b, h], v[b, h], None, S, mask=mask, window=window)
        for name, g, w in zip(("dq", "dk", "dv"), gh, want):
            if window == 1 and name != "dv":
                # one pair per row: P = 1, so dS = dP - delta is exactly 0 and so
                # are dQ and dK (the oracle's too).  The GPU forms delta and dP by
                # different sums; what is left must stay within the tolerance of
                # the cancelled terms, scale |dO_i| |v_i| |q or k|.
                cancelled = S * np.max(np.linalg.norm(oh[b, h], axis=1) *
                                       np.linalg.norm(v[b, h], axis=1))
                other = np.abs(k[b, h] if name == "dq" else q[b, h]).max()
                assert np.abs(g[b, h]).max() <= tol * cancelled * other, name
                assert np.array_equal(w, np.zeros_like(w)), name
                continue
            assert_close(f"{name}[{b},{h}] {mask} {window}", g[b, h], w, tol)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("mask,window", MASKS, ids=lambda x: str(x))
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_mask_fwd_bwd(dtype, mask, window, shape):
    B, H, N = shape
    a = inp.attention_inputs(500 + N + window, B, H, N, dtype)
    note(f"{mask} window={window} {dtype} B={B} H={H} N={N}")
    q, k, v = (to_dev(getattr(a, x), dtype) for x in "qkv")
    o, lse = run_fwd(q, k, v, S, mask=mask, window=window)
    grads = run_bwd(q, k, v, o, o, lse, S, mask=mask, window=window)
    _check(a, o, lse, grads, mask, window)


@pytest.mark.parametrize("dtype", ["f64", "bf16"])
@pytest.mark.parametrize("mask,window", [("full", 0), ("window", 37), ("window", 400)],
                         ids=lambda x: str(x))
def test_mask_peaked_scores(dtype, mask, window):
    """q and k drawn N(0, 36) (scores 36 times the unit workload's): a peaked
    softmax under the other predicates, where a window's first key tile can
    hold a lane's largest score after tiles of smaller ones (the forward's
    reference exponent must then move).  float32 is left out as in
    test_gpu_attention.test_peaked_scores: its own rounding of such scores
    exceeds its tolerance."""
    B, H, N = 1, 2, 777
    a = inp.attention_inputs(600 + window, B, H, N, dtype, qk_mult=6.0)
    note(f"peaked {mask} window={window} {dtype} B={B} H={H} N={N}")
    q, k, v = (to_dev(getattr(a, x), dtype) for x in "qkv")
    o, lse = run_fwd(q, k, v, S, mask=mask, window=window)
    grads = run_bwd(q, k, v, o, o, lse, S, mask=mask, window=window)
    _check(a, o, lse, grads, mask, window)


@pytest.mark.parametrize("dtype", DTYPES)
def test_causal_entry_points_agree(dtype):
    """attn_fwd / attn_bwd with the causal mask are attn_causal_fwd / _bwd, bit for bit."""
    a = inp.attention_inputs(77, 1, 2, 333, dtype)
    note(f"causal entry points {dtype}")
    q, k, v = (to_dev(getattr(a, x), dtype) for x in "qkv")
    o1, l1 = run_fwd(q, k, v, S)
    o2, l2 = run_fwd(q, k, v, S, mask="causal")
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    g1 = run_bwd(q, k, v, o1, o1, l1, S)
    g2 = run_bwd(q, k, v, o1, o1, l1, S, mask="causal")
    assert all(torch.equal(x, y) for x, y in zip(g1, g2))


@pytest.mark.parametrize("dtype", DTYPES)
def test_inf_value_under_masks(dtype):
    """V[150, 5] = +inf reaches, in column 5 only, exactly the rows whose
    predicate admits key 150: rows 150 .. 150 + w - 1 under a window of w, and
    every row under the full predicate."""
    B, H, N, j, w = 1, 1, 400, 150, 37
    a = inp.attention_inputs(41, B, H, N, dtype)
    q, k, v = (to_dev(getattr(a, x), dtype) for x in "qkv")
    v[0, 0, j, 5] = float("inf")
    vh = a.as_f64("v")[0, 0].copy()
    vh[j, 5] = np.inf
    for mask, window, rows in (("window", w, np.arange(j, j + w)), ("full", 0, np.arange(N))):
        note(f"inf in V under {mask} {dtype}")
        o, lse = run_fwd(q, k, v, S, mask=mask, window=window)
        oh = to_host(o)[0, 0]
        hit = np.zeros(N, dtype=bool)
        hit[rows] = True
        assert np.isposinf(oh[hit, 5]).all()
        assert np.isfinite(oh[~hit]).all() and np.isfinite(np.delete(oh, 5, axis=1)).all()
        wo, wl = oracle.forward_head(a.as_f64("q")[0, 0], a.as_f64("k")[0, 0], vh, S,
                                     mask=mask, window=window)[:2]
        assert_close(f"o inf {mask}", oh, wo, TOL[dtype])
        assert_close(f"lse inf {mask}", to_host(lse)[0, 0], wl, TOL[dtype])


@pytest.mark.parametrize("dtype", DTYPES)
def test_equal_scores_under_masks(dtype):
    """Q = 0: o_i is the mean of the V rows the predicate admits and lse_i the
    log of their count; sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i."""
    B, H, N, w = 1, 2, 500, 23
    tol = TOL[dtype]
    a = inp.attention_inputs(42, B, H, N, dtype)
    q, k, v = (to_dev(getattr(a, x), dtype) for x in "qkv")
    vh = a.as_f64("v")
    z = torch.zeros_like(q)
    note(f"Q = 0 under masks {dtype}")
    o, lse = run_fwd(z, k, v, S, mask="full")
    assert rel_err(to_host(o), np.broadcast_to(vh.mean(axis=2, keepdims=True), vh.shape)) <= tol
    assert rel_err(to_host(lse), np.full((B, H, N), np.log(N))) <= tol
    o, lse = run_fwd(z, k, v, S, mask="window", window=w)
    want = np.stack([vh[:, :, max(0, i - w + 1):i + 1].mean(axis=2) for i in range(N)], axis=2)
    assert rel_err(to_host(o), want) <= tol
    assert rel_err(to_host(lse), np.broadcast_to(np.log(np.minimum(np.arange(1, N + 1), w)),
                                                 (B, H, N))) <= tol
    for mask, window in (("full", 0), ("window", w)):
        o, lse = run_fwd(q, k, v, S, mask=mask, window=window)
        dq, dk, dv = run_bwd(q, k, v, o, o, lse, S, mask=mask, window=window)
        dkh, dvh, oh = to_host(dk), to_host(dv), to_host(o)
        assert np.abs(dkh.sum(axis=2)).max() <= tol * N * np.abs(dkh).max()
        assert rel_err(dvh.sum(axis=2), oh.sum(axis=2)) <= tol


@pytest.mark.parametrize("mask,window", [("window", 512), ("full", 0)], ids=str)
def test_bf16_4k_masks(mask, window):
    """bf16 fwd + bwd at the 8 x 32 heads x 4096 tokens size under the full
    predicate and a 512-key window; two sampled heads checked in full."""
    a = inp.workload("bf16_4k")
    note(f"bf16_4k {mask} {window}")
    q, k, v = (to_dev(getattr(a, x), "bf16") for x in "qkv")
    o, lse = run_fwd(q, k, v, S, guard=False, mask=mask, window=window)
    grads = run_bwd(q, k, v, o, o, lse, S, guard=False, mask=mask, window=window)
    torch.cuda.synchronize()
    _check(a, o, lse, grads, mask, window, sel=[(0, 0), (7, 31)])
