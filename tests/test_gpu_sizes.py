"""GPU parity at the size limits: very long heads and very many heads, each
checked in the launch configuration the library uses for them.

Where the oracle cannot finish the whole output in seconds, rows are checked
against it through properties that hold at any size: output row i and dQ row
i depend only on tokens <= i (so the first rows equal the oracle's result on
that prefix), sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i.  Error measure and
tolerances as in the other GPU tests."""
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_softmax_attention_amd as csa
    csa.lib()


def _prefix_check(a, o, lse, dq, t, tol, b=0, h=0):
    q, k, v = (a.as_f64(x)[b, h, :t] for x in "qkv")
    wo, wl = oracle.forward_head(q, k, v, S)[:2]
    assert_close("o prefix", to_host(o)[b, h, :t], wo, tol)
    assert_close("lse prefix", to_host(lse)[b, h, :t], wl, tol)
    if dq is not None:
        # dQ_i = scale sum_{j<=i} dS_ij k_j with dO = O: rows < t see only the prefix
        wq = oracle.backward_head(q, k, v, None, S)[0]
        assert_close("dq prefix", to_host(dq)[b, h, :t], wq, tol)


def _grad_invariants(o, dk, dv, tol):
    dkh, dvh, oh = to_host(dk), to_host(dv), to_host(o)
    n = dkh.shape[2]
    assert np.abs(dkh.sum(axis=2)).max() <= tol * n * np.abs(dkh).max()
    assert rel_err(dvh.sum(axis=2), oh.sum(axis=2)) <= tol


def test_bf16_131072_tokens():
    """One head of 2^17 tokens (the bf16 path's largest-grid shape per head)."""
    N = 1 << 17
    a = inp.attention_inputs(123, 1, 1, N, "bf16")
    note(f"bf16 one head N={N}")
    q, k, v = (to_dev(getattr(a, x), "bf16") for x in "qkv")
    o, lse = run_fwd(q, k, v, S)
    dq, dk, dv = run_bwd(q, k, v, o, o, lse, S)
    assert np.isfinite(to_host(o)).all() and np.isfinite(to_host(dk)).all()
    _prefix_check(a, o, lse, dq, 1500, TOL["bf16"])
    _grad_invariants(o, dk, dv, TOL["bf16"])


def test_bf16_65536_heads():
    """65,536 heads of 65 tokens (one key block and a ragged tail per head)."""
    B, H, N = 4096, 16, 65
    a = inp.attention_inputs(124, B, H, N, "bf16")
    note(f"bf16 B={B} H={H} N={N}")
    q, k, v = (to_dev(getattr(a, x), "bf16") for x in "qkv")
    o, lse = run_fwd(q, k, v, S)
    dq, dk, dv = run_bwd(q, k, v, o, o, lse, S)
    qh, kh, vh = (a.as_f64(x) for x in "qkv")
    oh, lh = to_host(o), to_host(lse)
    gh = [to_host(g) for g in (dq, dk, dv)]
    for b, h in [(0, 0), (1234, 7), (2048, 15), (4095, 15)]:
        wo, wl = oracle.forward_head(qh[b, h], kh[b, h], vh[b, h], S)[:2]
        assert_close(f"o[{b},{h}]", oh[b, h], wo, TOL["bf16"])
        assert_close(f"lse[{b},{h}]", lh[b, h], wl, TOL["bf16"])
        for name, g, w in zip(("dq", "dk", "dv"), gh,
                              oracle.backward_head(qh[b, h], kh[b, h], vh[b, h], None, S)):
            assert_close(f"{name}[{b},{h}]", g[b, h], w, TOL["bf16"])


def test_f32_65536_tokens():
    """float32 forward (MFMA) and backward on one head of 2^16 tokens."""
    N = 1 << 16
    a = inp.attention_inputs(125, 1, 1, N, "f32")
    note(f"f32 one head N={N}")
    q, k, v = (to_dev(getattr(a, x), "f32") for x in "qkv")
    o, lse = run_fwd(q, k, v, S)
    dq, dk, dv = run_bwd(q, k, v, o, o, lse, S)
    _prefix_check(a, o, lse, dq, 1200, TOL["f32"])
    _grad_invariants(o, dk, dv, TOL["f32"])


def test_f64_4096_tokens():
    """float64 at 4096 tokens, two heads, checked in full."""
    a = inp.attention_inputs(126, 1, 2, 4096, "f64")
    note("f64 N=4096")
    q, k, v = (to_dev(getattr(a, x), "f64") for x in "qkv")
    o, lse = run_fwd(q, k, v, S)
    grads = run_bwd(q, k, v, o, o, lse, S)
    qh, kh, vh = (a.as_f64(x) for x in "qkv")
    for h in range(2):
        wo, wl = oracle.forward_head(qh[0, h], kh[0, h], vh[0, h], S)[:2]
        assert_close("o", to_host(o)[0, h], wo, TOL["f64"])
        assert_close("lse", to_host(lse)[0, h], wl, TOL["f64"])
        for name, g, w in zip(("dq", "dk", "dv"), grads,
                              oracle.backward_head(qh[0, h], kh[0, h], vh[0, h], None, S)):
            assert_close(name, to_host(g)[0, h], w, TOL["f64"])


@pytest.mark.parametrize("mask,window", [(None, 0), ("window", 200), ("full", 0)], ids=str)
def test_f64_many_heads_unsplit(mask, window):
    """float64 with 32 heads of 512 tokens: enough 32-row blocks (512) that the
    row kernels walk each row with one group (a few heads, or short rows, make
    them split each row's walk over 8 groups).  Heads 0, 13 and 31 against the
    oracle in full."""
    B, H, N = 4, 8, 512
    a = inp.attention_inputs(127, B, H, N, "f64")
    note(f"f64 unsplit rows B={B} H={H} N={N} mask={mask} window={window}")
    q, k, v = (to_dev(getattr(a, x), "f64") for x in "qkv")
    o, lse = run_fwd(q, k, v, S, mask=mask, window=window)
    grads = run_bwd(q, k, v, o, o, lse, S, mask=mask, window=window)
    qh, kh, vh = (a.as_f64(x) for x in "qkv")
    kw = {} if mask is None else {"mask": mask, "window": window}
    for bh in (0, 13, 31):
        b, h = divmod(bh, H)
        wo, wl = oracle.forward_head(qh[b, h], kh[b, h], vh[b, h], S, **kw)[:2]
        assert_close(f"o[{b},{h}]", to_host(o)[b, h], wo, TOL["f64"])
        assert_close(f"lse[{b},{h}]", to_host(lse)[b, h], wl, TOL["f64"])
        want = oracle.backward_head(qh[b, h], kh[b, h], vh[b, h], None, S, **kw)
        for name, g, w in zip(("dq", "dk", "dv"), grads, want):
            assert_close(f"{name}[{b},{h}]", to_host(g)[b, h], w, TOL["f64"])
