"""GPU parity for the fused training step: attn_fwd_train (the forward plus the
loss sum(o^2)/2 of the pages' GRADIENT statement and the backward's per-row
values) and attn_bwd_from_fwd (its gradient without the per-row pass), against
the float64 oracle.  Same error measure and tolerances as the other GPU tests."""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import causal_softmax_attention_amd.inputs as inp  # noqa: E402
import oracle  # noqa: E402
from gpu_util import note, to_dev, to_host  # noqa: E402
from metrics import TOL, assert_close  # noqa: E402

S = 0.125


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_softmax_attention_amd as csa
    csa.lib()


@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
@pytest.mark.parametrize("mask,window", [("causal", 0), ("full", 0), ("window", 37)], ids=str)
def test_train_step(dtype, mask, window):
    import causal_softmax_attention_amd as csa
    B, H, N = 2, 1, 300
    tol = TOL[dtype]
    a = inp.attention_inputs(90 + window, B, H, N, dtype)
    note(f"train step {dtype} {mask} {window}")
    q, k, v = (to_dev(getattr(a, x), dtype) for x in "qkv")
    o, lse, loss, ws = csa.attn_fwd_train(q, k, v, S, mask, window)
    o2, lse2 = csa.attn_fwd(q, k, v, S, mask, window)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)   # the same forward
    # the loss of the stored o, summed in a fixed order: the same bits twice
    loss_b = csa.attn_fwd_train(q, k, v, S, mask, window)[2]
    torch.cuda.synchronize()
    assert torch.equal(loss, loss_b)
    # each row's |o_i|^2 is accumulated in the path's accumulation type
    # (float32 for float32 and bf16: 64 additions within 2^-24 each)
    oh = to_host(o)
    acc_tol = 1e-12 if dtype == "f64" else 1e-5
    assert abs(loss.item() - 0.5 * np.sum(oh * oh)) <= acc_tol * 0.5 * np.sum(oh * oh)
    qh, kh, vh = (a.as_f64(x) for x in "qkv")
    want_loss = sum(oracle.loss(oracle.forward_head(qh[b, h], kh[b, h], vh[b, h], S, mask=mask,
                                                    window=window)[0])
                    for b in range(B) for h in range(H))
    assert abs(loss.item() - want_loss) <= tol * want_loss
    dq, dk, dv = csa.attn_bwd_from_fwd(q, k, v, o, lse, ws, S, mask, window)
    torch.cuda.synchronize()
    gh = [to_host(g) for g in (dq, dk, dv)]
    for b in range(B):
        for h in range(H):
            want = oracle.backward_head(qh[b, h], kh[b, h], vh[b, h], None, S, mask=mask,
                                        window=window)
            for name, g, w in zip(("dq", "dk", "dv"), gh, want):
                assert_close(f"{name}[{b},{h}] {mask}", g[b, h], w, tol)


def test_train_step_bf16_4k():
    """The fused step at 8 x 32 heads x 4096 tokens: gradients match the
    unfused backward of dout = o, and the loss matches the stored o."""
    import causal_softmax_attention_amd as csa
    a = inp.workload("bf16_4k")
    note("train step bf16_4k")
    q, k, v = (to_dev(getattr(a, x), "bf16") for x in "qkv")
    o, lse, loss, ws = csa.attn_fwd_train(q, k, v, S)
    g1 = csa.attn_bwd_from_fwd(q, k, v, o, lse, ws, S)
    g2 = csa.attn_causal_bwd(q, k, v, o, o, lse, S)
    torch.cuda.synchronize()
    of = o.double()
    assert abs(loss.item() - 0.5 * float((of * of).sum())) <= 1e-5 * loss.item()
    for x, y in zip(g1, g2):
        x, y = x.double(), y.double()
        # delta_i comes from a different sum order than the per-row pass: the
        # gradients agree to bf16 rounding
        assert float((x - y).abs().max()) <= 1e-2 * float(y.abs().max())
    sel = [(0, 0), (7, 31)]
    qh, kh, vh = (a.as_f64(x) for x in "qkv")
    gh = [to_host(g) for g in g1]
    for b, h in sel:
        want = oracle.backward_head(qh[b, h], kh[b, h], vh[b, h], None, S)
        for name, g, w in zip(("dq", "dk", "dv"), gh, want):
            assert_close(f"{name}[{b},{h}]", g[b, h], w, TOL["bf16"])
