"""The allocation-free backward (attn_causal_bwd_noalloc, its workspace in the
library's static per-GPU scratch) against attn_causal_bwd with a caller
workspace: two calls in a row, the second smaller, in every dtype.  Same
kernels, no atomics, so the gradients must agree bit for bit (and so within
the parity tolerance)."""
from __future__ import annotations

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import causal_softmax_attention_amd as csa  # noqa: E402
import causal_softmax_attention_amd.inputs as inp  # noqa: E402
from gpu_util import note, to_dev, to_host  # noqa: E402
from metrics import TOL, rel_err  # noqa: E402

S = 0.125


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa.lib()


@pytest.mark.parametrize("dtype", ["bf16", "f32", "f64"])
def test_noalloc_matches_workspace_backward(dtype):
    for shape in ((2, 3, 1000), (1, 2, 300)):   # the second call is smaller
        B, H, N = shape
        note(f"noalloc bwd {dtype} B={B} H={H} N={N}")
        a = inp.attention_inputs(700 + N, B, H, N, dtype)
        q, k, v = (to_dev(getattr(a, x), dtype) for x in "qkv")
        o, lse = csa.attn_causal_fwd(q, k, v, S)
        want = csa.attn_causal_bwd(q, k, v, o, o, lse, S)
        got = csa.attn_causal_bwd_noalloc(q, k, v, o, o, lse, S)
        torch.cuda.synchronize()
        for name, g, w in zip(("dq", "dk", "dv"), got, want):
            assert torch.equal(g, w), f"{name} {dtype} {shape}: differs from attn_causal_bwd"
            assert rel_err(to_host(g), to_host(w)) <= TOL[dtype]


def test_noalloc_full_bench_size_and_limit():
    """The bf16 bench workload (1,048,576 rows) fits the scratch; a size past
    it is refused before any launch."""
    a = inp.workload("bf16_4k")
    note("noalloc bwd bf16_4k full size")
    q, k, v = (to_dev(getattr(a, x), "bf16") for x in "qkv")
    o, lse = csa.attn_causal_fwd(q, k, v, S)
    want = csa.attn_causal_bwd(q, k, v, o, o, lse, S)
    got = csa.attn_causal_bwd_noalloc(q, k, v, o, o, lse, S)
    torch.cuda.synchronize()
    for g, w in zip(got, want):
        assert torch.equal(g, w)
    del q, k, v, o, lse, got, want
    L = csa.lib()
    rc = L.attn_causal_bwd_noalloc(csa.ATTN_BF16, 1, 8, 1 << 18, 64, S, *([None] * 9), None)
    assert rc == csa.ATTN_EINVAL and "static scratch" in csa.attn_last_error()
