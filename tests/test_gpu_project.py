"""GPU parity for the Q / K / V input projections (attn_qkv_project) against
the oracle's float64 products.  Error measure and tolerances as in the other
GPU tests (float64 1e-12, float32 1e-5, bfloat16 2e-2 relative to the largest
output; the bfloat16 results are rounded once, to nearest even, from float32
sums of exact products, so they sit within one bfloat16 ulp of the oracle)."""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import causal_softmax_attention_amd.inputs as inp  # noqa: E402
from oracle import projection  # noqa: E402
from gpu_util import note, to_dev, to_host  # noqa: E402
from metrics import TOL, assert_close  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_softmax_attention_amd as csa
    csa.lib()


def _run(a):
    import causal_softmax_attention_amd as csa
    dev = [to_dev(getattr(a, n), a.dtype) for n in ("x", "wq", "wk", "wv")]
    return csa.attn_qkv_project(*dev, a.heads)


# (B, N, Dm, H): several token blocks and a ragged tail, a batch boundary
# inside a block, Dm a multiple of 64 (the MFMA kernel for bf16) or not, and
# head counts that fill groups of 4 heads and leave a short one (5, 9)
SHAPES = [(1, 256, 64, 1), (3, 300, 128, 2), (2, 77, 192, 3), (1, 513, 320, 1),
          (2, 100, 100, 2), (1, 5, 7, 1), (2, 700, 128, 5), (1, 300, 64, 9)]


@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
@pytest.mark.parametrize("B,N,Dm,H", SHAPES, ids=str)
def test_project(dtype, B, N, Dm, H):
    a = inp.projection_inputs(50 + B + N + Dm, B, N, Dm, H, dtype)
    note(f"qkv_project {dtype} B={B} N={N} Dm={Dm} H={H}")
    got = _run(a)
    torch.cuda.synchronize()
    want = projection.project_qkv(a.as_f64("x"), a.as_f64("wq"), a.as_f64("wk"), a.as_f64("wv"), H)
    for name, g, w in zip("qkv", got, want):
        assert tuple(g.shape) == (B, H, N, 64)
        assert_close(f"{name} {dtype}", to_host(g), w, TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_identity_weights_are_exact(dtype):
    """W = identity (Dm = H * 64): every output equals its x element bit for
    bit (products by 1 and sums with 0 are exact)."""
    import causal_softmax_attention_amd as csa
    B, N, H = 2, 300, 2
    a = inp.projection_inputs(61, B, N, 64 * H, H, dtype)
    note(f"qkv_project identity {dtype}")
    x = to_dev(a.x, dtype)
    eye = torch.eye(64 * H, dtype=x.dtype, device=x.device)
    q, k, v = csa.attn_qkv_project(x, eye, eye, eye, H)
    torch.cuda.synchronize()
    want = x.view(B, N, H, 64).permute(0, 2, 1, 3).contiguous()
    for t in (q, k, v):
        assert torch.equal(t, want)


def test_project_workload_sampled():
    """The bench workload (x [8, 4096, 2048] -> Q, K, V [8, 32, 4096, 64] bf16):
    200 sampled tokens against the oracle, all heads and features."""
    name = "proj_4k"
    seed, B, N, Dm, H, dtype = inp.PROJECTION_WORKLOADS[name]
    a = inp.projection_workload(name)
    note(f"qkv_project workload {name}")
    got = _run(a)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    tok = rng.choice(B * N, size=200, replace=False)
    b, n = tok // N, tok % N
    xs = a.as_f64("x")[b, n][None]                     # [1, 200, Dm]
    want = projection.project_qkv(xs, a.as_f64("wq"), a.as_f64("wk"), a.as_f64("wv"), H)
    for nm, g, w in zip("qkv", got, want):
        gs = to_host(g[torch.from_numpy(b), :, torch.from_numpy(n)])   # [200, H, 64]
        assert_close(f"{nm} sampled", gs, w[0].transpose(1, 0, 2), TOL[dtype])
        assert torch.isfinite(g).all()
