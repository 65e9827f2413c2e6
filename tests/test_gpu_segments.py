"""GPU parity for the segment predicate: attn_fwd_seg / attn_bwd_seg, where a
pair (i, j) also needs seg[b, i] == seg[b, j], against the float64 oracle
under the same predicate (oracle.forward_head / backward_head with seg).
Error measure and tolerances as in test_gpu_attention.py (metrics.py): 1e-12
float64, 1e-5 float32, 2e-2 bf16.

Segment ids come from inputs.segment_ids: "packed" documents (contiguous ids,
a geometric length mix) and "interleaved" ids (uniform over a few values per
token, so no key tile is one segment and every tile takes the masked body)."""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import causal_softmax_attention_amd.inputs as inp  # noqa: E402
import oracle  # noqa: E402
from gpu_util import DEV, note, run_bwd, run_fwd, to_dev, to_host  # noqa: E402
from metrics import TOL, assert_close, rel_err  # noqa: E402

S = 0.125
DTYPES = ["f64", "f32", "bf16"]
MASKS = [("causal", 0), ("full", 0), ("window", 37), ("window", 400)]
# (B, H, N, mean document length): several tiles and a ragged tail; B = 2
# checks that batch b reads its own row of ids for each of its heads
SHAPES = [(1, 2, 65, 16), (2, 2, 300, 40), (1, 1, 777, 90)]
KINDS = ["packed", "interleaved"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_softmax_attention_amd as csa
    csa.lib()


def _seg_dev(seg: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(seg, dtype=np.int32)).to(DEV)


def _check(a, seg, o, lse, grads, mask, window, sel=None, tol=None):
    tol = tol or TOL[a.dtype]
    q, k, v = (a.as_f64(x) for x in "qkv")
    B, H = q.shape[:2]
    sel = sel if sel is not None else [(b, h) for b in range(B) for h in range(H)]
    oh, lh = to_host(o), to_host(lse)
    gh = [to_host(g) for g in grads] if grads is not None else None
    for b, h in sel:
        tag = f"[{b},{h}] {mask} {window}"
        wo, wl = oracle.forward_head(q[b, h], k[b, h], v[b, h], S, mask=mask, window=window,
                                     seg=seg[b])[:2]
        assert_close(f"o{tag}", oh[b, h], wo, tol)
        assert_close(f"lse{tag}", lh[b, h], wl, tol)
        if gh is None:
            continue
        want = oracle.backward_head(q[b, h], k[b, h], v[b, h], None, S, mask=mask,
                                    window=window, seg=seg[b])
        for name, g, w in zip(("dq", "dk", "dv"), gh, want):
            assert_close(f"{name}{tag}", g[b, h], w, tol)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("mask,window", MASKS, ids=lambda x: str(x))
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_seg_fwd_bwd(kind, dtype, mask, window, shape):
    B, H, N, mean = shape
    a = inp.attention_inputs(700 + N + window, B, H, N, dtype)
    seg = inp.segment_ids(800 + N, B, N, kind, mean_len=mean)
    note(f"segments {kind} {mask} window={window} {dtype} B={B} H={H} N={N}")
    q, k, v = (to_dev(getattr(a, x), dtype) for x in "qkv")
    sd = _seg_dev(seg)
    o, lse = run_fwd(q, k, v, S, mask=mask, window=window, seg=sd)
    grads = run_bwd(q, k, v, o, o, lse, S, mask=mask, window=window, seg=sd)
    _check(a, seg, o, lse, grads, mask, window)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("mask,window", MASKS, ids=lambda x: str(x))
@pytest.mark.parametrize("shape", [(1, 2, 333), (2, 3, 1000), (2, 3, 1024), (1, 2, 4096)],
                         ids=lambda s: "x".join(map(str, s)))
def test_one_segment_is_no_segment(dtype, mask, window, shape):
    """Every token in one segment (id 7): the segment entry points give the
    results of attn_fwd / attn_bwd under the same mask (equal ids only keep
    weights).  Bit for bit when N fills whole query blocks (256 rows); with a
    ragged last block the padding rows past N see no key in the segment
    kernels (their id is none of the keys') but some keys in the plain ones,
    and a lane's vote for the wave's shared exact-max step can then differ, so
    there the two agree to the tolerance.  For the bf16 causal forward the
    bit-for-bit cases also pin the loop that carries each plain tile's P V into
    the next tile's step (the segment kernel runs the plain loop)."""
    B, H, N = shape
    exact = N % 256 == 0
    a = inp.attention_inputs(91, B, H, N, dtype)
    note(f"one segment {mask} {window} {dtype} {shape}")
    q, k, v = (to_dev(getattr(a, x), dtype) for x in "qkv")
    sd = _seg_dev(np.full((B, N), 7))
    o1, l1 = run_fwd(q, k, v, S, mask=mask, window=window)
    o2, l2 = run_fwd(q, k, v, S, mask=mask, window=window, seg=sd)
    g1 = run_bwd(q, k, v, o1, o1, l1, S, mask=mask, window=window)
    g2 = run_bwd(q, k, v, o1, o1, l1, S, mask=mask, window=window, seg=sd)
    pairs = [("o", o1, o2), ("lse", l1, l2)] + [(n, x, y) for n, x, y in zip(("dq", "dk", "dv"), g1, g2)]
    for name, x, y in pairs:
        if exact:
            assert torch.equal(x, y), name
        else:
            assert_close(name, to_host(y), to_host(x), TOL[dtype])


@pytest.mark.parametrize("dtype", DTYPES)
def test_every_token_its_own_segment(dtype):
    """Distinct ids: each row keeps only its own pair, so o = v, lse_i =
    scale q_i . k_i and dV = dO = o, under every mask."""
    B, H, N = 1, 2, 200
    tol = TOL[dtype]
    a = inp.attention_inputs(92, B, H, N, dtype)
    qh, kh, vh = (a.as_f64(x) for x in "qkv")
    q, k, v = (to_dev(getattr(a, x), dtype) for x in "qkv")
    sd = _seg_dev(np.arange(N)[None] * 3 - 100)
    for mask, window in MASKS:
        note(f"distinct ids {mask} {window} {dtype}")
        o, lse = run_fwd(q, k, v, S, mask=mask, window=window, seg=sd)
        assert rel_err(to_host(o), vh) <= tol
        assert rel_err(to_host(lse), S * np.einsum("bhnd,bhnd->bhn", qh, kh)) <= tol
        dv = run_bwd(q, k, v, o, o, lse, S, mask=mask, window=window, seg=sd)[2]
        assert rel_err(to_host(dv), to_host(o)) <= tol


@pytest.mark.parametrize("dtype", DTYPES)
def test_inf_value_within_its_segment(dtype):
    """V[j, 5] = +inf reaches, in column 5 only, exactly the rows that see key
    j: rows i >= j of j's segment under the causal mask, every row of it under
    the full one.  Ids interleave, so those rows are scattered."""
    B, H, N, j = 1, 1, 400, 150
    a = inp.attention_inputs(43, B, H, N, dtype)
    seg = inp.segment_ids(44, B, N, "interleaved", n_ids=3)
    q, k, v = (to_dev(getattr(a, x), dtype) for x in "qkv")
    v[0, 0, j, 5] = float("inf")
    vh = a.as_f64("v")[0, 0].copy()
    vh[j, 5] = np.inf
    same = seg[0] == seg[0, j]
    for mask, hit in (("causal", same & (np.arange(N) >= j)), ("full", same)):
        note(f"inf in V within segment {mask} {dtype}")
        o, lse = run_fwd(q, k, v, S, mask=mask, seg=_seg_dev(seg))
        oh = to_host(o)[0, 0]
        assert np.isposinf(oh[hit, 5]).all()
        assert np.isfinite(oh[~hit]).all() and np.isfinite(np.delete(oh, 5, axis=1)).all()
        wo, wl = oracle.forward_head(a.as_f64("q")[0, 0], a.as_f64("k")[0, 0], vh, S,
                                     mask=mask, seg=seg[0])[:2]
        assert_close(f"o inf {mask}", oh, wo, TOL[dtype])
        assert_close(f"lse inf {mask}", to_host(lse)[0, 0], wl, TOL[dtype])


@pytest.mark.parametrize("pattern", ["long documents", "a document split by another",
                                     "ids returning", "two long documents, full mask"])
def test_seg_uniform_blocks(pattern):
    """bf16 fwd + bwd where whole key blocks lie in one document, so the
    dK/dV walk takes the plain body on stages wholly inside their document:
    long contiguous documents; one document interrupted by another (its key
    blocks see the other document's rows inside their span, which must stay
    masked); ids that come back after other ids; and the full predicate."""
    B, H, N = 1, 2, 1500
    mask = "full" if "full" in pattern else "causal"
    if pattern == "long documents":
        seg = np.repeat(np.arange(3), [700, 500, 300])[None]
    elif pattern == "a document split by another":
        seg = np.concatenate([np.zeros(600), np.ones(300), np.zeros(600)]).astype(np.int64)[None]
    elif pattern == "ids returning":
        seg = np.tile(np.repeat([4, 9], 250), 3)[None]
    else:
        seg = np.repeat(np.arange(2), [1000, 500])[None]
    a = inp.attention_inputs(1234, B, H, N, "bf16")
    note(f"uniform segment blocks: {pattern}")
    q, k, v = (to_dev(getattr(a, x), "bf16") for x in "qkv")
    sd = _seg_dev(seg)
    o, lse = run_fwd(q, k, v, S, mask=mask, seg=sd)
    grads = run_bwd(q, k, v, o, o, lse, S, mask=mask, seg=sd)
    _check(a, seg, o, lse, grads, mask, 0)


def _segment_starts_equal_v(o, v, seg, tol):
    """Causal with contiguous documents: a document's first row sees only its
    own key, so o there equals v (any size, every head)."""
    starts = np.flatnonzero(np.diff(seg, prepend=seg[:1] - 1) != 0)
    idx = torch.from_numpy(starts).to(DEV)
    got = o[:, :, idx].double()
    want = v[:, :, idx].double()
    err = (got - want).abs().amax() / want.abs().amax()
    assert float(err) <= tol, f"document starts: o vs v {float(err):.3e}"


@pytest.mark.parametrize("kind", KINDS)
def test_bf16_4k_segments(kind):
    """bf16 fwd + bwd at the 8 x 32 heads x 4096 tokens size with packed
    documents (mean 512 tokens) or interleaved ids (2 values), causal; two
    sampled heads checked in full against the oracle, and for packed documents
    o = v at every document start on every head."""
    a = inp.workload("bf16_4k")
    B, H, N = a.q.shape[:3]
    seg = inp.segment_ids(45, B, N, kind, mean_len=512, n_ids=2)
    note(f"bf16_4k segments {kind}")
    q, k, v = (to_dev(getattr(a, x), "bf16") for x in "qkv")
    o, lse = run_fwd(q, k, v, S, guard=False, seg=_seg_dev(seg))
    grads = run_bwd(q, k, v, o, o, lse, S, guard=False, seg=_seg_dev(seg))
    torch.cuda.synchronize()
    for t in (o, lse) + tuple(grads):
        assert bool(torch.isfinite(t).all())
    if kind == "packed":
        for b in range(B):
            _segment_starts_equal_v(o[b:b + 1], v[b:b + 1], seg[b], TOL["bf16"])
    _check(a, seg, o, lse, grads, "causal", 0, sel=[(0, 0), (7, 31)])
