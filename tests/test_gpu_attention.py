"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Error measure and tolerances (metrics.py): per tensor, max|got - want| /
max|want| over finite entries, with non-finite entries matching exactly;
1e-12 for float64, 1e-5 for float32, 2e-2 for bfloat16 inputs.

The upstream gradient of the loss sum(o^2)/2 is o itself; each side uses its
own o (the oracle its float64 o, the GPU the o its forward returned), so the
oracle's gradient is the exact gradient at the stored inputs.
"""
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_softmax_attention_amd as csa
    csa.lib()


def _heads(a: inp.AttentionInputs, sel=None):
    """float64 views of selected (b, h) heads: list of (q, k, v)."""
    q, k, v = (a.as_f64(x) for x in "qkv")
    B, H = q.shape[:2]
    sel = sel if sel is not None else [(b, h) for b in range(B) for h in range(H)]
    return sel, [(q[b, h], k[b, h], v[b, h]) for b, h in sel]


def _stacked(a, sel):
    """The selected heads as float64 arrays [1, len(sel), N, D] (q, k, v), for the
    oracle's batched functions and their thread pool over heads."""
    sel, heads = _heads(a, sel)
    return sel, [np.stack([hd[i] for hd in heads])[None] for i in range(3)]


WORKERS = 8


def _check_fwd(a, o, lse, sel=None, tol=None):
    tol = tol or TOL[a.dtype]
    sel, (q, k, v) = _stacked(a, sel)
    oh, lh = to_host(o), to_host(lse)
    wo, wl = oracle.forward(q, k, v, S, workers=WORKERS)
    for n, (b, h) in enumerate(sel):
        assert_close(f"o[{b},{h}]", oh[b, h], wo[0, n], tol)
        assert_close(f"lse[{b},{h}]", lh[b, h], wl[0, n], tol)


def _check_bwd(a, grads, sel=None, dout=None):
    tol = TOL[a.dtype]
    sel, (q, k, v) = _stacked(a, sel)
    gh = [to_host(g) for g in grads]
    d = None if dout is None else np.stack([dout[b, h] for b, h in sel])[None]
    want = oracle.backward(q, k, v, d, S, workers=WORKERS)
    for n, (b, h) in enumerate(sel):
        for name, g, w in zip(("dq", "dk", "dv"), gh, want):
            assert_close(f"{name}[{b},{h}]", g[b, h], w[0, n], tol)


def _check_all_heads(a, o, lse, grads, tol):
    """Per-head properties that hold at any size, on every head of a full-size
    run (computed on the device): every output finite; row 0 of o equals V[0]
    (its only pair); the rows of P sum to 1, so sum_j dV_j = sum_i dO_i (dO = o);
    each row of dS sums to 0, so sum_j dK_j = 0 up to rounding."""
    v = to_dev(a.v, a.dtype)
    for name, t in (("o", o), ("lse", lse)) + tuple(zip(("dq", "dk", "dv"), grads)):
        assert bool(torch.isfinite(t).all()), f"{name} has a non-finite entry"
    o64, v64 = o.double(), v.double()
    B, H = o.shape[:2]
    e0 = ((o64[:, :, 0] - v64[:, :, 0]).abs().amax(dim=-1) /
          v64[:, :, 0].abs().amax(dim=-1).clamp_min(1e-30))
    assert float(e0.max()) <= tol, f"row 0 of o vs V[0]: worst head {float(e0.max()):.3e}"
    dk64, dv64 = grads[1].double(), grads[2].double()
    sdv, so = dv64.sum(dim=2), o64.sum(dim=2)
    edv = (sdv - so).abs().amax(dim=-1) / so.abs().amax(dim=-1)
    assert float(edv.max()) <= tol, f"sum dV vs sum dO: worst head {float(edv.max()):.3e}"
    N = o.shape[2]
    edk = dk64.sum(dim=2).abs().amax(dim=-1) / (N * dk64.abs().amax(dim=(-1, -2)))
    assert float(edk.max()) <= tol, f"sum dK: worst head {float(edk.max()):.3e}"
    assert e0.shape == (B, H)


def _grid_heads(B, H):
    """Flat heads covering every XCD (workgroup b runs on XCD b % 8 and takes
    heads b % 8, b % 8 + 8, ...) and the first and last 8 heads of each XCD's
    sequence, so every position in its first and last groups (groups of 4
    heads in the forward, whose last two form one group of 8, and in the
    backward): head x + 8 x (the XCD's head x) and head x + 8 (n - 1 - x)
    (its head n - 1 - x), as (b, h)."""
    n = (B * H) // 8
    flat = sorted({x + 8 * min(x, n - 1) for x in range(8)} |
                  {x + 8 * max(n - 1 - x, 0) for x in range(8)})
    return [(f // H, f % H) for f in flat if f < B * H]


SMALL = [(1, 1, 1), (1, 1, 2), (1, 1, 17), (2, 3, 63), (1, 2, 64), (1, 2, 65), (1, 1, 127),
         (2, 1, 129), (1, 1, 300), (1, 2, 1000)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_small_fwd_bwd(dtype, shape):
    B, H, N = shape
    a = inp.attention_inputs(100 + N, B, H, N, dtype)
    note(f"fwd+bwd {dtype} B={B} H={H} N={N}")
    q, k, v = (to_dev(getattr(a, x), dtype) for x in "qkv")
    o, lse = run_fwd(q, k, v, S)
    _check_fwd(a, o, lse)
    grads = run_bwd(q, k, v, o, o, lse, S)
    _check_bwd(a, grads)


# (dtype, qk_mult).  At qk_mult 6 the scores reach about +-100, and float32's
# own rounding of a 64-term dot product (about 1e-4 of the score's terms) moves
# the weights by more than the float32 tolerance of 1e-5: that case is float32
# arithmetic, not the kernel, so it is checked in float64 and bfloat16 only.
PEAKED = [("f64", 3.0), ("f32", 3.0), ("bf16", 3.0), ("f64", 6.0), ("bf16", 6.0)]


@pytest.mark.parametrize("dtype,qk_mult", PEAKED, ids=lambda x: str(x))
def test_peaked_scores(dtype, qk_mult):
    """q and k drawn N(0, qk_mult^2): scores qk_mult^2 times those of the unit
    workload, so the softmax is peaked and any rounding of the score operands
    moves the weights in proportion to the score.  Fwd and bwd checked in full
    against the oracle, at the same tolerances."""
    B, H, N = 1, 2, 1000
    a = inp.attention_inputs(131, B, H, N, dtype, qk_mult=qk_mult)
    note(f"peaked scores {dtype} qk_mult={qk_mult} B={B} H={H} N={N}")
    q, k, v = (to_dev(getattr(a, x), dtype) for x in "qkv")
    o, lse = run_fwd(q, k, v, S)
    _check_fwd(a, o, lse)
    grads = run_bwd(q, k, v, o, o, lse, S)
    _check_bwd(a, grads)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_head_groups(dtype):
    """21 heads: an XCD's heads (workgroup b runs on XCD b % 8) come in groups
    of 4 or 8 whose last group is short here (3 and 2 heads per XCD), and
    each head has several blocks.  Every (head, block) must be computed
    exactly once: all heads against the oracle."""
    B, H, N = 3, 7, 300
    a = inp.attention_inputs(21, B, H, N, dtype)
    note(f"head groups fwd+bwd {dtype} B={B} H={H} N={N}")
    q, k, v = (to_dev(getattr(a, x), dtype) for x in "qkv")
    o, lse = run_fwd(q, k, v, S)
    _check_fwd(a, o, lse)
    grads = run_bwd(q, k, v, o, o, lse, S)
    _check_bwd(a, grads)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_merged_last_group(dtype):
    """100 heads: 12 or 13 per XCD, so the bf16 forward's groups of 4 heads
    end in one merged group of 8 or 9 after a whole group of 4.  Every (head,
    block) must be computed exactly once: all heads against the oracle."""
    B, H, N = 4, 25, 200
    a = inp.attention_inputs(22, B, H, N, dtype)
    note(f"merged last head group fwd+bwd {dtype} B={B} H={H} N={N}")
    q, k, v = (to_dev(getattr(a, x), dtype) for x in "qkv")
    o, lse = run_fwd(q, k, v, S)
    _check_fwd(a, o, lse)
    grads = run_bwd(q, k, v, o, o, lse, S)
    _check_bwd(a, grads)


@pytest.mark.parametrize("dtype", DTYPES)
def test_general_dout(dtype):
    """An upstream gradient that is not o (same seeded dout on both sides)."""
    B, H, N = 2, 2, 200
    a = inp.attention_inputs(7, B, H, N, dtype)
    d = inp.attention_inputs(8, B, H, N, dtype)      # its q serves as dout
    dout_f64 = d.as_f64("q")
    note(f"bwd general dout {dtype}")
    q, k, v = (to_dev(getattr(a, x), dtype) for x in "qkv")
    dout = to_dev(d.q, dtype)
    o, lse = run_fwd(q, k, v, S)
    grads = run_bwd(q, k, v, o, dout, lse, S)
    _check_bwd(a, grads, dout=dout_f64)


def test_fp64_256_with_inf():
    """The 256-token float64 workload: fwd + bwd at 1e-12, then V[100, 5] = +inf
    reaches only rows >= 100, in column 5 only."""
    a = inp.workload("fp64_256")
    note("fp64_256 fwd+bwd")
    q, k, v = (to_dev(getattr(a, x), "f64") for x in "qkv")
    o, lse = run_fwd(q, k, v, S)
    _check_fwd(a, o, lse)
    grads = run_bwd(q, k, v, o, o, lse, S)
    _check_bwd(a, grads)
    note("fp64_256 inf run")
    v2 = v.clone()
    v2[0, 0, 100, 5] = float("inf")
    o2, lse2 = run_fwd(q, k, v2, S)
    oh = to_host(o2)[0, 0]
    assert np.isfinite(oh[:100]).all()
    assert np.isposinf(oh[100:, 5]).all()
    assert np.isfinite(np.delete(oh, 5, axis=1)).all()
    assert np.isfinite(to_host(lse2)).all()
    vh = a.as_f64("v")[0, 0].copy()
    vh[100, 5] = np.inf
    wo, wl = oracle.forward_head(a.as_f64("q")[0, 0], a.as_f64("k")[0, 0], vh, S)[:2]
    assert_close("o (inf run)", oh, wo, TOL["f64"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_inf_value_several_tiles(dtype):
    """V[150, 5] = +inf with 2 heads of 700 tokens: it reaches rows >= 150 of its
    head, in column 5 only, and every other entry matches the oracle."""
    B, H, N, j = 1, 2, 700, 150
    a = inp.attention_inputs(31, B, H, N, dtype)
    note(f"inf in V, several tiles, {dtype}")
    q, k, v = (to_dev(getattr(a, x), dtype) for x in "qkv")
    v[0, 1, j, 5] = float("inf")
    o, lse = run_fwd(q, k, v, S)
    oh, lh = to_host(o)[0, 1], to_host(lse)[0, 1]
    assert np.isposinf(oh[j:, 5]).all()
    assert np.isfinite(np.delete(oh, 5, axis=1)).all() and np.isfinite(oh[:j]).all()
    vh = a.as_f64("v")[0, 1].copy()
    vh[j, 5] = np.inf
    wo, wl = oracle.forward_head(a.as_f64("q")[0, 1], a.as_f64("k")[0, 1], vh, S)[:2]
    assert_close("o (inf run)", oh, wo, TOL[dtype])
    assert_close("lse (inf run)", lh, wl, TOL[dtype])
    _check_fwd(a, o, lse, sel=[(0, 0)])


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("mask,window", [(None, 0), ("full", 0), ("window", 300)],
                         ids=lambda x: str(x))
def test_negative_inf_and_nan_values(dtype, mask, window):
    """V[150, 3] = -inf and V[400, 7] = NaN in one head of 700 tokens: each reaches
    exactly the rows whose pairs include its key (causal: rows >= j; full: every
    row; a 300-key window: rows j .. j + 299), in its own column only, so the
    masked tiles' scan for non-finite V must catch both kinds."""
    B, H, N = 1, 1, 700
    a = inp.attention_inputs(77, B, H, N, dtype)
    note(f"-inf and NaN in V, {mask} {window} {dtype}")
    q, k, v = (to_dev(getattr(a, x), dtype) for x in "qkv")
    v[0, 0, 150, 3] = float("-inf")
    v[0, 0, 400, 7] = float("nan")
    vh = a.as_f64("v")[0, 0].copy()
    vh[150, 3] = -np.inf
    vh[400, 7] = np.nan
    o, lse = run_fwd(q, k, v, S, mask=mask, window=window)
    oh, lh = to_host(o)[0, 0], to_host(lse)[0, 0]
    rows = np.arange(N)
    for j, c in ((150, 3), (400, 7)):
        if mask == "full":
            hit = np.ones(N, bool)
        elif mask == "window":
            hit = (rows >= j) & (rows - j < window)
        else:
            hit = rows >= j
        assert (~np.isfinite(oh[hit, c])).all() and np.isfinite(oh[~hit, c]).all()
    assert np.isfinite(np.delete(oh, [3, 7], axis=1)).all() and np.isfinite(lh).all()
    omode = mask or "causal"
    wo, wl = oracle.forward_head(a.as_f64("q")[0, 0], a.as_f64("k")[0, 0], vh, S, mask=omode,
                                 window=window)[:2]
    assert_close("o (-inf / NaN run)", oh, wo, TOL[dtype])
    assert_close("lse (-inf / NaN run)", lh, wl, TOL[dtype])


@pytest.mark.parametrize("dtype", DTYPES)
def test_page_mask_case(dtype):
    """The demo's own mask check: n = 16, +inf at v[9, 0], seed 1."""
    q, k, v, j = inp.page_mask_inputs()
    note(f"page mask case {dtype}")
    qd, kd, vd = (to_dev(inp.cast(x, dtype), dtype)[None, None] for x in (q, k, v))
    o, lse = run_fwd(qd, kd, vd, S)
    oh = to_host(o)[0, 0]
    assert np.isfinite(oh[:j]).all()
    assert np.isposinf(oh[j:, 0]).all()
    assert np.isfinite(oh[:, 1:]).all()


def test_page_sizes_fp64():
    """The demo's sizes (64 and 256 tokens, seed 0): fwd and gradients."""
    for n, (q, k, v) in inp.page_sizes_inputs().items():
        note(f"page size n={n} f64")
        qd, kd, vd = (to_dev(x, "f64")[None, None] for x in (q, k, v))
        o, lse = run_fwd(qd, kd, vd, S)
        wo, wl = oracle.forward_head(q, k, v, S)[:2]
        assert_close("o", to_host(o)[0, 0], wo, 1e-12)
        assert_close("lse", to_host(lse)[0, 0], wl, 1e-12)
        grads = run_bwd(qd, kd, vd, o, o, lse, S)
        for name, g, w in zip(("dq", "dk", "dv"), grads, oracle.backward_head(q, k, v, None, S)):
            assert_close(name, to_host(g)[0, 0], w, 1e-12)


@pytest.mark.parametrize("dtype", DTYPES)
def test_invariants(dtype):
    """Properties that hold at any size: Q = 0 gives prefix means of V and
    lse = ln(i+1); constant V gives that constant; row 0 equals V[0]; sum_j dK_j
    = 0 and sum_j dV_j = sum_i dO_i; rows < t do not depend on tokens >= t."""
    tol = TOL[dtype]
    B, H, N = 1, 2, 777
    a = inp.attention_inputs(55, B, H, N, dtype)
    q, k, v = (to_dev(getattr(a, x), dtype) for x in "qkv")
    note(f"invariants {dtype}")
    vh = a.as_f64("v")
    o, lse = run_fwd(torch.zeros_like(q), k, v, S)
    means = np.cumsum(vh, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    assert rel_err(to_host(o), means) <= tol
    assert rel_err(to_host(lse), np.broadcast_to(np.log(np.arange(1, N + 1)), (B, H, N))) <= tol
    c = v[:, :, :1, :].expand(B, H, N, 64).contiguous()
    o, _ = run_fwd(q, k, c, S)
    assert rel_err(to_host(o), np.broadcast_to(to_host(c), (B, H, N, 64))) <= tol
    o, lse = run_fwd(q, k, v, S)
    assert rel_err(to_host(o)[:, :, 0], vh[:, :, 0]) <= tol
    dq, dk, dv = run_bwd(q, k, v, o, o, lse, S)
    dkh, dvh, oh = to_host(dk), to_host(dv), to_host(o)
    assert np.abs(dkh.sum(axis=2)).max() <= tol * N * np.abs(dkh).max()
    assert rel_err(dvh.sum(axis=2), oh.sum(axis=2)) <= tol
    t = 333
    o_t, _ = run_fwd(q[:, :, :t].contiguous(), k[:, :, :t].contiguous(), v[:, :, :t].contiguous(), S)
    assert rel_err(to_host(o_t), oh[:, :, :t]) <= tol


def test_fp32_2k_fwd():
    """Float32 forward at full size (4 x 16 heads x 2048 tokens); sampled heads vs the oracle."""
    a = inp.workload("fp32_2k")
    note("fp32_2k fwd full size")
    q, k, v = (to_dev(getattr(a, x), "f32") for x in "qkv")
    o, lse = run_fwd(q, k, v, S, guard=False)
    torch.cuda.synchronize()
    _check_fwd(a, o, lse, sel=_grid_heads(4, 16))


def test_bf16_4k_fwd_bwd():
    """bfloat16 fwd + bwd at full size (8 x 32 heads x 4096 tokens), in the
    launch configuration the bench times: 16 heads covering every XCD and every
    position of the forward's and backward's head groups checked in full
    against the oracle, and every head against the per-head invariants."""
    a = inp.workload("bf16_4k")
    note("bf16_4k fwd+bwd full size")
    q, k, v = (to_dev(getattr(a, x), "bf16") for x in "qkv")
    o, lse = run_fwd(q, k, v, S, guard=False)
    grads = run_bwd(q, k, v, o, o, lse, S, guard=False)
    torch.cuda.synchronize()
    _check_all_heads(a, o, lse, grads, TOL["bf16"])
    sel = _grid_heads(8, 32)
    assert len(sel) == 16
    _check_fwd(a, o, lse, sel=sel)
    _check_bwd(a, grads, sel=sel)


def test_bf16_32k_fwd_bwd():
    """bfloat16 fwd + bwd at full size (16 heads x 32768 tokens, q and k scaled
    by 2: peaked rows); three heads (XCDs 0, 3 and 7) checked in full, every
    head against the per-head invariants."""
    a = inp.workload("bf16_32k")
    note("bf16_32k fwd+bwd full size")
    q, k, v = (to_dev(getattr(a, x), "bf16") for x in "qkv")
    o, lse = run_fwd(q, k, v, S, guard=False)
    grads = run_bwd(q, k, v, o, o, lse, S, guard=False)
    torch.cuda.synchronize()
    _check_all_heads(a, o, lse, grads, TOL["bf16"])
    sel = [(0, 0), (0, 11), (0, 15)]
    _check_fwd(a, o, lse, sel=sel)
    _check_bwd(a, grads, sel=sel)


def test_non_default_stream():
    a = inp.attention_inputs(9, 1, 2, 300, "bf16")
    q, k, v = (to_dev(getattr(a, x), "bf16") for x in "qkv")
    import causal_softmax_attention_amd as csa
    note("non-default stream")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = csa.attn_causal_fwd(q, k, v, S)
        grads = csa.attn_causal_bwd(q, k, v, o, o, lse, S)
    s.synchronize()
    _check_fwd(a, o, lse)
    _check_bwd(a, grads)
