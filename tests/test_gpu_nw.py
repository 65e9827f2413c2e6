"""GPU parity for the Nadaraya-Watson control against the float64 oracle
(float32 tolerance 1e-5, max-norm relative)."""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import causal_softmax_attention_amd as csa  # noqa: E402
import causal_softmax_attention_amd.inputs as inp  # noqa: E402
import oracle  # noqa: E402
from gpu_util import DEV, Guarded, note  # noqa: E402
from metrics import assert_close  # noqa: E402

TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa.lib()


def _dev(*arrs):
    return [torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV) for a in arrs]


def _run(a: inp.NWInputs, denom=0.25):
    tx, ty, sx, sy, sv = _dev(a.tx, a.ty, a.sx, a.sy, a.sv)
    g = Guarded((len(a.tx),), torch.float32)
    out = csa.nw_gauss_average(tx, ty, sx, sy, sv, denom, out=g.view)
    torch.cuda.synchronize()
    assert g.intact(), "nw wrote outside its output"
    return out.cpu().numpy().astype(np.float64)


def _f32(a: inp.NWInputs) -> inp.NWInputs:
    f = lambda x: np.asarray(x, dtype=np.float32)
    return inp.NWInputs(f(a.tx), f(a.ty), f(a.sx), f(a.sy), f(a.sv))


@pytest.mark.parametrize("nt,ns", [(1, 1), (1, 300), (300, 77), (257, 64), (1000, 1000),
                                   (4096, 129)])
def test_small(nt, ns):
    a = _f32(inp.nw_inputs(nt, ns, seed=nt + ns))
    note(f"nw {nt}x{ns}")
    got = _run(a)
    assert_close("nw", got, oracle.nw_average(a.tx, a.ty, a.sx, a.sy, a.sv, 0.25), TOL)


def test_page_case():
    """The demo's control: 64 targets, 256 sources on [0, 1)^2, seed 2."""
    a = _f32(inp.page_nw_inputs())
    note("nw page case")
    got = _run(a)
    assert_close("nw", got, oracle.nw_average(a.tx, a.ty, a.sx, a.sy, a.sv, 0.25), TOL)


def test_far_targets_and_late_maximum():
    """Targets far from every source (unshifted weights underflow to 0/0) and
    sources ordered so that the nearest one comes last (the running max must
    rise many times)."""
    rng = np.random.default_rng(5)
    ns = 1000
    sx = np.linspace(50.0, 0.0, ns)       # nearest to the origin last
    sy = np.zeros(ns)
    sv = rng.normal(size=ns)
    tx = np.array([0.0, -30.0, 400.0, 25.0, 1e3])
    ty = np.array([0.0, 5.0, -300.0, 0.5, 1e3])
    a = _f32(inp.NWInputs(tx, ty, sx, sy, sv))
    note("nw far targets")
    got = _run(a)
    want = oracle.nw_average(a.tx, a.ty, a.sx, a.sy, a.sv, 0.25)
    assert np.isfinite(got).all()
    assert_close("nw", got, want, TOL)


def test_other_denominator():
    a = _f32(inp.nw_inputs(500, 700, seed=6))
    note("nw denom 3.0")
    got = _run(a, denom=3.0)
    assert_close("nw", got, oracle.nw_average(a.tx, a.ty, a.sx, a.sy, a.sv, 3.0), TOL)


def test_nw_64k():
    """The 65,536 x 65,536 workload at full size; 2,048 sampled targets vs the oracle."""
    a = inp.nw_inputs()
    note("nw_64k full size")
    got = _run(a)
    idx = np.random.default_rng(0).choice(len(a.tx), 2048, replace=False)
    want = oracle.nw_average(a.tx[idx], a.ty[idx], a.sx, a.sy, a.sv, 0.25)
    assert_close("nw", got[idx], want, TOL)
