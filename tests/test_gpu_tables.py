"""GPU parity for the long-table <-> matrix adapter (attn_matrix_to_table,
attn_table_to_matrix) against the oracle's table() / matrix().  Index and byte
work: every comparison is bit-exact (t, d as integers; values as raw bits,
holes as the element type's quiet NaN)."""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import causal_softmax_attention_amd.inputs as inp  # noqa: E402
from oracle import tables  # noqa: E402
from gpu_util import DEV, note  # noqa: E402

NP_BITS = {"f64": np.uint64, "f32": np.uint32, "bf16": np.uint16}
TORCH_BITS = {"f64": torch.int64, "f32": torch.int32, "bf16": torch.int16}
TORCH_DT = {"f64": torch.float64, "f32": torch.float32, "bf16": torch.bfloat16}
NAN_BITS = {"f64": 0x7FF8000000000000, "f32": 0x7FC00000, "bf16": 0x7FC0}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_softmax_attention_amd as csa
    csa.lib()


def _values(seed, T, D, dtype):
    """Storage-format values (bit patterns for bf16) with special values mixed in."""
    m, _ = inp.table_matrix(seed, T, D, dtype)
    flat = m.reshape(-1)
    if dtype == "bf16":
        specials = np.array([0x8000, 0x7F80, 0xFF80, 0x0001, 0x0080], dtype=np.uint16)
    else:
        ft = np.float64 if dtype == "f64" else np.float32
        specials = np.array([-0.0, np.inf, -np.inf, np.finfo(ft).tiny / 4, np.finfo(ft).tiny],
                            dtype=ft)
    k = min(flat.size, specials.size)
    flat[:k] = specials[:k]
    return m


def _to_dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a).view(NP_BITS[dtype]).view(
        {"f64": np.int64, "f32": np.int32, "bf16": np.int16}[dtype])).to(DEV).view(TORCH_DT[dtype])


def _bits(t, dtype):
    return t.view(TORCH_BITS[dtype]).cpu().numpy().view(NP_BITS[dtype])


@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
@pytest.mark.parametrize("T,D", [(1, 1), (3, 64), (257, 65), (64, 64), (5, 3)])
def test_matrix_to_table(dtype, T, D):
    import causal_softmax_attention_amd as csa
    m = _values(30 + T + D, T, D, dtype)
    note(f"matrix_to_table {dtype} {T}x{D}")
    t, d, x = csa.attn_matrix_to_table(_to_dev(m, dtype))
    torch.cuda.synchronize()
    wt, wd, wx = tables.table(m.view(NP_BITS[dtype]))
    assert np.array_equal(t.cpu().numpy(), wt) and np.array_equal(d.cpu().numpy(), wd)
    assert np.array_equal(_bits(x, dtype), wx)


@pytest.mark.parametrize("order", ["shuffled", "ordered"])
@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
@pytest.mark.parametrize("T,D,holes", [(1, 1, 0), (3, 64, 0), (257, 65, 0), (64, 64, 37),
                                       (9, 7, 5)])
def test_table_to_matrix(dtype, T, D, holes, order):
    """Rows shuffled, or in (t, d) order (whole waves of consecutive cells),
    some cells left out: the pivot equals the oracle's bit for bit (oracle on
    the row numbers, holes = NaN bits)."""
    import causal_softmax_attention_amd as csa
    m = _values(40 + T + D, T, D, dtype)
    t, d, x = tables.table(m.view(NP_BITS[dtype]))
    rng = np.random.default_rng(T * 100 + D)
    keep = rng.permutation(t.size)[: t.size - holes]
    if order == "ordered":
        keep = np.sort(keep)
    t, d, x = t[keep], d[keep], x[keep]
    note(f"table_to_matrix {dtype} {T}x{D} holes={holes} {order}")
    got = csa.attn_table_to_matrix(torch.from_numpy(t).to(DEV), torch.from_numpy(d).to(DEV),
                                   _to_dev(x, dtype), T, D)
    torch.cuda.synchronize()
    # the oracle pivots the row numbers (exact in float64); a cell it leaves
    # NaN is a hole, any other holds the bits of the row it names
    src = tables.matrix(t, d, np.arange(t.size, dtype=np.float64), T, D)
    hole = np.isnan(src)
    assert hole.sum() == holes
    gb = _bits(got, dtype)
    assert np.all(gb[hole] == NAN_BITS[dtype])
    assert np.array_equal(gb[~hole], x[src[~hole].astype(np.int64)])


@pytest.mark.parametrize("case,code", [("dup", 2), ("range", 1), ("both", 3)])
def test_table_to_matrix_status(case, code):
    """A cell named twice or a coordinate out of range: the oracle raises, the
    library sets the matching status bits (and the binding raises)."""
    import causal_softmax_attention_amd as csa
    T, D = 6, 5
    t, d, x = tables.table(np.arange(T * D, dtype=np.float32).reshape(T, D))
    if case in ("dup", "both"):
        d = d.copy(); d[7] = d[8]; t = t.copy(); t[7] = t[8]
    if case in ("range", "both"):
        t = t.copy(); t[3] = T
    with pytest.raises(ValueError):
        tables.matrix(t, d, x, T, D)
    note(f"table_to_matrix status {case}")
    td, dd, xd = (torch.from_numpy(a).to(DEV) for a in (t, d, x))
    _, status = csa.attn_table_to_matrix(td, dd, xd, T, D, check=False)
    torch.cuda.synchronize()
    assert int(status.item()) == code
    with pytest.raises(ValueError):
        csa.attn_table_to_matrix(td, dd, xd, T, D)
    # a clean call on the same status word clears it
    _, status2 = csa.attn_table_to_matrix(*(torch.from_numpy(a).to(DEV)
                                            for a in tables.table(np.ones((T, D), np.float32))),
                                          T, D, status=status, check=False)
    torch.cuda.synchronize()
    assert int(status2.item()) == 0


@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
def test_complete_tables_near_order(dtype):
    """T x D rows that are almost in (t, d) order: two rows swapped (a valid
    table: the pivot equals the oracle's bit for bit), and one row renamed to
    its neighbour's cell (a cell named twice and a hole: status 2)."""
    import causal_softmax_attention_amd as csa
    T, D = 37, 64
    m = _values(23, T, D, dtype)
    t, d, x = tables.table(m.view(NP_BITS[dtype]))
    for i, j in ((0, 1), (1000, 2367), (T * D - 2, T * D - 1)):
        p = np.arange(T * D)
        p[i], p[j] = p[j], p[i]
        note(f"near-ordered swap {i} {j} {dtype}")
        got = csa.attn_table_to_matrix(torch.from_numpy(t[p]).to(DEV),
                                       torch.from_numpy(d[p]).to(DEV), _to_dev(x[p], dtype), T, D)
        torch.cuda.synchronize()
        src = tables.matrix(t[p], d[p], np.arange(T * D, dtype=np.float64), T, D)
        assert np.array_equal(_bits(got, dtype).reshape(-1), x[p][src.reshape(-1).astype(np.int64)])
    for i in (0, 700, T * D - 1):
        t2, d2 = t.copy(), d.copy()
        k = i + 1 if i + 1 < T * D else i - 1
        t2[i], d2[i] = t[k], d[k]
        note(f"near-ordered duplicate at {i} {dtype}")
        _, status = csa.attn_table_to_matrix(torch.from_numpy(t2).to(DEV),
                                             torch.from_numpy(d2).to(DEV), _to_dev(x, dtype), T, D,
                                             check=False)
        torch.cuda.synchronize()
        assert int(status.item()) == 2


def test_duplicate_with_equal_values():
    """The same row (t, d, x) sent twice is still a cell named twice, and a
    duplicate whose second copy lies out of range is not: it is skipped."""
    import causal_softmax_attention_amd as csa
    T, D = 4, 3
    t, d, x = tables.table(np.arange(T * D, dtype=np.float32).reshape(T, D))
    for extra_t, code in ((t[5], 2), (T + 1, 1)):
        t2 = np.concatenate([t, [extra_t]])
        d2 = np.concatenate([d, d[5:6]])
        x2 = np.concatenate([x, x[5:6]])
        note(f"duplicate row, extra t={extra_t}")
        _, status = csa.attn_table_to_matrix(*(torch.from_numpy(a).to(DEV) for a in (t2, d2, x2)),
                                             T, D, check=False)
        torch.cuda.synchronize()
        assert int(status.item()) == code


@pytest.mark.parametrize("where", ["run", "lane"])
def test_duplicate_in_ordered_rows(where):
    """An ordered table with one 64-row stretch sent twice, starting on a
    64-row boundary ("run") or off it ("lane"): the repeated rows store into
    cells already staged, so fewer cells are marked than rows counted."""
    import causal_softmax_attention_amd as csa
    T, D = 8, 64
    t, d, x = tables.table(np.arange(T * D, dtype=np.float32).reshape(T, D))
    start = 64 if where == "run" else 70
    t2 = np.concatenate([t, t[start:start + 64]])
    d2 = np.concatenate([d, d[start:start + 64]])
    x2 = np.concatenate([x, x[start:start + 64]])
    with pytest.raises(ValueError):
        tables.matrix(t2, d2, x2, T, D)
    note(f"duplicate in ordered rows ({where})")
    _, status = csa.attn_table_to_matrix(*(torch.from_numpy(a).to(DEV) for a in (t2, d2, x2)),
                                         T, D, check=False)
    torch.cuda.synchronize()
    assert int(status.item()) == 2
    # the table without the repeat is clean and exact
    got = csa.attn_table_to_matrix(*(torch.from_numpy(a).to(DEV) for a in (t, d, x)), T, D)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), tables.matrix(t, d, x, T, D))


@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
@pytest.mark.parametrize("T,D,holes", [(300, 301, 0), (300, 301, 1000), (257, 512, 3)])
def test_table_to_matrix_binned(dtype, T, D, holes):
    """Tables of at least 65536 shuffled rows and cells take the binned form
    (rows sorted by cell block, one workgroup per block); the last block is
    partial when T*D is not a multiple of the block size."""
    import causal_softmax_attention_amd as csa
    m = _values(60 + T + D, T, D, dtype)
    t, d, x = tables.table(m.view(NP_BITS[dtype]))
    rng = np.random.default_rng(T + 7 * D)
    keep = rng.permutation(t.size)[: t.size - holes]
    t, d, x = t[keep], d[keep], x[keep]
    note(f"table_to_matrix binned {dtype} {T}x{D} holes={holes}")
    got = csa.attn_table_to_matrix(torch.from_numpy(t).to(DEV), torch.from_numpy(d).to(DEV),
                                   _to_dev(x, dtype), T, D)
    torch.cuda.synchronize()
    src = tables.matrix(t, d, np.arange(t.size, dtype=np.float64), T, D)
    hole = np.isnan(src)
    assert hole.sum() == holes
    gb = _bits(got, dtype)
    assert np.all(gb[hole] == NAN_BITS[dtype])
    assert np.array_equal(gb[~hole], x[src[~hole].astype(np.int64)])


@pytest.mark.parametrize("case,code", [("dup", 2), ("range", 1), ("both", 3), ("every row twice", 2)])
def test_table_to_matrix_binned_status(case, code):
    """The binned form's checks: a repeated cell (fewer marked cells than
    counted rows), rows out of range, and more rows in range than cells (the
    sorted rows would not fit: status 2 before the scatter)."""
    import causal_softmax_attention_amd as csa
    T, D = 256, 300
    t, d, x = tables.table(np.arange(T * D, dtype=np.float32).reshape(T, D))
    rng = np.random.default_rng(5)
    if case == "every row twice":
        t, d, x = (np.concatenate([a, a]) for a in (t, d, x))
    p = rng.permutation(t.size)
    t, d, x = t[p].copy(), d[p].copy(), x[p].copy()
    if case in ("dup", "both"):
        t[100], d[100] = t[60000], d[60000]
    if case in ("range", "both"):
        d[5] = -1
        t[7000] = T
    note(f"table_to_matrix binned status {case}")
    _, status = csa.attn_table_to_matrix(*(torch.from_numpy(a).to(DEV) for a in (t, d, x)),
                                         T, D, check=False)
    torch.cuda.synchronize()
    assert int(status.item()) == code


def test_table_workload_round_trip():
    """The bench workload: a 524288 x 64 bfloat16 matrix (16 heads of 32768
    tokens), its 2^25 rows in a seeded random order, pivoted back.  The whole
    result equals the original bit for bit; the oracle's pivot of a sampled
    stretch of the shuffled rows agrees cell by cell."""
    import causal_softmax_attention_amd as csa
    seed, T, D, dtype = inp.TABLE_WORKLOADS["table_16x32k"]
    m, perm = inp.table_matrix(seed, T, D, dtype)
    note(f"table workload {T}x{D}")
    md = _to_dev(m, dtype)
    t, d, x = csa.attn_matrix_to_table(md)
    p = torch.from_numpy(perm).to(DEV)
    got = csa.attn_table_to_matrix(t[p], d[p], x[p], T, D)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), md.view(torch.int16))
    # oracle on 20000 of the shuffled rows, pivoted into a T x D matrix of holes
    sel = perm[:20000]
    ts, ds = sel // D, sel % D
    want = tables.matrix(ts, ds, m.reshape(-1)[sel].astype(np.float64), T, D)
    gb = _bits(got, dtype).reshape(-1)
    assert np.array_equal(gb[sel], want.reshape(-1)[sel].astype(np.uint16))
