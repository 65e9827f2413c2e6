"""The C ABI on the host: the library loads, exports every entry point that
include/attn.h declares, and rejects invalid arguments before any launch.
No call here reaches a kernel (these run without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

import causal_softmax_attention_amd as csa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(csa.LIB_PATH):
        from causal_softmax_attention_amd import _build
        _build.build()
    return csa.lib()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^ATTN_API\s+[\w\s\*]*?\b(\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    assert declared_symbols() == sorted(["attn_causal_fwd", "attn_causal_bwd",
                                         "attn_causal_bwd_workspace_bytes",
                                         "attn_causal_bwd_noalloc", "attn_fwd",
                                         "attn_bwd", "attn_bwd_workspace_bytes",
                                         "attn_fwd_train", "attn_bwd_from_fwd",
                                         "nw_gauss_average", "attn_set_kernel_timer",
                                         "attn_last_error", "attn_matrix_to_table",
                                         "attn_table_workspace_bytes", "attn_table_to_matrix",
                                         "attn_qkv_project", "attn_fwd_seg",
                                         "attn_bwd_seg"])


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", csa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for sym in declared_symbols():
        assert sym in exported, sym
        assert hasattr(L, sym)
    # nothing else leaks out of the library
    assert exported == set(declared_symbols())


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "attn.h"\n'
                   'int main(void){return ATTN_OK + ATTN_BF16 + ATTN_MASK_WINDOW;}\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), "-c",
                    str(src), "-o", str(tmp_path / "t.o")], check=True)


P = ctypes.c_void_p(0x1000)  # a non-null, aligned dummy: never dereferenced on these paths


def fwd(L, dtype=2, B=1, H=1, N=16, D=64, scale=0.125, q=P, k=P, v=P, o=None, lse=None):
    o = ctypes.c_void_p(0x100000) if o is None else o
    lse = ctypes.c_void_p(0x200000) if lse is None else lse
    return L.attn_causal_fwd(dtype, B, H, N, D, scale, q, k, v, o, lse, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), csa.ATTN_EINVAL),
    (dict(B=0), csa.ATTN_EINVAL),
    (dict(H=-1), csa.ATTN_EINVAL),
    (dict(N=0), csa.ATTN_EINVAL),
    (dict(D=32), csa.ATTN_EUNSUPPORTED),
    (dict(D=128), csa.ATTN_EUNSUPPORTED),
    (dict(scale=0.0), csa.ATTN_EINVAL),
    (dict(scale=float("nan")), csa.ATTN_EINVAL),
    (dict(scale=float("inf")), csa.ATTN_EINVAL),
    (dict(q=ctypes.c_void_p(0)), csa.ATTN_EINVAL),
    (dict(lse=ctypes.c_void_p(0)), csa.ATTN_EINVAL),
    (dict(k=ctypes.c_void_p(0x1004)), csa.ATTN_EINVAL),          # misaligned
    (dict(o=P), csa.ATTN_EINVAL),                                 # o aliases q
    (dict(N=1 << 25), csa.ATTN_EINVAL),
])
def test_fwd_rejects(L, kw, code):
    assert fwd(L, **kw) == code
    assert csa.attn_last_error() != ""


def test_workspace_bytes(L):
    for dt, acc in ((0, 8), (1, 4), (2, 4)):
        n = L.attn_causal_bwd_workspace_bytes(dt, 2, 3, 100, 64)
        assert n >= 2 * 3 * 100 * acc          # at least delta, one value per row
    assert L.attn_causal_bwd_workspace_bytes(2, 1, 1, 16, 32) == 0
    assert L.attn_causal_bwd_workspace_bytes(9, 1, 1, 16, 64) == 0


def bwd(L, ws_bytes=None, **over):
    a = dict(dtype=2, B=1, H=1, N=16, D=64, scale=0.125)
    a.update({k: v for k, v in over.items() if k in a})
    ptrs = {name: ctypes.c_void_p(0x100000 * (i + 1)) for i, name in
            enumerate(["q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "ws"])}
    ptrs.update({k: v for k, v in over.items() if k in ptrs})
    need = L.attn_causal_bwd_workspace_bytes(a["dtype"], a["B"], a["H"], a["N"], 64)
    return L.attn_causal_bwd(a["dtype"], a["B"], a["H"], a["N"], a["D"], a["scale"],
                             ptrs["q"], ptrs["k"], ptrs["v"], ptrs["o"], ptrs["dout"],
                             ptrs["lse"], ptrs["dq"], ptrs["dk"], ptrs["dv"], ptrs["ws"],
                             need if ws_bytes is None else ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), csa.ATTN_EINVAL),
    (dict(N=0), csa.ATTN_EINVAL),
    (dict(D=16), csa.ATTN_EUNSUPPORTED),
    (dict(scale=-1.0), csa.ATTN_EINVAL),
    (dict(dk=ctypes.c_void_p(0)), csa.ATTN_EINVAL),
    (dict(ws=ctypes.c_void_p(0)), csa.ATTN_EINVAL),
    (dict(ws_bytes=8), csa.ATTN_EINVAL),
    (dict(dq=ctypes.c_void_p(0x100000)), csa.ATTN_EINVAL),      # dq aliases q
    (dict(dv=ctypes.c_void_p(0x800000)), csa.ATTN_EINVAL),      # dv aliases dk
    (dict(dq=ctypes.c_void_p(0x700008)), csa.ATTN_EINVAL),      # misaligned
])
def test_bwd_rejects(L, kw, code):
    assert bwd(L, **kw) == code
    assert csa.attn_last_error() != ""


def mfwd(L, mask, window, **kw):
    a = dict(dtype=2, B=1, H=1, N=16, D=64, scale=0.125)
    a.update(kw)
    return L.attn_fwd(a["dtype"], a["B"], a["H"], a["N"], a["D"], a["scale"], mask, window, P,
                      P, P, ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000), None)


def mbwd(L, mask, window, **kw):
    a = dict(dtype=2, B=1, H=1, N=16, D=64, scale=0.125)
    a.update(kw)
    p = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(10)]
    need = L.attn_bwd_workspace_bytes(2, 1, 1, 16, 64)
    return L.attn_bwd(a["dtype"], a["B"], a["H"], a["N"], a["D"], a["scale"], mask, window,
                      *p, need, None)


@pytest.mark.parametrize("mask,window", [(3, 0), (-1, 0), (csa.ATTN_MASK_WINDOW, 0),
                                         (csa.ATTN_MASK_WINDOW, -5)])
def test_mask_rejects(L, mask, window):
    """An unknown mask kind, or a window narrower than one key, is refused before
    any launch, by both passes."""
    assert mfwd(L, mask, window) == csa.ATTN_EINVAL
    assert "mask" in csa.attn_last_error() or "window" in csa.attn_last_error()
    assert mbwd(L, mask, window) == csa.ATTN_EINVAL


def test_masked_entry_points_check_sizes_first(L):
    for m in (csa.ATTN_MASK_CAUSAL, csa.ATTN_MASK_FULL, csa.ATTN_MASK_WINDOW):
        assert mfwd(L, m, 4, D=32) == csa.ATTN_EUNSUPPORTED
        assert mfwd(L, m, 4, N=0) == csa.ATTN_EINVAL
        assert mbwd(L, m, 4, scale=0.0) == csa.ATTN_EINVAL
    assert L.attn_bwd_workspace_bytes(2, 2, 3, 100, 64) == \
        L.attn_causal_bwd_workspace_bytes(2, 2, 3, 100, 64)


def sfwd(L, seg=0x900000, **kw):
    a = dict(dtype=2, B=1, H=1, N=16, D=64, scale=0.125, mask=0, window=0,
             o=0x100000, lse=0x200000)
    a.update(kw)
    return L.attn_fwd_seg(a["dtype"], a["B"], a["H"], a["N"], a["D"], a["scale"], a["mask"],
                          a["window"], ctypes.c_void_p(seg), P, P, P, ctypes.c_void_p(a["o"]),
                          ctypes.c_void_p(a["lse"]), None)


def sbwd(L, seg=0xb00000, **kw):
    a = dict(dtype=2, B=1, H=1, N=16, D=64, scale=0.125, mask=0, window=0)
    a.update(kw)
    p = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(10)]
    if "dq" in kw:
        p[6] = ctypes.c_void_p(kw["dq"])
    need = L.attn_bwd_workspace_bytes(2, 1, 1, 16, 64)
    return L.attn_bwd_seg(a["dtype"], a["B"], a["H"], a["N"], a["D"], a["scale"], a["mask"],
                          a["window"], ctypes.c_void_p(seg), *p, need, None)


@pytest.mark.parametrize("kw,code", [
    (dict(seg=0), csa.ATTN_EINVAL),                      # null segment ids
    (dict(seg=0x900002), csa.ATTN_EINVAL),               # not 4-byte aligned
    (dict(seg=0x100010), csa.ATTN_EINVAL),               # o overlaps the ids
    (dict(seg=0x200000), csa.ATTN_EINVAL),               # lse overlaps the ids
    (dict(D=32), csa.ATTN_EUNSUPPORTED),
    (dict(mask=2, window=0), csa.ATTN_EINVAL),
    (dict(mask=9), csa.ATTN_EINVAL),
])
def test_fwd_seg_rejects(L, kw, code):
    assert sfwd(L, **kw) == code
    assert csa.attn_last_error() != ""


@pytest.mark.parametrize("kw,code", [
    (dict(seg=0), csa.ATTN_EINVAL),
    (dict(seg=0xb00001), csa.ATTN_EINVAL),
    (dict(seg=0x700000), csa.ATTN_EINVAL),               # dq overlaps the ids
    (dict(seg=0xa00000), csa.ATTN_EINVAL),               # the workspace overlaps the ids
    (dict(N=0), csa.ATTN_EINVAL),
    (dict(mask=2, window=-1), csa.ATTN_EINVAL),
])
def test_bwd_seg_rejects(L, kw, code):
    assert sbwd(L, **kw) == code
    assert csa.attn_last_error() != ""


def train_fwd(L, ws_bytes=None, loss=0x900000, ws=0x800000, **kw):
    a = dict(dtype=2, B=1, H=1, N=16, D=64, scale=0.125, mask=0, window=0)
    a.update(kw)
    need = L.attn_bwd_workspace_bytes(a["dtype"], 1, 1, 16, 64)
    return L.attn_fwd_train(a["dtype"], a["B"], a["H"], a["N"], a["D"], a["scale"], a["mask"],
                            a["window"], P, P, P, ctypes.c_void_p(0x100000),
                            ctypes.c_void_p(0x200000), ctypes.c_void_p(ws),
                            need if ws_bytes is None else ws_bytes, ctypes.c_void_p(loss), None)


@pytest.mark.parametrize("kw,code", [
    (dict(loss=0), csa.ATTN_EINVAL),                     # null loss
    (dict(loss=0x900004), csa.ATTN_EINVAL),              # loss not 8-byte aligned
    (dict(ws=0), csa.ATTN_EINVAL),                       # null workspace
    (dict(ws_bytes=64), csa.ATTN_EINVAL),                # short workspace
    (dict(ws=0x100000), csa.ATTN_EINVAL),                # workspace aliases o
    (dict(loss=0x800000), csa.ATTN_EINVAL),              # loss inside the workspace
    (dict(D=32), csa.ATTN_EUNSUPPORTED),
    (dict(mask=2, window=0), csa.ATTN_EINVAL),
])
def test_fwd_train_rejects(L, kw, code):
    assert train_fwd(L, **kw) == code
    assert csa.attn_last_error() != ""


def test_bwd_from_fwd_rejects(L):
    p = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(9)]
    need = L.attn_bwd_workspace_bytes(2, 1, 1, 16, 64)
    call = lambda ws_bytes=need, ws=p[8], **kw: L.attn_bwd_from_fwd(
        2, 1, 1, kw.get("N", 16), 64, 0.125, 0, 0, *p[:8], ws, ws_bytes, None)
    assert call(ws_bytes=need - 1) == csa.ATTN_EINVAL
    assert call(ws=ctypes.c_void_p(0)) == csa.ATTN_EINVAL
    assert call(N=0) == csa.ATTN_EINVAL


def test_nw_rejects(L):
    p = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(6)]
    call = lambda nt=8, ns=8, denom=0.25, ptrs=p: L.nw_gauss_average(
        nt, ptrs[0], ptrs[1], ns, ptrs[2], ptrs[3], ptrs[4], denom, ptrs[5], None)
    assert call(nt=0) == csa.ATTN_EINVAL
    assert call(ns=0) == csa.ATTN_EINVAL
    assert call(denom=0.0) == csa.ATTN_EINVAL
    assert call(denom=float("inf")) == csa.ATTN_EINVAL
    assert call(ptrs=p[:5] + [ctypes.c_void_p(0)]) == csa.ATTN_EINVAL
    assert call(ptrs=p[:5] + [ctypes.c_void_p(0x100002)]) == csa.ATTN_EINVAL
    assert call(ptrs=p[:5] + [p[0]]) == csa.ATTN_EINVAL     # out aliases tx


def test_timer_hook(L):
    assert L.attn_set_kernel_timer(0, P, None) == csa.ATTN_EINVAL
    assert L.attn_set_kernel_timer(7, None, None) == csa.ATTN_EINVAL
    assert L.attn_set_kernel_timer(-1, None, None) == csa.ATTN_EINVAL
    for slot in range(7):
        assert L.attn_set_kernel_timer(slot, None, None) == csa.ATTN_OK
    assert csa.attn_last_error() == ""


def _addr(i):
    return ctypes.c_void_p(0x1000000 * (i + 1))


def test_matrix_to_table_rejects(L):
    m, t, d, x = (_addr(i) for i in range(4))
    call = lambda dtype=2, T=4, D=8, m=m, t=t, d=d, x=x: L.attn_matrix_to_table(
        dtype, T, D, m, t, d, x, None)
    assert call(dtype=5) == csa.ATTN_EINVAL
    assert call(T=0) == csa.ATTN_EINVAL
    assert call(D=-2) == csa.ATTN_EINVAL
    assert call(T=1 << 30, D=1 << 20) == csa.ATTN_EINVAL          # over 2^40 cells
    assert call(t=ctypes.c_void_p(0)) == csa.ATTN_EINVAL
    assert call(d=ctypes.c_void_p(0x1000008)) == csa.ATTN_EINVAL  # not 16-byte aligned
    assert call(x=ctypes.c_void_p(0x3000002)) == csa.ATTN_EINVAL  # not 16-byte aligned
    assert call(x=t) == csa.ATTN_EINVAL                           # outputs overlap
    assert call(t=m) == csa.ATTN_EINVAL                           # output overlaps the matrix


def test_table_workspace_bytes(L):
    # 256 bytes of counters, then a staging word per cell (bf16 4, f32 8, f64 16
    # bytes) in whole 16-byte stores
    assert L.attn_table_workspace_bytes(csa.ATTN_BF16, 4, 8) == 256 + 128
    assert L.attn_table_workspace_bytes(csa.ATTN_BF16, 3, 1) == 256 + 16
    assert L.attn_table_workspace_bytes(csa.ATTN_F32, 1000, 64) == 256 + 1000 * 64 * 8
    assert L.attn_table_workspace_bytes(csa.ATTN_F64, 1000, 64) == 256 + 1000 * 64 * 16
    assert L.attn_table_workspace_bytes(csa.ATTN_BF16, 0, 8) == 0
    assert L.attn_table_workspace_bytes(csa.ATTN_BF16, 1 << 30, 1 << 20) == 0
    assert L.attn_table_workspace_bytes(9, 4, 8) == 0
    assert "dtype" in csa.attn_last_error()


def test_table_to_matrix_rejects(L):
    t, d, x, m, st, ws = (_addr(i) for i in range(6))
    need = L.attn_table_workspace_bytes(csa.ATTN_F32, 4, 8)
    call = lambda dtype=1, rows=32, t=t, d=d, x=x, T=4, D=8, m=m, st=st, ws=ws, wb=need: \
        L.attn_table_to_matrix(dtype, rows, t, d, x, T, D, m, st, ws, wb, None)
    assert call(dtype=9) == csa.ATTN_EINVAL
    assert call(rows=0) == csa.ATTN_EINVAL
    assert call(T=0) == csa.ATTN_EINVAL
    assert call(wb=need - 1) == csa.ATTN_EINVAL
    assert call(st=ctypes.c_void_p(0)) == csa.ATTN_EINVAL
    assert call(ws=ctypes.c_void_p(0x6000008)) == csa.ATTN_EINVAL  # workspace not 16-aligned
    assert call(m=ctypes.c_void_p(0x5000004)) == csa.ATTN_EINVAL   # matrix not 16-aligned
    assert call(st=ctypes.c_void_p(0x5000002)) == csa.ATTN_EINVAL  # status misaligned
    assert call(m=x) == csa.ATTN_EINVAL                            # matrix aliases x
    assert call(ws=t) == csa.ATTN_EINVAL                           # workspace aliases t
    assert call(st=d) == csa.ATTN_EINVAL                           # status aliases d


def test_qkv_project_rejects(L):
    x, wq, wk, wv, q, k, v = (_addr(i) for i in range(7))
    call = lambda dtype=2, B=1, N=16, Dm=64, H=1, ptrs=(x, wq, wk, wv, q, k, v): \
        L.attn_qkv_project(dtype, B, N, Dm, H, *ptrs, None)
    assert call(dtype=3) == csa.ATTN_EINVAL
    assert call(B=0) == csa.ATTN_EINVAL
    assert call(Dm=0) == csa.ATTN_EINVAL
    assert call(H=70000) == csa.ATTN_EINVAL
    assert call(B=1 << 20, N=1 << 12) == csa.ATTN_EINVAL            # B*N >= 2^31
    assert call(ptrs=(x, wq, wk, wv, q, k, ctypes.c_void_p(0))) == csa.ATTN_EINVAL
    assert call(ptrs=(x, wq, wk, ctypes.c_void_p(0x4000008), q, k, v)) == csa.ATTN_EINVAL
    assert call(ptrs=(x, wq, wk, wv, x, k, v)) == csa.ATTN_EINVAL   # q aliases x
    assert call(ptrs=(x, wq, wk, wv, q, q, v)) == csa.ATTN_EINVAL   # k overlaps q
    assert "overlap" in csa.attn_last_error()


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    """With no built library every entry point raises (there is no fallback
    path): the binding's loader names the missing file."""
    monkeypatch.setattr(csa, "LIB_PATH", str(tmp_path / "libattn.so"))
    monkeypatch.setattr(csa, "_LIB", None)
    with pytest.raises(RuntimeError, match="is missing"):
        csa.lib()
    with pytest.raises(RuntimeError, match="is missing"):
        csa.attn_table_workspace_bytes(csa.ATTN_BF16, 4, 4)


@pytest.mark.parametrize("B,H,N,ok", [
    (1 << 14, 1 << 10, 128, False),   # 2^24 heads of 128 tokens: 2^26 workgroups of 32 rows
    (1 << 12, 1 << 10, 512, False),   # 2^22 heads x 16 blocks = 2^26
    (1 << 11, 1 << 10, 256, False),   # 2^21 heads x 8 blocks = 2^24 (the first size refused)
    (1 << 11, 1 << 10, 224, True),    # 2^21 heads x 7 blocks < 2^24
    (1, 1, 1 << 24, True),            # the longest head: 2^19 blocks
])
def test_grid_limit(L, B, H, N, ok):
    """A launch over heads x 32-row blocks must stay below 2^32 work-items: the
    size check refuses it (ATTN_EINVAL) instead of the launch failing.  The
    accepted sizes are checked through the workspace query, which runs the
    same size check and launches nothing."""
    if ok:
        assert L.attn_causal_bwd_workspace_bytes(2, B, H, N, 64) > 0, csa.attn_last_error()
    else:
        # refused by the size check, before the dummy pointers are looked at
        assert fwd(L, B=B, H=H, N=N) == csa.ATTN_EINVAL
        assert "workgroups" in csa.attn_last_error()
        assert L.attn_causal_bwd_workspace_bytes(2, B, H, N, 64) == 0


# ---- the binding validates every tensor, outputs included (the C side sees
# only pointers, so a short or mistyped output would be written past its end)

import torch  # noqa: E402


def _qkv(dtype=torch.bfloat16, shape=(1, 2, 5, 64)):
    return [torch.zeros(shape, dtype=dtype) for _ in range(3)]


def test_binding_requires_device_tensors():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="device tensor"):
        csa.attn_causal_fwd(q, k, v)
    with pytest.raises(ValueError, match="device tensor"):
        csa.attn_causal_bwd(q, k, v, q, q, torch.zeros(1, 2, 5))


@pytest.mark.parametrize("dtype,lse_dtype", [(torch.bfloat16, torch.float32),
                                              (torch.float32, torch.float32),
                                              (torch.float64, torch.float64)])
def test_binding_accepts_matching_outputs(dtype, lse_dtype):
    q, k, v = _qkv(dtype)
    shape, o, lse = csa._fwd_args(q, k, v, torch.empty_like(q), torch.empty(1, 2, 5, dtype=lse_dtype))
    assert tuple(shape) == (1, 2, 5, 64)
    csa._bwd_args(q, k, v, o, o, lse, torch.empty_like(q), torch.empty_like(q),
                  torch.empty_like(q), torch.empty(64, dtype=torch.uint8))
    csa._train_args(q, k, v, o, lse, torch.empty(64, dtype=torch.uint8),
                    torch.empty(1, dtype=torch.float64))


@pytest.mark.parametrize("case", ["o short", "o dtype", "o strided", "lse dtype f64 path",
                                  "lse short", "lse float64 for bf16", "lse strided"])
def test_binding_rejects_bad_forward_outputs(case):
    dtype = torch.float64 if "f64 path" in case else torch.bfloat16
    q, k, v = _qkv(dtype)
    o = torch.empty_like(q)
    lse = torch.empty(1, 2, 5, dtype=torch.float64 if dtype == torch.float64 else torch.float32)
    if case == "o short":
        o = torch.empty(1, 2, 4, 64, dtype=dtype)
    elif case == "o dtype":
        o = torch.empty(1, 2, 5, 64, dtype=torch.float32)
    elif case == "o strided":
        o = torch.empty(1, 2, 64, 5, dtype=dtype).transpose(2, 3)
    elif case == "lse dtype f64 path":
        lse = torch.empty(1, 2, 5, dtype=torch.float32)
    elif case == "lse short":
        lse = torch.empty(1, 2, 4)
    elif case == "lse float64 for bf16":
        lse = torch.empty(1, 2, 5, dtype=torch.float64)
    elif case == "lse strided":
        lse = torch.empty(1, 5, 2).transpose(1, 2)
    with pytest.raises(ValueError):
        csa._fwd_args(q, k, v, o, lse)


@pytest.mark.parametrize("case", ["dq short", "dk dtype", "dv strided", "lse short", "lse dtype",
                                  "dout shape"])
def test_binding_rejects_bad_backward_tensors(case):
    q, k, v = _qkv()
    o, dout = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty(1, 2, 5)
    g = {n: torch.empty_like(q) for n in ("dq", "dk", "dv")}
    if case == "dq short":
        g["dq"] = torch.empty(1, 2, 5, 32, dtype=q.dtype)
    elif case == "dk dtype":
        g["dk"] = torch.empty(1, 2, 5, 64, dtype=torch.float32)
    elif case == "dv strided":
        g["dv"] = torch.empty(1, 2, 64, 5, dtype=q.dtype).transpose(2, 3)
    elif case == "lse short":
        lse = torch.empty(1, 2, 3)
    elif case == "lse dtype":
        lse = torch.empty(1, 2, 5, dtype=torch.float64)
    elif case == "dout shape":
        dout = torch.empty(1, 2, 6, 64, dtype=q.dtype)
    with pytest.raises(ValueError):
        csa._bwd_args(q, k, v, o, dout, lse, g["dq"], g["dk"], g["dv"],
                      torch.empty(64, dtype=torch.uint8))


@pytest.mark.parametrize("case", ["ok", "dtype", "shape", "heads axis", "strided"])
def test_binding_checks_segment_ids(case):
    q, _, _ = _qkv(shape=(2, 3, 5, 64))
    B, _, N, _ = q.shape
    seg = {"ok": torch.zeros(B, N, dtype=torch.int32),
           "dtype": torch.zeros(B, N, dtype=torch.int64),
           "shape": torch.zeros(B, N + 1, dtype=torch.int32),
           "heads axis": torch.zeros(B, 2, N, dtype=torch.int32),
           "strided": torch.zeros(N, B, dtype=torch.int32).t()}[case]
    if case == "ok":
        csa._check_seg(seg, q)
    else:
        with pytest.raises(ValueError, match="seg"):
            csa._check_seg(seg, q)


@pytest.mark.parametrize("loss", [torch.empty(1, dtype=torch.float32), torch.empty(2, dtype=torch.float64),
                                  torch.empty(0, dtype=torch.float64)])
def test_binding_rejects_bad_loss(loss):
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="loss"):
        csa._train_args(q, k, v, None, None, torch.empty(64, dtype=torch.uint8), loss)


def test_noalloc_refuses_sizes_past_its_scratch(L):
    """attn_causal_bwd_noalloc checks sizes, then whether the workspace fits
    the static scratch (ATTN_NOALLOC_SCRATCH_BYTES = 16 MiB), before it looks
    at the device or the pointers."""
    text = open(HEADER).read()
    assert "#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)" in text
    assert csa.NOALLOC_SCRATCH_BYTES == 16 << 20
    for dtype, rows in ((csa.ATTN_BF16, 2096896), (csa.ATTN_F64, 2096896), (csa.ATTN_F32, 4193792)):
        assert L.attn_causal_bwd_workspace_bytes(dtype, 1, 1, rows, 64) <= csa.NOALLOC_SCRATCH_BYTES
        assert L.attn_causal_bwd_workspace_bytes(dtype, 1, 1, rows + 32, 64) > csa.NOALLOC_SCRATCH_BYTES
        rc = L.attn_causal_bwd_noalloc(dtype, 1, 1, rows + 32, 64, 0.125, *([None] * 9), None)
        assert rc == csa.ATTN_EINVAL and "static scratch" in csa.attn_last_error()
    assert L.attn_causal_bwd_noalloc(csa.ATTN_BF16, 1, 1, 16, 32, 0.125, *([None] * 9), None) \
        == csa.ATTN_EUNSUPPORTED
