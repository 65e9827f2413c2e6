"""Causal softmax attention (D = 64) and the Nadaraya-Watson control on MI355X,
with the steps before it: the long-table <-> matrix adapter and the Q / K / V
input projections.

A thin ctypes binding over the C ABI in ``include/attn.h`` (``libattn.so``,
built in-tree by ``python -m causal_softmax_attention_amd._build``).  The
functions here carry the C entry points' names and only marshal arguments:
torch supplies device memory and the current stream; every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the
library is missing or fails, these functions raise.
"""
from __future__ import annotations

import ctypes
import os

ATTN_F64, ATTN_F32, ATTN_BF16 = 0, 1, 2
ATTN_MASK_CAUSAL, ATTN_MASK_FULL, ATTN_MASK_WINDOW = 0, 1, 2
MASKS = {"causal": ATTN_MASK_CAUSAL, "full": ATTN_MASK_FULL, "window": ATTN_MASK_WINDOW}
ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_EHIP = 0, 1, 2, 3
DEFAULT_SCALE = 0.125
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

_LIB = None


class AttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m causal_softmax_attention_amd._build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
        L.attn_causal_fwd.argtypes = [ctypes.c_int, i64, i64, i64, i64, ctypes.c_double,
                                      vp, vp, vp, vp, vp, vp]
        L.attn_causal_fwd.restype = ctypes.c_int
        L.attn_causal_bwd_workspace_bytes.argtypes = [ctypes.c_int, i64, i64, i64, i64]
        L.attn_causal_bwd_workspace_bytes.restype = sz
        L.attn_causal_bwd.argtypes = [ctypes.c_int, i64, i64, i64, i64, ctypes.c_double,
                                      vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.attn_causal_bwd.restype = ctypes.c_int
        L.attn_causal_bwd_noalloc.argtypes = [ctypes.c_int, i64, i64, i64, i64, ctypes.c_double,
                                              vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.attn_causal_bwd_noalloc.restype = ctypes.c_int
        L.attn_fwd.argtypes = [ctypes.c_int, i64, i64, i64, i64, ctypes.c_double, ctypes.c_int,
                               i64, vp, vp, vp, vp, vp, vp]
        L.attn_fwd.restype = ctypes.c_int
        L.attn_bwd_workspace_bytes.argtypes = [ctypes.c_int, i64, i64, i64, i64]
        L.attn_bwd_workspace_bytes.restype = sz
        L.attn_bwd.argtypes = [ctypes.c_int, i64, i64, i64, i64, ctypes.c_double, ctypes.c_int,
                               i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.attn_bwd.restype = ctypes.c_int
        L.attn_fwd_seg.argtypes = [ctypes.c_int, i64, i64, i64, i64, ctypes.c_double,
                                   ctypes.c_int, i64] + [vp] * 7
        L.attn_fwd_seg.restype = ctypes.c_int
        L.attn_bwd_seg.argtypes = [ctypes.c_int, i64, i64, i64, i64, ctypes.c_double,
                                   ctypes.c_int, i64] + [vp] * 11 + [ctypes.c_size_t, vp]
        L.attn_bwd_seg.restype = ctypes.c_int
        L.attn_fwd_train.argtypes = [ctypes.c_int, i64, i64, i64, i64, ctypes.c_double,
                                     ctypes.c_int, i64, vp, vp, vp, vp, vp, vp, sz, vp, vp]
        L.attn_fwd_train.restype = ctypes.c_int
        L.attn_bwd_from_fwd.argtypes = [ctypes.c_int, i64, i64, i64, i64, ctypes.c_double,
                                        ctypes.c_int, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                        sz, vp]
        L.attn_bwd_from_fwd.restype = ctypes.c_int
        L.nw_gauss_average.argtypes = [i64, vp, vp, i64, vp, vp, vp, ctypes.c_float, vp, vp]
        L.nw_gauss_average.restype = ctypes.c_int
        L.attn_matrix_to_table.argtypes = [ctypes.c_int, i64, i64, vp, vp, vp, vp, vp]
        L.attn_matrix_to_table.restype = ctypes.c_int
        L.attn_table_workspace_bytes.argtypes = [ctypes.c_int, i64, i64]
        L.attn_table_workspace_bytes.restype = sz
        L.attn_table_to_matrix.argtypes = [ctypes.c_int, i64, vp, vp, vp, i64, i64, vp, vp, vp,
                                           sz, vp]
        L.attn_table_to_matrix.restype = ctypes.c_int
        L.attn_qkv_project.argtypes = [ctypes.c_int, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp,
                                       vp, vp]
        L.attn_qkv_project.restype = ctypes.c_int
        L.attn_set_kernel_timer.argtypes = [ctypes.c_int, vp, vp]
        L.attn_set_kernel_timer.restype = ctypes.c_int
        L.attn_last_error.argtypes = []
        L.attn_last_error.restype = ctypes.c_char_p
        _LIB = L
    return _LIB


def attn_last_error() -> str:
    return lib().attn_last_error().decode()


def _check(rc: int):
    if rc != ATTN_OK:
        raise AttnError(rc, attn_last_error())


def _dtype_code(t) -> int:
    import torch
    codes = {torch.float64: ATTN_F64, torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _stream(t, stream):
    import torch
    s = torch.cuda.current_stream(t.device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _on_gpu(t, name):
    """The public entry points run on device tensors only (no host fallback)."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _bhnd(t, name):
    if t.dim() != 4 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous [B, H, N, D] tensor")
    return t.shape


def _same(t, ref, name, what):
    """t must be a contiguous tensor of ref's shape, dtype and device."""
    if (tuple(t.shape) != tuple(ref.shape) or t.dtype != ref.dtype or t.device != ref.device
            or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous tensor matching {what} in shape, "
                         "dtype and device")


def _lse_dtype(q):
    import torch
    return torch.float64 if q.dtype == torch.float64 else torch.float32


def _check_lse(lse, q):
    B, H, N, _ = q.shape
    if (tuple(lse.shape) != (B, H, N) or lse.dtype != _lse_dtype(q) or lse.device != q.device
            or not lse.is_contiguous()):
        raise ValueError(f"lse must be a contiguous [B, H, N] {_lse_dtype(q)} tensor on q's device")


def _check_buffer(ws, q, name="workspace"):
    if ws.device != q.device or not ws.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor on q's device")


def _mask_code(mask) -> int:
    if mask not in MASKS:
        raise ValueError(f"mask must be one of {sorted(MASKS)}")
    return MASKS[mask]


def _fwd_args(q, k, v, o, lse):
    """Validate the forward's tensors (outputs included: the C side sees only
    pointers, so a short or mistyped output would be written past its end) and
    allocate the outputs not given."""
    import torch
    B, H, N, D = _bhnd(q, "q")
    _dtype_code(q)
    for name, t in (("k", k), ("v", v)):
        _same(t, q, name, "q")
    if o is None:
        o = torch.empty_like(q)
    _same(o, q, "o", "q")
    if lse is None:
        lse = torch.empty((B, H, N), dtype=_lse_dtype(q), device=q.device)
    _check_lse(lse, q)
    return (B, H, N, D), o, lse


def attn_causal_fwd(q, k, v, scale: float = DEFAULT_SCALE, o=None, lse=None, stream=None):
    """Forward pass; returns (o, lse).  q, k, v: [B, H, N, 64] float64/float32/bfloat16."""
    _on_gpu(q, "q")
    (B, H, N, D), o, lse = _fwd_args(q, k, v, o, lse)
    _check(lib().attn_causal_fwd(_dtype_code(q), B, H, N, D, float(scale), _ptr(q), _ptr(k),
                                 _ptr(v), _ptr(o), _ptr(lse), _stream(q, stream)))
    return o, lse


def attn_fwd(q, k, v, scale: float = DEFAULT_SCALE, mask: str = "causal", window: int = 0,
             o=None, lse=None, stream=None):
    """Forward pass under a join predicate ("causal", "full" or "window" of
    `window` keys); returns (o, lse)."""
    _on_gpu(q, "q")
    (B, H, N, D), o, lse = _fwd_args(q, k, v, o, lse)
    _check(lib().attn_fwd(_dtype_code(q), B, H, N, D, float(scale), _mask_code(mask), int(window),
                          _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _stream(q, stream)))
    return o, lse


def attn_causal_bwd_workspace_bytes(dtype_code: int, B: int, H: int, N: int, D: int = 64) -> int:
    return int(lib().attn_causal_bwd_workspace_bytes(dtype_code, B, H, N, D))


def _bwd_args(q, k, v, o, dout, lse, dq, dk, dv, workspace, need=None, own_workspace=True):
    """Validate the backward's tensors (lse and the gradients included) and
    allocate the outputs and workspace not given.  ``need`` is the workspace
    size in bytes (the library's own figure when None); with
    ``own_workspace=False`` there is none (returned as None)."""
    import torch
    B, H, N, D = _bhnd(q, "q")
    code = _dtype_code(q)
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        _same(t, q, name, "q")
    _check_lse(lse, q)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _same(t, q, name, "q")
    if not own_workspace:
        return (code, B, H, N, D), dq, dk, dv, None
    if workspace is None:
        if need is None:
            need = attn_causal_bwd_workspace_bytes(code, B, H, N, D)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_buffer(workspace, q)
    return (code, B, H, N, D), dq, dk, dv, workspace


def attn_causal_bwd(q, k, v, o, dout, lse, scale: float = DEFAULT_SCALE, dq=None, dk=None,
                    dv=None, workspace=None, stream=None):
    """Backward pass; returns (dq, dk, dv).  Pass dout = o for the loss sum(o^2)/2."""
    _on_gpu(q, "q")
    (code, B, H, N, D), dq, dk, dv, ws = _bwd_args(q, k, v, o, dout, lse, dq, dk, dv, workspace)
    _check(lib().attn_causal_bwd(code, B, H, N, D, float(scale), _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                                 _ptr(ws), ws.numel() * ws.element_size(), _stream(q, stream)))
    return dq, dk, dv


NOALLOC_SCRATCH_BYTES = 16 << 20  # ATTN_NOALLOC_SCRATCH_BYTES of include/attn.h


def attn_causal_bwd_noalloc(q, k, v, o, dout, lse, scale: float = DEFAULT_SCALE, dq=None,
                            dk=None, dv=None, stream=None):
    """attn_causal_bwd with the library's static per-GPU scratch as workspace
    (the C call allocates nothing; outputs not given are allocated here by
    torch).  Calls that can overlap on one GPU race on that scratch."""
    _on_gpu(q, "q")
    (code, B, H, N, D), dq, dk, dv, _ = _bwd_args(q, k, v, o, dout, lse, dq, dk, dv, None,
                                                  own_workspace=False)
    _check(lib().attn_causal_bwd_noalloc(code, B, H, N, D, float(scale), _ptr(q), _ptr(k),
                                         _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                                         _ptr(dk), _ptr(dv), _stream(q, stream)))
    return dq, dk, dv


def attn_bwd_workspace_bytes(dtype_code: int, B: int, H: int, N: int, D: int = 64) -> int:
    return int(lib().attn_bwd_workspace_bytes(dtype_code, B, H, N, D))


def attn_bwd(q, k, v, o, dout, lse, scale: float = DEFAULT_SCALE, mask: str = "causal",
             window: int = 0, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Backward pass under a join predicate (as attn_fwd); returns (dq, dk, dv)."""
    _on_gpu(q, "q")
    (code, B, H, N, D), dq, dk, dv, ws = _bwd_args(q, k, v, o, dout, lse, dq, dk, dv, workspace)
    _check(lib().attn_bwd(code, B, H, N, D, float(scale), _mask_code(mask), int(window), _ptr(q),
                          _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                          _ptr(dv), _ptr(ws), ws.numel() * ws.element_size(),
                          _stream(q, stream)))
    return dq, dk, dv


def _check_seg(seg, q):
    """Segment ids: a contiguous int32 [B, N] tensor on q's device."""
    import torch
    B, _, N, _ = q.shape
    if (tuple(seg.shape) != (B, N) or seg.dtype != torch.int32 or seg.device != q.device
            or not seg.is_contiguous()):
        raise ValueError("seg must be a contiguous int32 [B, N] tensor on q's device")


def attn_fwd_seg(q, k, v, seg, scale: float = DEFAULT_SCALE, mask: str = "causal",
                 window: int = 0, o=None, lse=None, stream=None):
    """attn_fwd with the segment predicate: pair (i, j) also needs
    seg[b, i] == seg[b, j] (seg: int32 [B, N]); returns (o, lse)."""
    _on_gpu(q, "q")
    (B, H, N, D), o, lse = _fwd_args(q, k, v, o, lse)
    _check_seg(seg, q)
    _check(lib().attn_fwd_seg(_dtype_code(q), B, H, N, D, float(scale), _mask_code(mask),
                              int(window), _ptr(seg), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                              _ptr(lse), _stream(q, stream)))
    return o, lse


def attn_bwd_seg(q, k, v, o, dout, lse, seg, scale: float = DEFAULT_SCALE, mask: str = "causal",
                 window: int = 0, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """attn_bwd with the segment predicate (lse from attn_fwd_seg with the same
    seg, mask and window); returns (dq, dk, dv)."""
    _on_gpu(q, "q")
    (code, B, H, N, D), dq, dk, dv, ws = _bwd_args(q, k, v, o, dout, lse, dq, dk, dv, workspace)
    _check_seg(seg, q)
    _check(lib().attn_bwd_seg(code, B, H, N, D, float(scale), _mask_code(mask), int(window),
                              _ptr(seg), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                              _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(q, stream)))
    return dq, dk, dv


def _train_args(q, k, v, o, lse, workspace, loss, need=None):
    """Validate attn_fwd_train's tensors; ``loss`` must be a one-element
    float64 tensor on q's device (the library writes one double there)."""
    import torch
    shape, o, lse = _fwd_args(q, k, v, o, lse)
    if workspace is None:
        if need is None:
            need = attn_bwd_workspace_bytes(_dtype_code(q), *shape)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_buffer(workspace, q)
    if loss is None:
        loss = torch.empty(1, dtype=torch.float64, device=q.device)
    if loss.numel() != 1 or loss.dtype != torch.float64 or loss.device != q.device \
            or not loss.is_contiguous():
        raise ValueError("loss must be a one-element float64 tensor on q's device")
    return shape, o, lse, workspace, loss


def attn_fwd_train(q, k, v, scale: float = DEFAULT_SCALE, mask: str = "causal", window: int = 0,
                   o=None, lse=None, workspace=None, loss=None, stream=None):
    """Forward of the training step with the loss sum(o^2)/2 fused in; returns
    (o, lse, loss, workspace): loss is a one-element float64 device tensor, and
    the workspace carries the per-row values attn_bwd_from_fwd reads."""
    _on_gpu(q, "q")
    (B, H, N, D), o, lse, workspace, loss = _train_args(q, k, v, o, lse, workspace, loss)
    code = _dtype_code(q)
    _check(lib().attn_fwd_train(code, B, H, N, D, float(scale), _mask_code(mask), int(window),
                                _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _ptr(loss),
                                _stream(q, stream)))
    return o, lse, loss, workspace


def attn_bwd_from_fwd(q, k, v, o, lse, workspace, scale: float = DEFAULT_SCALE,
                      mask: str = "causal", window: int = 0, dq=None, dk=None, dv=None,
                      stream=None):
    """Gradients (dq, dk, dv) of the loss sum(o^2)/2 from attn_fwd_train's outputs."""
    _on_gpu(q, "q")
    (code, B, H, N, D), dq, dk, dv, ws = _bwd_args(q, k, v, o, o, lse, dq, dk, dv, workspace)
    _check(lib().attn_bwd_from_fwd(code, B, H, N, D, float(scale), _mask_code(mask), int(window),
                                   _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dq),
                                   _ptr(dk), _ptr(dv), _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(q, stream)))
    return dq, dk, dv


def nw_gauss_average(tx, ty, sx, sy, sv, denom: float = 0.25, out=None, stream=None):
    """Nadaraya-Watson average at every target; float32 1-D device tensors."""
    import torch
    for name, t in (("tx", tx), ("ty", ty), ("sx", sx), ("sy", sy), ("sv", sv)):
        if t.dim() != 1 or t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous 1-D float32 device tensor")
        if t.device != tx.device:
            raise ValueError(f"{name} must be on tx's device")
    if ty.shape != tx.shape or sy.shape != sx.shape or sv.shape != sx.shape:
        raise ValueError("target columns and source columns must have matching lengths")
    if out is None:
        out = torch.empty_like(tx)
    _same(out, tx, "out", "tx")
    _check(lib().nw_gauss_average(tx.numel(), _ptr(tx), _ptr(ty), sx.numel(), _ptr(sx),
                                  _ptr(sy), _ptr(sv), float(denom), _ptr(out),
                                  _stream(tx, stream)))
    return out


def _dev(t, name, dim):
    if t.dim() != dim or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name} must be a contiguous {dim}-D device tensor")


def attn_matrix_to_table(m, t=None, d=None, x=None, stream=None):
    """The long table (t, d, x) of a [T, D] device matrix, rows in (t, d) order."""
    import torch
    _dev(m, "m", 2)
    T, D = m.shape
    t = torch.empty(T * D, dtype=torch.int64, device=m.device) if t is None else t
    d = torch.empty(T * D, dtype=torch.int64, device=m.device) if d is None else d
    x = torch.empty(T * D, dtype=m.dtype, device=m.device) if x is None else x
    for name, c, dt in (("t", t, torch.int64), ("d", d, torch.int64), ("x", x, m.dtype)):
        if (c.dim() != 1 or c.numel() != T * D or c.dtype != dt or c.device != m.device
                or not c.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous 1-D {dt} tensor of T * D elements "
                             "on m's device")
    _check(lib().attn_matrix_to_table(_dtype_code(m), T, D, _ptr(m), _ptr(t), _ptr(d), _ptr(x),
                                      _stream(m, stream)))
    return t, d, x


def attn_table_workspace_bytes(dtype_code: int, T: int, D: int) -> int:
    return lib().attn_table_workspace_bytes(dtype_code, T, D)


def attn_table_to_matrix(t, d, x, T: int, D: int, m=None, workspace=None, status=None,
                         stream=None, check: bool = True):
    """Pivot rows (t, d, x) into a [T, D] matrix (NaN where no row names a cell).

    With check (the default) the call waits for the stream and raises ValueError
    when a coordinate was out of range or a cell was named twice; without it,
    returns (m, status) and the caller reads the int32 status word itself."""
    import torch
    for name, c in (("t", t), ("d", d), ("x", x)):
        _dev(c, name, 1)
    if t.dtype != torch.int64 or d.dtype != torch.int64:
        raise ValueError("t and d must be int64")
    if not (t.numel() == d.numel() == x.numel()):
        raise ValueError("t, d and x must have one length")
    if t.device != x.device or d.device != x.device:
        raise ValueError("t, d and x must be on one device")
    m = torch.empty((T, D), dtype=x.dtype, device=x.device) if m is None else m
    if (tuple(m.shape) != (T, D) or m.dtype != x.dtype or m.device != x.device
            or not m.is_contiguous()):
        raise ValueError("m must be a contiguous [T, D] tensor of x's dtype on x's device")
    need = attn_table_workspace_bytes(_dtype_code(x), T, D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _check_buffer(workspace, x)
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=x.device)
    if status.numel() != 1 or status.dtype != torch.int32 or status.device != x.device:
        raise ValueError("status must be a one-element int32 tensor on x's device")
    _check(lib().attn_table_to_matrix(_dtype_code(x), t.numel(), _ptr(t), _ptr(d), _ptr(x), T, D,
                                      _ptr(m), _ptr(status), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(),
                                      _stream(x, stream)))
    if not check:
        return m, status
    code = int(status.item())
    if code:
        what = [w for bit, w in ((1, "a coordinate is out of range"), (2, "a cell is named twice"))
                if code & bit]
        raise ValueError("table_to_matrix: " + " and ".join(what))
    return m


def attn_qkv_project(x, wq, wk, wv, heads: int, q=None, k=None, v=None, stream=None):
    """(q, k, v) = (x Wq, x Wk, x Wv) laid out [B, heads, N, 64]; x is [B, N, Dm],
    each weight [Dm, heads * 64]."""
    import torch
    _dev(x, "x", 3)
    B, N, Dm = x.shape
    for name, w in (("wq", wq), ("wk", wk), ("wv", wv)):
        _dev(w, name, 2)
        if tuple(w.shape) != (Dm, heads * 64) or w.dtype != x.dtype:
            raise ValueError(f"{name} must be [{Dm}, {heads * 64}] of x's dtype")
    for name, w in (("wq", wq), ("wk", wk), ("wv", wv)):
        if w.device != x.device:
            raise ValueError(f"{name} must be on x's device")
    outs = [torch.empty((B, heads, N, 64), dtype=x.dtype, device=x.device) if o is None else o
            for o in (q, k, v)]
    for name, o in zip("qkv", outs):
        if (tuple(o.shape) != (B, heads, N, 64) or o.dtype != x.dtype or o.device != x.device
                or not o.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous [B, heads, N, 64] tensor of x's "
                             "dtype on x's device")
    _check(lib().attn_qkv_project(_dtype_code(x), B, N, Dm, heads, _ptr(x), _ptr(wq), _ptr(wk),
                                  _ptr(wv), *(_ptr(o) for o in outs), _stream(x, stream)))
    return tuple(outs)


TIMER_FWD, TIMER_BWD_PRE, TIMER_BWD_DKDV, TIMER_BWD_DQ, TIMER_NW, TIMER_TABLE, TIMER_PROJECT = range(7)
TIMER_NAMES = {TIMER_FWD: "fwd", TIMER_BWD_PRE: "bwd_pre", TIMER_BWD_DKDV: "bwd_dkdv",
               TIMER_BWD_DQ: "bwd_dq", TIMER_NW: "nw", TIMER_TABLE: "table_to_matrix",
               TIMER_PROJECT: "qkv_project"}


def attn_set_kernel_timer(slot: int, start, stop):
    """Record two already-recorded torch.cuda.Event objects (or None, None)
    around every later launch of the kernel in ``slot`` (TIMER_*)."""
    h = (lambda e: None if e is None else ctypes.c_void_p(e.cuda_event))
    _check(lib().attn_set_kernel_timer(slot, h(start), h(stop)))


__all__ = ["attn_causal_fwd", "attn_causal_bwd", "attn_causal_bwd_workspace_bytes",
           "attn_causal_bwd_noalloc", "attn_fwd",
           "attn_bwd", "attn_bwd_workspace_bytes", "attn_fwd_train", "attn_bwd_from_fwd", "MASKS",
           "attn_fwd_seg", "attn_bwd_seg",
           "nw_gauss_average", "attn_matrix_to_table", "attn_table_to_matrix",
           "attn_table_workspace_bytes", "attn_qkv_project", "attn_set_kernel_timer",
           "attn_last_error", "lib", "AttnError",
           "ATTN_F64", "ATTN_F32", "ATTN_BF16"]
