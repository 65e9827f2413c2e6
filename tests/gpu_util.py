"""Helpers for the GPU parity tests: host arrays <-> device tensors, and calls
through the C ABI binding with canary guard bands around every output."""
from __future__ import annotations

import sys

import numpy as np
import torch

import causal_softmax_attention_amd as csa

DEV = "cuda:0"
CANARY_F32 = np.float32(-1.2345678e30)


def note(msg: str):
    """Name the case on stdout before a GPU step (flushed, so it survives a crash)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


TORCH_DT = {"f64": torch.float64, "f32": torch.float32, "bf16": torch.bfloat16}


class Guarded:
    """A device buffer with `pad` canary elements before and after the view."""

    def __init__(self, shape, dtype, pad=256):
        n = int(np.prod(shape))
        self.raw = torch.empty(n + 2 * pad, dtype=dtype, device=DEV)
        self.raw.fill_(-1.2345678e30 if dtype != torch.bfloat16 else -1.2e30)
        self.pad, self.n = pad, n
        self.ref = self.raw.clone()
        self.view = self.raw[pad:pad + n].view(*shape)

    def intact(self) -> bool:
        p, n = self.pad, self.n
        return bool(torch.equal(self.raw[:p], self.ref[:p]) and
                    torch.equal(self.raw[p + n:], self.ref[p + n:]))


def run_fwd(q, k, v, scale=0.125, guard=True, mask=None, window=0, seg=None):
    """The forward through attn_causal_fwd, or attn_fwd when a mask is named,
    or attn_fwd_seg with segment ids (mask default causal)."""
    B, H, N, D = q.shape
    if seg is not None:
        call = lambda **kw: csa.attn_fwd_seg(q, k, v, seg, scale, mask or "causal", window, **kw)
    elif mask is None:
        call = lambda **kw: csa.attn_causal_fwd(q, k, v, scale, **kw)
    else:
        call = lambda **kw: csa.attn_fwd(q, k, v, scale, mask, window, **kw)
    if not guard:
        return call()
    lse_dt = torch.float64 if q.dtype == torch.float64 else torch.float32
    og, lg = Guarded((B, H, N, D), q.dtype), Guarded((B, H, N), lse_dt)
    o, lse = call(o=og.view, lse=lg.view)
    torch.cuda.synchronize()
    assert og.intact() and lg.intact(), "forward wrote outside its outputs"
    return o, lse


def run_bwd(q, k, v, o, dout, lse, scale=0.125, guard=True, mask=None, window=0, seg=None):
    """The backward through attn_causal_bwd, or attn_bwd when a mask is named,
    or attn_bwd_seg with segment ids (mask default causal)."""
    if seg is not None:
        call = lambda **kw: csa.attn_bwd_seg(q, k, v, o, dout, lse, seg, scale,
                                             mask or "causal", window, **kw)
    elif mask is None:
        call = lambda **kw: csa.attn_causal_bwd(q, k, v, o, dout, lse, scale, **kw)
    else:
        call = lambda **kw: csa.attn_bwd(q, k, v, o, dout, lse, scale, mask, window, **kw)
    if not guard:
        return call()
    gs = [Guarded(tuple(q.shape), q.dtype) for _ in range(3)]
    dq, dk, dv = call(dq=gs[0].view, dk=gs[1].view, dv=gs[2].view)
    torch.cuda.synchronize()
    assert all(g.intact() for g in gs), "backward wrote outside its outputs"
    return dq, dk, dv
