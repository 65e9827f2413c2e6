"""Seeded synthetic inputs shared by the tests, the bench and the oracle's callers.

This module draws and casts numbers; it holds none of the method's arithmetic
(no scores, no softmax, no weighted sums).  Every draw uses
``numpy.random.default_rng(seed)`` in float64, in the order the demo script on
"Show HN: automatic deduction of FlashAttention kernel from 25 lines of SQL"
(neshdevtech.com, ``main()`` and the ``check_*`` helpers) draws its arrays:
q, then k, then v, each ``rng.normal(size=...)``.

bfloat16 inputs are made once, here: float64 -> float32 (numpy, round to
nearest even) -> bfloat16 (round to nearest even on the float32 bits).  Both
the GPU path and the oracle consume the same 16-bit patterns.

Workloads (B, H, N, D = 64, layout [B, H, N, D] row-major):

=========  ====  ======================  =====================================
name       seed  shape                   values
=========  ====  ======================  =====================================
fp64_256      0  (1, 1, 256, 64)         q, k, v ~ N(0, 1), float64
fp32_2k       1  (4, 16, 2048, 64)       q, k, v ~ N(0, 1) -> float32
bf16_4k       2  (8, 32, 4096, 64)       q, k, v ~ N(0, 1) -> bfloat16
nw_64k        3  65,536 x 65,536         targets, sources ~ U[0, 10)^2,
                                         v = sin(x)cos(y) + 0.1 N(0, 1)
bf16_32k      4  (1, 16, 32768, 64)      q, k ~ 2 N(0, 1), v ~ N(0, 1) -> bf16
proj_4k       5  x (8, 4096, 2048),      x ~ N(0, 1); wq, wk, wv ~ N(0, 1/2048)
                 w (2048, 32 * 64)       -> bfloat16 (Q, K, V of bf16_4k's shape)
table_16x32k  6  (524288, 64) matrix     m ~ N(0, 1) -> bfloat16; its 2^25 rows
                                         (t, d, x) in a seeded random order
=========  ====  ======================  =====================================

The projection draws follow the page on MLIR attention heads (x, then Wq, Wk,
Wv); weights are scaled by 1/sqrt(d_model) so the projected values are of
order one, as the attention inputs above are.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

D = 64

# name -> (seed, B, H, N, dtype, q/k multiplier)
ATTENTION_WORKLOADS = {
    "fp64_256": (0, 1, 1, 256, "f64", 1.0),
    "fp32_2k": (1, 4, 16, 2048, "f32", 1.0),
    "bf16_4k": (2, 8, 32, 4096, "bf16", 1.0),
    "bf16_32k": (4, 1, 16, 32768, "bf16", 2.0),
}


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    f32 = np.ascontiguousarray(x, dtype=np.float32)
    u = f32.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact widening)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class AttentionInputs:
    """q, k, v in the storage format of ``dtype``.

    For "f64" and "f32" the arrays are float64 / float32.  For "bf16" they are
    uint16 bit patterns.  ``*_f64`` are the float64 values the stored numbers
    represent exactly (what the oracle consumes).
    """

    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray

    def as_f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if self.dtype == "bf16":
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)


def cast(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f64":
        return np.ascontiguousarray(x, dtype=np.float64)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f64_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def attention_inputs(seed: int, B: int, H: int, N: int, dtype: str,
                     qk_mult: float = 1.0, d: int = D) -> AttentionInputs:
    """q, k, v drawn N(0,1) from ``default_rng(seed)`` in q, k, v order."""
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(B, H, N, d)) * qk_mult
    k = rng.normal(size=(B, H, N, d)) * qk_mult
    v = rng.normal(size=(B, H, N, d))
    return AttentionInputs(dtype, cast(q, dtype), cast(k, dtype), cast(v, dtype))


def workload(name: str) -> AttentionInputs:
    seed, B, H, N, dtype, mult = ATTENTION_WORKLOADS[name]
    return attention_inputs(seed, B, H, N, dtype, mult)


def segment_ids(seed: int, B: int, N: int, kind: str = "packed", mean_len: int = 512,
                n_ids: int = 3) -> np.ndarray:
    """Segment ids int32 [B, N] from ``default_rng(seed)``.

    "packed": documents packed back to back, one id per document (0, 1, 2, ...
    along the row), lengths drawn from a geometric law of mean ``mean_len``
    (at least 1 token), a mix of short and long documents.
    "interleaved": every token an id drawn uniformly from ``n_ids`` values, so
    equal ids are scattered (no key tile is one segment).
    """
    rng = np.random.default_rng(seed)
    if kind == "interleaved":
        return rng.integers(0, n_ids, size=(B, N)).astype(np.int32)
    if kind != "packed":
        raise ValueError(f"unknown segment kind {kind!r}")
    out = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        lens = []
        while sum(lens) < N:
            lens.append(int(rng.geometric(1.0 / mean_len)))
        out[b] = np.repeat(np.arange(len(lens), dtype=np.int32), lens)[:N]
    return out


def page_sizes_inputs() -> dict[int, tuple[np.ndarray, np.ndarray, np.ndarray]]:
    """The demo's forward/gradient sizes: one rng (seed 0) drawn for n = 64, then n = 256."""
    rng = np.random.default_rng(0)
    out = {}
    for n in (64, 256):
        q, k, v = (rng.normal(size=(n, D)) for _ in range(3))
        out[n] = (q, k, v)
    return out


def page_mask_inputs() -> tuple[np.ndarray, np.ndarray, np.ndarray, int]:
    """The demo's infinity-in-V case: n = 16, seed 1, v[9, 0] = +inf."""
    n, j = 16, 9
    rng = np.random.default_rng(1)
    q, k, v = (rng.normal(size=(n, D)) for _ in range(3))
    v[j, 0] = np.inf
    return q, k, v, j


@dataclass
class NWInputs:
    tx: np.ndarray
    ty: np.ndarray
    sx: np.ndarray
    sy: np.ndarray
    sv: np.ndarray


def nw_inputs(n_targets: int = 65536, n_sources: int = 65536, seed: int = 3) -> NWInputs:
    """Targets and sources uniform on [0, 10)^2, v = sin(x)cos(y) + 0.1 N(0,1), float32."""
    rng = np.random.default_rng(seed)
    t = rng.uniform(0.0, 10.0, size=(n_targets, 2))
    s = rng.uniform(0.0, 10.0, size=(n_sources, 2))
    noise = rng.normal(size=n_sources)
    v = np.sin(s[:, 0]) * np.cos(s[:, 1]) + 0.1 * noise
    f = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    return NWInputs(f(t[:, 0]), f(t[:, 1]), f(s[:, 0]), f(s[:, 1]), f(v))


def page_nw_inputs() -> NWInputs:
    """The demo's control case: 64 targets, 256 sources on [0, 1)^2, seed 2,
    y = sin(4x) + cos(3y), kept in float64 (cast by the caller)."""
    rng = np.random.default_rng(2)
    targets, sources = rng.uniform(size=(64, 2)), rng.uniform(size=(256, 2))
    y = np.sin(4 * sources[:, 0]) + np.cos(3 * sources[:, 1])
    return NWInputs(targets[:, 0].copy(), targets[:, 1].copy(),
                    sources[:, 0].copy(), sources[:, 1].copy(), y)


@dataclass
class ProjectionInputs:
    """x [B, N, Dm] and wq, wk, wv [Dm, H * 64] in the storage format of dtype
    (uint16 bit patterns for "bf16"), with ``as_f64`` as for AttentionInputs."""

    dtype: str
    heads: int
    x: np.ndarray
    wq: np.ndarray
    wk: np.ndarray
    wv: np.ndarray

    def as_f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if self.dtype == "bf16":
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)


def projection_inputs(seed: int, B: int, N: int, Dm: int, H: int, dtype: str) -> ProjectionInputs:
    """x ~ N(0, 1) [B, N, Dm], then wq, wk, wv ~ N(0, 1/Dm) [Dm, H * 64]."""
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(B, N, Dm))
    ws = [rng.normal(size=(Dm, H * D)) / np.sqrt(Dm) for _ in range(3)]
    return ProjectionInputs(dtype, H, cast(x, dtype), *(cast(w, dtype) for w in ws))


PROJECTION_WORKLOADS = {"proj_4k": (5, 8, 4096, 2048, 32, "bf16")}


def projection_workload(name: str) -> ProjectionInputs:
    seed, B, N, Dm, H, dtype = PROJECTION_WORKLOADS[name]
    return projection_inputs(seed, B, N, Dm, H, dtype)


def table_matrix(seed: int, T: int, Dc: int, dtype: str):
    """A T x Dc matrix ~ N(0, 1) in the storage format of dtype, and a
    permutation of its T * Dc cells (the order its table rows arrive in)."""
    rng = np.random.default_rng(seed)
    m = cast(rng.normal(size=(T, Dc)), dtype)
    perm = rng.permutation(T * Dc)
    return m, perm


TABLE_WORKLOADS = {"table_16x32k": (6, 16 * 32768, 64, "bf16")}
