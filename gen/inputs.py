"""Seeded synthetic inputs for fused alpha-entmax attention.

This module only draws random tensors and rounds them to the storage type the
kernels read; it holds none of the attention arithmetic.  Both the float64
oracle (tests, CPU baseline) and the GPU path consume exactly the arrays
produced here, so the two sides see bit-identical inputs.

Workload recipes (the pages describe trained RoBERTa / ModernBERT / GPT-2
attention, which needs datasets and weights; these synthetic recipes stand in
for it):

* ``iid``      Q, K ~ N(0, c^2), V, dO ~ N(0, 1); c trades element sparsity
               against density.
* ``planted``  "locality" workload: 64 random centroids c_k = sqrt(d) * u_k with
               u_k a uniformly random unit vector; token i belongs to cluster
               k = (i // span) % 64;  Q_i = a * c_k + N(0, I),
               K_i = c_k + 0.3 * N(0, I), V, dO ~ N(0, 1).  With a = 3 this
               yields >95 % block sparsity at 64-key tiles.
* ``tied``     many exactly equal keys: one centroid c = sqrt(d) * u;
               Q_i = a * c + N(0, I); K_j = c for j < ties (identical rows),
               K_j ~ N(0, I) after; V, dO ~ N(0, 1).  Rows that see more than
               65536 of the tied keys put them all in one histogram bin.

Draw order (fixed, one ``standard_normal`` call per tensor, PCG64 via
``numpy.random.default_rng(seed)``): centroids (planted only), Q, K, V, dO.
Rounding to bfloat16 is round-to-nearest-even on the float32 bit pattern.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "bf16_round",
    "make_inputs",
    "make_score_rows",
    "workload",
]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float values to the nearest bfloat16 (ties to even), returned as float32.

    NaN is not expected in generated data; infinities pass through unchanged.
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16) << np.uint64(16)
    return u.astype(np.uint32).view(np.float32).reshape(f.shape)


@dataclass(frozen=True)
class Workload:
    """One synthetic attention problem: shapes, dtype, alpha, causality, generator."""

    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "f32" or "bf16": storage type of q, k, v, dout
    causal: bool
    alpha: float
    gen: str              # "iid" or "planted"
    scale: float = 1.0    # iid: std of Q and K (c); V scaled too when scale_v
    scale_v: bool = False
    strength: float = 3.0  # planted: Q = strength * centroid + noise
    span: int = 256        # planted: tokens per cluster run
    ties: int = 0          # tied: number of leading identical keys
    backward: bool = True
    seed: int = 0
    extra: dict = field(default_factory=dict)

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


def make_inputs(w: Workload, heads: slice | None = None) -> dict:
    """Draw q, k, v, dout for workload ``w`` as float32 arrays of shape [B,H,N,d].

    Values are exactly representable in the storage dtype (bf16-rounded for
    "bf16").  ``heads`` optionally restricts the returned arrays to a slice of
    the flattened (B*H) head axis *after* the full draw, so a subset always
    equals the corresponding part of the full problem.
    """
    rng = np.random.default_rng(w.seed)
    shape = (w.B, w.H, w.N, w.d)
    out = {}
    if w.gen == "planted":
        g = rng.standard_normal((w.B, w.H, 64, w.d))
        u = g / np.linalg.norm(g, axis=-1, keepdims=True)
        cent = np.sqrt(w.d) * u
        cluster = (np.arange(w.N) // w.span) % 64
        c_tok = cent[:, :, cluster, :]
        q = w.strength * c_tok + rng.standard_normal(shape)
        k = c_tok + 0.3 * rng.standard_normal(shape)
        v = rng.standard_normal(shape)
        do = rng.standard_normal(shape)
    elif w.gen == "tied":
        g = rng.standard_normal((w.B, w.H, 1, w.d))
        cent = np.sqrt(w.d) * g / np.linalg.norm(g, axis=-1, keepdims=True)
        q = w.strength * cent + rng.standard_normal(shape)
        k = rng.standard_normal(shape)
        k[:, :, :w.ties, :] = cent
        v = rng.standard_normal(shape)
        do = rng.standard_normal(shape)
    elif w.gen == "iid":
        q = w.scale * rng.standard_normal(shape)
        k = w.scale * rng.standard_normal(shape)
        v = rng.standard_normal(shape)
        if w.scale_v:
            v = w.scale * v
        do = rng.standard_normal(shape)
    else:
        raise ValueError(f"unknown generator {w.gen!r}")
    for name, arr in (("q", q), ("k", k), ("v", v), ("dout", do)):
        a = arr.astype(np.float32)
        if w.dtype == "bf16":
            a = bf16_round(a)
        if heads is not None:
            a = a.reshape(w.B * w.H, w.N, w.d)[heads]
        out[name] = np.ascontiguousarray(a)
    return out


def make_score_rows(rows: int, n: int, scale: float = 1.0, seed: int = 0, dtype: str = "f32",
                    masked: float = 0.0) -> np.ndarray:
    """Score rows for the stand-alone entmax transform: s ~ N(0, scale^2),
    float32 [rows, n] rounded to the storage dtype; a share `masked` of the
    entries (drawn after the scores) is set to -inf."""
    rng = np.random.default_rng(seed)
    s = (scale * rng.standard_normal((rows, n))).astype(np.float32)
    if dtype == "bf16":
        s = bf16_round(s)
    if masked > 0.0:
        s[rng.random((rows, n)) < masked] = -np.inf
    return np.ascontiguousarray(s)


# The five reference workloads.  Index 0 is the small fp32 parity case; the
# others are the bf16 performance shapes.  Sweeps (c, alpha) are variants.
WORKLOADS = {
    "small_f32": Workload("small_f32", 1, 1, 256, 64, "f32", False, 1.5, "iid",
                          backward=False),
    "iid_causal_4k": Workload("iid_causal_4k", 4, 16, 4096, 64, "bf16", True, 1.5,
                              "iid", scale=1.0),
    "planted_16k": Workload("planted_16k", 1, 16, 16384, 128, "bf16", True, 1.5,
                            "planted", span=256),
    "encoder_8k": Workload("encoder_8k", 2, 32, 8192, 64, "bf16", False, 1.5, "iid",
                           scale=2.0, scale_v=True),
    "planted_32k": Workload("planted_32k", 1, 8, 32768, 128, "bf16", True, 1.5,
                            "planted", span=512),
}


def workload(name: str, **overrides) -> Workload:
    """Look up a named workload, optionally overriding fields (c, alpha sweeps, small N)."""
    w = WORKLOADS[name]
    return w.with_(**overrides) if overrides else w
