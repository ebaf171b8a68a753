"""Helpers for GPU-vs-oracle parity tests (imported by the gpu tests).

Tolerances follow the stated targets:
  * outputs (out, dq, dk, dv): max |gpu - ref| <= tol * max(1, max |ref|),
    tol = 1e-2 for bf16 inputs, 1e-4 for fp32 inputs;
  * tau: |gpu - ref| <= 1e-3 * max(1, |ref|);
  * support: {j : x_ref > tau_gpu} equals {j : x_ref > tau_ref} except for
    entries with |x_ref - tau_ref| <= 1e-4;
  * block mask: a superset of every tile holding an entry with x_ref - tau_ref > 1e-4.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import entmax_oracle as O

TAU_RTOL = 1e-3
SUPPORT_BAND = 1e-4


def out_tol(dtype: str) -> float:
    return 1e-2 if dtype == "bf16" else 1e-4


def to_device(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)
    return t.cuda()


def check_close(name, gpu, ref, tol):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{name}: non-finite values"
    err = float(np.max(np.abs(gpu - ref))) if gpu.size else 0.0
    scale = max(1.0, float(np.max(np.abs(ref)))) if ref.size else 1.0
    assert err <= tol * scale, f"{name}: max abs err {err:.3e} > {tol:.1e} * {scale:.3g}"
    return err


def check_tau(tau_gpu, tau_ref):
    tau_gpu = np.asarray(tau_gpu, dtype=np.float64)
    lim = TAU_RTOL * np.maximum(1.0, np.abs(tau_ref))
    bad = np.abs(tau_gpu - tau_ref) > lim
    assert not bad.any(), f"tau: {bad.sum()} rows off, worst {np.abs(tau_gpu - tau_ref).max():.3e}"
    return float(np.max(np.abs(tau_gpu - tau_ref))) if tau_ref.size else 0.0


def check_support(q, k, alpha, causal, tau_gpu, tau_ref):
    """Support of every row from the oracle's float64 scores, thresholded at
    the GPU's tau and at the oracle's tau; mismatches must sit in the band."""
    qh = np.asarray(q, np.float64).reshape((-1,) + q.shape[-2:])
    kh = np.asarray(k, np.float64).reshape((-1,) + k.shape[-2:])
    nh, n, _ = qh.shape
    tg = np.asarray(tau_gpu, np.float64).reshape(nh, n)
    tr = np.asarray(tau_ref, np.float64).reshape(nh, n)
    mism = 0
    for h in range(nh):
        for i0 in range(0, n, 256):
            i1 = min(n, i0 + 256)
            x = O.scores(qh[h, i0:i1], kh[h], alpha, causal, i0)
            a = x > tg[h, i0:i1, None]
            b = x > tr[h, i0:i1, None]
            diff = a != b
            if diff.any():
                near = np.abs(x - tr[h, i0:i1, None]) <= SUPPORT_BAND
                assert np.all(near[diff]), "support differs away from the threshold"
                mism += int(diff.sum())
    return mism


def check_mask(mask_gpu, margins, band=SUPPORT_BAND):
    """mask_gpu must cover every tile the oracle finds active beyond the band.
    Returns (false_positive_tiles, active_tiles)."""
    m = np.asarray(mask_gpu).astype(bool)
    need = margins > band
    missing = need & ~m
    assert not missing.any(), f"block mask misses {missing.sum()} active tiles"
    fp = m & ~(margins > -band)
    return int(fp.sum()), int(need.sum())


def visible_tiles(n, bm, bn, causal):
    nq, nk = -(-n // bm), -(-n // bn)
    vis = np.ones((nq, nk), dtype=bool)
    if causal:
        for qt in range(nq):
            last_q = min(n - 1, qt * bm + bm - 1)
            vis[qt, last_q // bn + 1:] = False
    return vis
