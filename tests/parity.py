"""Helpers for GPU-vs-oracle parity tests (imported by the gpu tests).

Tolerances follow the stated targets:
  * outputs (out, dq, dk, dv), two bounds, both required:
      - per row (one query's output or gradient, one key's dK / dV):
        max_j |gpu_ij - ref_ij| <= tol * max(1, max_j |ref_ij|);
      - over the whole tensor: max |gpu - ref| <= tol * max(1, max |ref|);
    tol = 1e-2 for bf16 inputs, 1e-4 for fp32 inputs.  The per-row bound keeps
    the stated absolute tolerance on rows of order one (and on rows that are
    exactly zero in the reference, such as keys outside every support) however
    large the largest row of the tensor is;
  * tau: |gpu - ref| <= 1e-3 * max(1, |ref|);
  * support: {j : x_ref > tau_gpu} equals {j : x_ref > tau_ref} except for
    entries with |x_ref - tau_ref| <= 1e-4;
  * block mask: a superset of every tile holding an entry with x_ref - tau_ref > 1e-4.
Every check prints the raw max-abs error it measured.
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
    """Per-row and tensor-wide max-abs bounds (rows are the last axis).
    Returns (raw max-abs error, worst per-row ratio err / bound)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{name}: non-finite values"
    if gpu.size == 0:
        return 0.0, 0.0
    diff = np.abs(gpu - ref)
    err = float(diff.max())
    scale = max(1.0, float(np.abs(ref).max()))
    rd = diff.reshape(-1, diff.shape[-1]).max(axis=1)
    rbound = tol * np.maximum(1.0, np.abs(ref).reshape(-1, ref.shape[-1]).max(axis=1))
    ratio = rd / rbound
    worst = int(np.argmax(ratio))
    zero_rows = np.abs(ref).reshape(-1, ref.shape[-1]).max(axis=1) == 0.0
    print(f"  {name}: max abs err {err:.3e} (tensor bound {tol * scale:.3e}); worst row {worst}: "
          f"{rd[worst]:.3e} = {ratio[worst]:.3f} of its bound; zero reference rows {int(zero_rows.sum())}, "
          f"largest gpu value there {float(rd[zero_rows].max()) if zero_rows.any() else 0.0:.3e}", flush=True)
    assert err <= tol * scale, f"{name}: max abs err {err:.3e} > {tol:.1e} * {scale:.3g}"
    assert ratio[worst] <= 1.0, (f"{name}: row {worst} max abs err {rd[worst]:.3e} > "
                                 f"{tol:.1e} * max(1, row max {rbound[worst] / tol:.3g})")
    return err, float(ratio[worst])


def check_tau(tau_gpu, tau_ref):
    tau_gpu = np.asarray(tau_gpu, dtype=np.float64)
    lim = TAU_RTOL * np.maximum(1.0, np.abs(tau_ref))
    bad = np.abs(tau_gpu - tau_ref) > lim
    worst = float(np.max(np.abs(tau_gpu - tau_ref))) if tau_ref.size else 0.0
    print(f"  tau: max abs err {worst:.3e}", flush=True)
    assert not bad.any(), f"tau: {bad.sum()} rows off, worst {worst:.3e}"
    return worst


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


def micro_mask(mask_gpu, n):
    """32x32 micro-tile bits from the mask bytes: bit 1 covers keys 0-31 of a
    64-key tile, bit 2 keys 32-63.  Shape [..., n_q32, ceil(n / 32)]."""
    m = np.asarray(mask_gpu).astype(np.uint8)
    halves = np.stack([(m >> 1) & 1, (m >> 2) & 1], axis=-1).astype(bool)
    halves &= (m != 0)[..., None]
    return halves.reshape(m.shape[:-1] + (2 * m.shape[-1],))[..., :-(-n // 32)]


def check_micro_mask(mask_gpu, margins32, n, band=SUPPORT_BAND):
    """Every 32x32 micro-tile the oracle finds active beyond the band has its
    bit set; returns (false-positive micro-tiles, active micro-tiles)."""
    mm = micro_mask(mask_gpu, n)
    need = margins32 > band
    missing = need & ~mm
    assert not missing.any(), f"micro-tile bits miss {missing.sum()} active 32x32 tiles"
    return int((mm & ~(margins32 > -band)).sum()), int(need.sum())


def visible_tiles(n, bm, bn, causal):
    nq, nk = -(-n // bm), -(-n // bn)
    vis = np.ones((nq, nk), dtype=bool)
    if causal:
        for qt in range(nq):
            last_q = min(n - 1, qt * bm + bm - 1)
            vis[qt, last_q // bn + 1:] = False
    return vis
