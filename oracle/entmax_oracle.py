"""Float64 CPU oracle for fused alpha-entmax attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test-suite, the smoke check of the package entry
point, and the CPU-baseline leg of the benchmark use it.  It shares no code,
constants or helpers with the HIP library.

What it computes (sources are the AdaSplash pages, cited by title and section):

* "AdaSplash: Adaptive Sparse Flash Attention" (ICML 2025 talk summary),
  section "Background": attention maps query-key scores to a probability
  distribution that weights the values; alpha-entmax replaces softmax, alpha=1
  being softmax and alpha=2 sparsemax.
* Same page, "Accelerated Alpha-Entmax Transformation": the normaliser tau is
  the root of f(tau) = 0, chosen so that the probabilities sum to one.
* The score scale, the (alpha-1) factor and the threshold convention are the
  plain reading adopted for this build:  s_ij = q_i . k_j / sqrt(d),
  x_ij = (alpha-1) s_ij,  p_ij = [x_ij - tau_i]_+^(1/(alpha-1)),
  sum_j p_ij = 1,  o_i = sum_j p_ij v_j.  tau is reported in this x-domain.
  Causal attention hides keys j > i.
* Same page, "AdaSplash: Fused GPU Kernel for Attention": the output is exact;
  S and P are tiled only to save memory, so the oracle may materialise them.
* Same page, "Exploiting Sparsity": a key tile can be skipped when every
  probability in it is zero; ``tile_margins`` gives the exact active-tile set.
* Backward (Jacobian of entmax): with t = [x - tau]_+ and u = t^(1/(alpha-1)-1)
  (= p^(2-alpha)) on the support and 0 off it,
  ds = u * (dp - delta),  delta = sum(u dp) / sum(u).  Derived from
  differentiating sum_j [x_j - tau]_+^beta = 1 (beta = 1/(alpha-1)).

tau is solved exactly: sort-based closed forms for alpha = 2 (sparsemax) and
alpha = 1.5, bisection to a bracket width of 1e-12 otherwise.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROW_BLOCK = 256


def beta_of(alpha: float) -> float:
    """Exponent 1/(alpha-1) of the thresholded scores."""
    return 1.0 / (alpha - 1.0)


def _visible_count(x: np.ndarray) -> np.ndarray:
    return np.sum(np.isfinite(x), axis=-1)


def tau_bracket(x: np.ndarray, alpha: float):
    """Provable bracket [lo, hi] for tau on each row of x (masked entries = -inf).

    At tau = max(x) - 1 the largest term is exactly 1, so f >= 0; at
    tau = max(x) - n^(1-alpha) every term is at most 1/n, so f <= 0.
    """
    xmax = np.max(x, axis=-1)
    n = _visible_count(x).astype(np.float64)
    return xmax - 1.0, xmax - n ** (1.0 - alpha)


def entmax_f(x: np.ndarray, tau: np.ndarray, alpha: float) -> np.ndarray:
    """f(tau) = sum_j [x_j - tau]_+^beta - 1 for each row."""
    t = np.maximum(x - tau[..., None], 0.0)
    return np.sum(t ** beta_of(alpha), axis=-1) - 1.0


def tau_sort(x: np.ndarray, alpha: float) -> np.ndarray:
    """Exact tau for alpha in {2, 1.5} from the sorted scores.

    For a support made of the k largest scores z_1 >= ... >= z_k:
      alpha = 2:   sum_{r<=k} (z_r - tau) = 1
                   => tau_k = (sum_{r<=k} z_r - 1) / k
      alpha = 1.5: sum_{r<=k} (z_r - tau)^2 = 1
                   => tau_k = M_k - sqrt(1/k - (S_k - M_k^2))
                   (M_k, S_k = mean and mean square of the top k; the smaller
                   root, since tau < z_k on the support).
    The support size is the unique k with z_k > tau_k >= z_{k+1}.
    """
    if alpha not in (1.5, 2.0):
        raise ValueError("closed form only for alpha in {1.5, 2}")
    x = np.asarray(x, dtype=np.float64)
    n = _visible_count(x)
    z = -np.sort(-x, axis=-1)                      # descending, -inf last
    top = z[..., :1]
    y = z - top                                    # shift: tau is shift-equivariant
    kk = np.arange(1, x.shape[-1] + 1, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        c1 = np.cumsum(y, axis=-1)
        if alpha == 2.0:
            tk = (c1 - 1.0) / kk
        else:
            c2 = np.cumsum(y * y, axis=-1)
            m = c1 / kk
            disc = 1.0 / kk - (c2 / kk - m * m)
            tk = np.where(disc >= 0.0, m - np.sqrt(np.where(disc >= 0.0, disc, 0.0)), np.nan)
        nxt = np.concatenate([y[..., 1:], np.full(y.shape[:-1] + (1,), -np.inf)], axis=-1)
        in_range = kk <= n[..., None]
        nxt = np.where(kk < n[..., None], nxt, -np.inf)
        ok = in_range & (y > tk) & (tk >= nxt)
    count = ok.sum(axis=-1)
    if np.any(count != 1):
        bad = int(np.argmax(count != 1))
        raise AssertionError(f"sort-based tau: {int(count.flat[bad])} valid support sizes in a row")
    k_idx = np.argmax(ok, axis=-1)
    tau = np.take_along_axis(tk, k_idx[..., None], axis=-1)[..., 0]
    return tau + top[..., 0]


def tau_bisect(x: np.ndarray, alpha: float, tol: float = 1e-12) -> np.ndarray:
    """tau by plain bisection on the provable bracket until hi - lo <= tol."""
    x = np.asarray(x, dtype=np.float64)
    lo, hi = tau_bracket(x, alpha)
    lo = lo.copy()
    hi = hi.copy()
    beta = beta_of(alpha)
    for _ in range(200):
        if np.all(hi - lo <= tol):
            break
        mid = 0.5 * (lo + hi)
        t = np.maximum(x - mid[..., None], 0.0)
        f = np.sum(t ** beta, axis=-1) - 1.0
        lo = np.where(f >= 0.0, mid, lo)
        hi = np.where(f >= 0.0, hi, mid)
    return 0.5 * (lo + hi)


def tau_exact(x: np.ndarray, alpha: float) -> np.ndarray:
    """tau for rows of x: sort-based for alpha in {1.5, 2}, bisection otherwise."""
    if alpha in (1.5, 2.0):
        return tau_sort(x, alpha)
    return tau_bisect(x, alpha)


def entmax_probs(x: np.ndarray, tau: np.ndarray, alpha: float) -> np.ndarray:
    """p_j = [x_j - tau]_+^beta (masked entries give 0)."""
    t = np.maximum(x - tau[..., None], 0.0)
    return t ** beta_of(alpha)


def entmax(s: np.ndarray, alpha: float) -> np.ndarray:
    """alpha-entmax of score rows s (no attention): returns probabilities."""
    x = (alpha - 1.0) * np.asarray(s, dtype=np.float64)
    return entmax_probs(x, tau_exact(x, alpha), alpha)


def scores(q: np.ndarray, k: np.ndarray, alpha: float, causal: bool, i0: int = 0) -> np.ndarray:
    """x = (alpha-1) q k^T / sqrt(d) for the query rows q (global index i0 + r)."""
    d = q.shape[-1]
    s = (q @ k.T) / np.sqrt(d)
    if causal:
        rows = i0 + np.arange(q.shape[0])[:, None]
        cols = np.arange(k.shape[0])[None, :]
        s = np.where(cols <= rows, s, -np.inf)
    return (alpha - 1.0) * s


def _heads(a):
    a = np.asarray(a, dtype=np.float64)
    return a.reshape((-1,) + a.shape[-2:])


def _workers(n):
    return n if n else len(os.sched_getaffinity(0))


def forward_rows(qh, kh, vh, alpha: float, causal: bool, i0: int, i1: int):
    """One head (2-D arrays [N, d]): (out, tau) of query rows i0 .. i1-1 in
    float64.  attention_forward is this function applied block by block."""
    x = scores(np.asarray(qh[i0:i1], np.float64), np.asarray(kh, np.float64), alpha, causal, i0)
    t = tau_exact(x, alpha)
    p = entmax_probs(x, t, alpha)
    return p @ np.asarray(vh, np.float64), t, p


def backward_rows(qh, kh, vh, doh, tau_rows, alpha: float, causal: bool, i0: int, i1: int):
    """One head: the gradient terms contributed by query rows i0 .. i1-1,
    (dq[i0:i1], dk_part, dv_part) with dk_part, dv_part of shape [N, d].
    dq rows are complete; dK and dV are the sums of these parts over all row
    blocks (attention_backward is exactly that sum), so for causal attention
    the key rows j >= i0 of the last block's parts are already complete."""
    qh, kh, vh, doh = (np.asarray(a, np.float64) for a in (qh, kh, vh, doh))
    beta = beta_of(alpha)
    rs = 1.0 / np.sqrt(qh.shape[-1])
    x = scores(qh[i0:i1], kh, alpha, causal, i0)
    t = np.maximum(x - np.asarray(tau_rows, np.float64)[:, None], 0.0)
    p = t ** beta
    u = np.where(t > 0.0, t ** (beta - 1.0), 0.0)
    dp = doh[i0:i1] @ vh.T
    delta = np.sum(u * dp, axis=-1) / np.sum(u, axis=-1)
    ds = u * (dp - delta[:, None])
    return (ds @ kh) * rs, (ds.T @ qh[i0:i1]) * rs, p.T @ doh[i0:i1]


def attention_forward(q, k, v, alpha: float, causal: bool, return_probs: bool = False,
                      workers: int = 0):
    """Forward: returns (out, tau[, P]) in float64 with the leading shape of q.

    Works one head at a time, over blocks of at most 256 query rows, so memory
    stays at 256 x N scores per worker.  ``workers`` threads share the blocks
    (numpy's sort and matmul release the interpreter lock).
    """
    lead = np.shape(q)[:-2]
    qh, kh, vh = _heads(q), _heads(k), _heads(v)
    nh, n, d = qh.shape
    out = np.zeros((nh, n, vh.shape[-1]))
    tau = np.zeros((nh, n))
    probs = np.zeros((nh, n, n)) if return_probs else None

    def block(job):
        h, i0 = job
        i1 = min(n, i0 + ROW_BLOCK)
        o, t, p = forward_rows(qh[h], kh[h], vh[h], alpha, causal, i0, i1)
        tau[h, i0:i1] = t
        out[h, i0:i1] = o
        if probs is not None:
            probs[h, i0:i1] = p

    jobs = [(h, i0) for h in range(nh) for i0 in range(0, n, ROW_BLOCK)]
    with ThreadPoolExecutor(_workers(workers)) as ex:
        list(ex.map(block, jobs))
    res = (out.reshape(lead + out.shape[1:]), tau.reshape(lead + (n,)))
    if return_probs:
        res = res + (probs.reshape(lead + (n, n)),)
    return res


def attention_backward(q, k, v, dout, alpha: float, causal: bool, tau=None, workers: int = 0):
    """Backward: returns (dq, dk, dv) in float64.

    tau defaults to the oracle's own exact tau (never a value from elsewhere
    unless the caller passes it explicitly for an oracle-internal check).
    """
    lead = np.shape(q)[:-2]
    qh, kh, vh, doh = _heads(q), _heads(k), _heads(v), _heads(dout)
    nh, n, d = qh.shape
    if tau is None:
        tau = attention_forward(q, k, v, alpha, causal, workers=workers)[1]
    tauh = np.asarray(tau, dtype=np.float64).reshape(nh, n)
    dq = np.zeros_like(qh)
    dk = np.zeros((nh,) + kh.shape[1:])
    dv = np.zeros((nh,) + vh.shape[1:])

    def head(h):
        for i0 in range(0, n, ROW_BLOCK):
            i1 = min(n, i0 + ROW_BLOCK)
            gq, gk, gv = backward_rows(qh[h], kh[h], vh[h], doh[h], tauh[h, i0:i1], alpha, causal, i0, i1)
            dq[h, i0:i1] = gq
            dk[h] += gk
            dv[h] += gv

    with ThreadPoolExecutor(_workers(workers)) as ex:
        list(ex.map(head, range(nh)))
    shp = lambda a: a.reshape(lead + a.shape[1:])
    return shp(dq), shp(dk), shp(dv)


def tile_margins(q, k, alpha: float, causal: bool, tau, bm: int, bn: int):
    """Per (query tile, key tile): max over visible entries of x_ij - tau_i.

    A tile is active (holds a nonzero probability) exactly when its margin is
    > 0; -inf marks tiles with no visible entry.  Shape [..., ceil(N/bm), ceil(N/bn)].
    """
    lead = np.shape(q)[:-2]
    qh, kh = _heads(q), _heads(k)
    nh, n, _ = qh.shape
    tauh = np.asarray(tau, dtype=np.float64).reshape(nh, n)
    nqt, nkt = -(-n // bm), -(-n // bn)
    m = np.full((nh, nqt, nkt), -np.inf)
    for h in range(nh):
        for qt in range(nqt):
            i0, i1 = qt * bm, min(n, qt * bm + bm)
            x = scores(qh[h, i0:i1], kh[h], alpha, causal, i0) - tauh[h, i0:i1, None]
            colmax = np.max(x, axis=0)                       # per key, over the tile's rows
            pad = np.full(nkt * bn - n, -np.inf)
            m[h, qt] = np.max(np.concatenate([colmax, pad]).reshape(nkt, bn), axis=1)
    return m.reshape(lead + (nqt, nkt))


def element_sparsity(q, k, alpha: float, causal: bool, tau) -> float:
    """Fraction of visible score entries with zero probability."""
    qh, kh = _heads(q), _heads(k)
    nh, n, _ = qh.shape
    tauh = np.asarray(tau, dtype=np.float64).reshape(nh, n)
    zeros = 0
    visible = 0
    for h in range(nh):
        for i0 in range(0, n, ROW_BLOCK):
            i1 = min(n, i0 + ROW_BLOCK)
            x = scores(qh[h, i0:i1], kh[h], alpha, causal, i0)
            vis = np.isfinite(x)
            visible += int(vis.sum())
            zeros += int((vis & (x <= tauh[h, i0:i1, None])).sum())
    return zeros / max(visible, 1)
