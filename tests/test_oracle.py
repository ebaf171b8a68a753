"""Pins for the float64 oracle: it is checked against facts fixed by the
mathematics (brute force, closed forms, the variational definition solved by a
library optimiser, limits, invariants, finite differences), never against
itself or the GPU path."""
import ast
import itertools
import json
import math
import operator
import os

import numpy as np
import pytest
import torch
from scipy.optimize import brentq, minimize

from oracle import entmax_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


# ---------------------------------------------------------------- helpers ---

_OPS = {ast.Add: operator.add, ast.Sub: operator.sub, ast.Mult: operator.mul,
        ast.Div: operator.truediv, ast.Pow: operator.pow, ast.USub: operator.neg}


def _eval(expr: str) -> float:
    """Evaluate a closed-form expression with + - * / ** and sqrt only."""
    def ev(n):
        if isinstance(n, ast.Expression):
            return ev(n.body)
        if isinstance(n, ast.Constant):
            return float(n.value)
        if isinstance(n, ast.BinOp):
            return _OPS[type(n.op)](ev(n.left), ev(n.right))
        if isinstance(n, ast.UnaryOp):
            return _OPS[type(n.op)](ev(n.operand))
        if isinstance(n, ast.Call) and n.func.id == "sqrt":
            return math.sqrt(ev(n.args[0]))
        raise ValueError(expr)
    return ev(ast.parse(expr, mode="eval"))


def brute_force_tau(x, alpha):
    """Enumerate every nonempty support S, solve the restricted equation
    sum_{j in S} (x_j - tau)^beta = 1 on its own, keep the self-consistent
    supports (x_j > tau inside, x_j <= tau outside).  Returns all solutions."""
    x = np.asarray(x, dtype=np.float64)
    n = len(x)
    beta = 1.0 / (alpha - 1.0)
    sols = []
    for r in range(1, n + 1):
        for S in itertools.combinations(range(n), r):
            xs = x[list(S)]
            if alpha == 2.0:
                tau = (xs.sum() - 1.0) / r
            elif alpha == 1.5:
                # r tau^2 - 2 tau sum x + sum x^2 - 1 = 0, smaller root
                a, b, c = r, -2.0 * xs.sum(), (xs ** 2).sum() - 1.0
                disc = b * b - 4 * a * c
                if disc < 0:
                    continue
                tau = (-b - math.sqrt(disc)) / (2 * a)
            else:
                g = lambda t: np.sum((xs - t) ** beta) - 1.0
                lo_, hi_ = xs.min() - 10.0, xs.min()
                if g(lo_) < 0 or g(hi_) > 0:
                    continue
                tau = brentq(g, lo_, hi_, xtol=1e-15, rtol=1e-15)
            rest = np.delete(x, list(S))
            if np.all(xs > tau) and np.all(rest <= tau + 1e-14):
                sols.append(tau)
    return sols


def softmax(s):
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


# -------------------------------------------------------------- tau pins ---

def test_golden_closed_forms():
    cases = json.load(open(GOLDEN))["cases"]
    assert len(cases) >= 8
    for c in cases:
        s = np.array(c["s"], dtype=np.float64)
        x = (c["alpha"] - 1.0) * s
        tau = O.tau_exact(x[None, :], c["alpha"])[0]
        assert tau == pytest.approx(_eval(c["tau"]), abs=1e-11), c["name"]
        p = O.entmax(s[None, :], c["alpha"])[0]
        want = np.array([_eval(e) for e in c["p"]])
        np.testing.assert_allclose(p, want, atol=1e-11, err_msg=c["name"])


@pytest.mark.parametrize("alpha", [1.5, 2.0, 1.25, 1.75, 1.1])
def test_brute_force_small_rows(alpha):
    rng = np.random.default_rng(1)
    for n in range(1, 9):
        for _ in range(12):
            x = rng.standard_normal(n) * rng.choice([0.3, 1.0, 3.0])
            sols = brute_force_tau(x, alpha)
            assert len(sols) == 1, (x, sols)
            tau = O.tau_exact(x[None, :], alpha)[0]
            assert tau == pytest.approx(sols[0], abs=1e-10)


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_sort_matches_bisection(alpha):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 300)) * 2.0
    x[:, 200:] = -np.inf                       # ragged visible lengths
    x[5, 1:] = -np.inf                         # single visible key
    a = O.tau_sort(x, alpha)
    b = O.tau_bisect(x, alpha)
    np.testing.assert_allclose(a, b, atol=1e-11)


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0, 1.9])
def test_invariants(alpha):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((32, 97)) * 1.7
    tau = O.tau_exact(x, alpha)
    p = O.entmax_probs(x, tau, alpha)
    assert np.all(p >= 0)
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-12)
    lo, hi = O.tau_bracket(x, alpha)
    assert np.all(tau >= lo - 1e-12) and np.all(tau <= hi + 1e-12)
    # shifting every score by c moves tau by (alpha-1) c and leaves p unchanged
    s = x / (alpha - 1.0)
    p2 = O.entmax(s + 3.25, alpha)
    np.testing.assert_allclose(p2, p, atol=1e-11)
    tau2 = O.tau_exact((alpha - 1.0) * (s + 3.25), alpha)
    np.testing.assert_allclose(tau2 - tau, (alpha - 1.0) * 3.25, atol=1e-11)


def test_special_rows():
    for alpha in (1.25, 1.5, 2.0):
        # one key: tau = x - 1
        assert O.tau_exact(np.array([[0.7]]), alpha)[0] == pytest.approx(-0.3, abs=1e-12)
        # n equal keys: uniform p, tau = x - n^(1-alpha)
        x = np.full((1, 7), 0.2)
        np.testing.assert_allclose(O.entmax_probs(x, O.tau_exact(x, alpha), alpha), 1 / 7, atol=1e-12)
        assert O.tau_exact(x, alpha)[0] == pytest.approx(0.2 - 7 ** (1 - alpha), abs=1e-12)


@pytest.mark.parametrize("alpha", [1.5, 2.0, 1.25])
def test_variational_definition(alpha):
    """entmax_alpha(s) = argmax_{p in simplex} p.s + H_alpha(p) with the Tsallis
    entropy H_alpha(p) = sum(p - p^alpha) / (alpha (alpha-1)); solved by a
    library optimiser.  Pins the (alpha-1) scaling and the threshold convention."""
    rng = np.random.default_rng(4)
    for _ in range(6):
        s = rng.standard_normal(5) * 1.5
        def neg(p):
            p = np.maximum(p, 0)
            return -(p @ s + np.sum(p - p ** alpha) / (alpha * (alpha - 1)))
        res = minimize(neg, np.full(5, 0.2), method="SLSQP",
                       bounds=[(0, 1)] * 5,
                       constraints=[{"type": "eq", "fun": lambda p: p.sum() - 1}],
                       options={"ftol": 1e-14, "maxiter": 500})
        np.testing.assert_allclose(O.entmax(s[None], alpha)[0], res.x, atol=2e-5)


def test_sparsemax_is_simplex_projection():
    """alpha = 2 is the Euclidean projection of s onto the simplex."""
    rng = np.random.default_rng(5)
    for _ in range(6):
        s = rng.standard_normal(6)
        res = minimize(lambda p: np.sum((p - s) ** 2), np.full(6, 1 / 6), method="SLSQP",
                       bounds=[(0, 1)] * 6,
                       constraints=[{"type": "eq", "fun": lambda p: p.sum() - 1}],
                       options={"ftol": 1e-15, "maxiter": 500})
        np.testing.assert_allclose(O.entmax(s[None], 2.0)[0], res.x, atol=1e-6)


def test_softmax_limit():
    rng = np.random.default_rng(6)
    s = rng.standard_normal((4, 40))
    errs = []
    for eps in (1e-2, 1e-3, 1e-4):
        p = O.entmax(s, 1.0 + eps)
        errs.append(np.abs(p - softmax(s)).max())
    assert errs[1] < errs[0] / 5 and errs[2] < errs[1] / 5
    assert errs[2] < 1e-3


# --------------------------------------------------------- attention pins ---

def _tiny(seed, n=7, d=3, scale=1.5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((2, n, d)) * scale
    k = rng.standard_normal((2, n, d)) * scale
    v = rng.standard_normal((2, n, d + 1))
    do = rng.standard_normal((2, n, d + 1))
    return q, k, v, do


@pytest.mark.parametrize("alpha,causal", [(1.5, False), (1.5, True), (2.0, False), (1.25, True), (1.75, False)])
def test_forward_matches_dense_definition(alpha, causal):
    q, k, v, _ = _tiny(7)
    out, tau, P = O.attention_forward(q, k, v, alpha, causal, return_probs=True)
    for h in range(2):
        s = q[h] @ k[h].T / math.sqrt(q.shape[-1])
        if causal:
            s = np.where(np.tril(np.ones_like(s)) > 0, s, -np.inf)
        for i in range(s.shape[0]):
            vis = np.isfinite(s[i])
            sols = brute_force_tau((alpha - 1) * s[i, vis], alpha)
            assert len(sols) == 1
            assert tau[h, i] == pytest.approx(sols[0], abs=1e-10)
        np.testing.assert_allclose(out[h], P[h] @ v[h], atol=1e-12)
        np.testing.assert_allclose(P[h].sum(-1), 1.0, atol=1e-12)
        if causal:
            assert np.all(np.triu(P[h], 1) == 0)
            assert P[h][0, 0] == pytest.approx(1.0)


def _loss(q, k, v, do, alpha, causal):
    out, _ = O.attention_forward(q, k, v, alpha, causal)
    return float(np.sum(out * do))


@pytest.mark.parametrize("alpha,causal", [(1.5, False), (1.5, True), (2.0, True), (1.25, False), (1.6, True)])
def test_backward_finite_differences(alpha, causal):
    q, k, v, do = _tiny(11, n=6, d=3, scale=0.9)
    dq, dk, dv = O.attention_backward(q, k, v, do, alpha, causal)
    # bisection (alpha not in {1.5, 2}) settles tau to 1e-12: keep eps well above it
    eps = 1e-5
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a1 = arr.copy(); a1[idx] += eps
            a2 = arr.copy(); a2[idx] -= eps
            args1 = {"q": q, "k": k, "v": v}; args1[name] = a1
            args2 = {"q": q, "k": k, "v": v}; args2[name] = a2
            num[idx] = (_loss(args1["q"], args1["k"], args1["v"], do, alpha, causal)
                        - _loss(args2["q"], args2["k"], args2["v"], do, alpha, causal)) / (2 * eps)
        np.testing.assert_allclose(grad, num, atol=2e-6 * max(1.0, np.abs(num).max()), err_msg=name)


def test_backward_row_sums_of_ds_vanish():
    """sum_j dS_ij = 0 (tau absorbs a uniform shift), so sum_j dK_j = 0."""
    q, k, v, do = _tiny(12, n=40, d=8)
    for alpha, causal in ((1.5, True), (2.0, False), (1.3, False)):
        _, dk, _ = O.attention_backward(q, k, v, do, alpha, causal)
        np.testing.assert_allclose(dk.sum(axis=-2), 0.0, atol=1e-10)
        _, _, dv = O.attention_backward(q, k, v, do, alpha, causal)
        np.testing.assert_allclose(dv.sum(axis=-2), do.sum(axis=-2), atol=1e-10)


def test_backward_softmax_limit_against_autograd():
    """Near alpha = 1 the gradients tend to softmax attention's (float64 torch autograd)."""
    q, k, v, do = _tiny(13, n=9, d=4, scale=0.7)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    p = torch.softmax(tq @ tk.transpose(-1, -2) / 2.0, dim=-1)
    (p @ tv).mul(torch.tensor(do)).sum().backward()
    errs = []
    for eps in (1e-2, 1e-3):
        g = O.attention_backward(q, k, v, do, 1.0 + eps, False)
        errs.append(max(np.abs(g[0] - tq.grad.numpy()).max(), np.abs(g[1] - tk.grad.numpy()).max(),
                        np.abs(g[2] - tv.grad.numpy()).max()))
    assert errs[1] < errs[0] / 5 and errs[1] < 5e-3


def test_backward_sparsemax_jacobian():
    """alpha = 2: dS = J dP with J = diag(1_S) - 1_S 1_S^T / |S| (support S)."""
    q, k, v, do = _tiny(14, n=8, d=3, scale=2.0)
    dq, dk, dv = O.attention_backward(q, k, v, do, 2.0, False)
    for h in range(2):
        s = q[h] @ k[h].T / math.sqrt(3)
        P = O.entmax(s, 2.0)
        dP = do[h] @ v[h].T
        dS = np.zeros_like(s)
        for i in range(8):
            m = (P[i] > 0).astype(float)
            J = np.diag(m) - np.outer(m, m) / m.sum()
            dS[i] = J @ dP[i]
        np.testing.assert_allclose(dq[h], dS @ k[h] / math.sqrt(3), atol=1e-12)
        np.testing.assert_allclose(dk[h], dS.T @ q[h] / math.sqrt(3), atol=1e-12)
        np.testing.assert_allclose(dv[h], P.T @ do[h], atol=1e-12)


def test_tile_margins_exact_active_set():
    q, k, v, _ = _tiny(15, n=37, d=5, scale=2.5)
    _, tau, P = O.attention_forward(q, k, v, 1.5, True, return_probs=True)
    m = O.tile_margins(q, k, 1.5, True, tau, 8, 16)
    assert m.shape == (2, 5, 3)
    for h in range(2):
        for qt in range(5):
            for kt in range(3):
                blk = P[h, qt * 8:qt * 8 + 8, kt * 16:kt * 16 + 16]
                assert (m[h, qt, kt] > 0) == bool(np.any(blk > 0))
    # causally invisible tiles carry -inf
    assert m[0, 0, 1] == -np.inf


def test_planted_mutation_is_caught():
    """A dropped delta term in the backward (a plausible slip) breaks the
    finite-difference pin: the pin is sensitive, not vacuous."""
    q, k, v, do = _tiny(16, n=5, d=2, scale=1.0)
    orig = O.attention_backward

    def mutated(q, k, v, dout, alpha, causal, tau=None, workers=0):
        qh, kh, vh, doh = (a.reshape((-1,) + a.shape[-2:]) for a in (q, k, v, dout))
        out = []
        for h in range(qh.shape[0]):
            x = O.scores(qh[h], kh[h], alpha, causal)
            t_ = O.tau_exact(x, alpha)
            t = np.maximum(x - t_[:, None], 0)
            u = np.where(t > 0, t ** (1 / (alpha - 1) - 1), 0)
            ds = u * (doh[h] @ vh[h].T)          # delta dropped
            out.append(ds @ kh[h] / math.sqrt(qh.shape[-1]))
        return np.stack(out)

    dq_bad = mutated(q, k, v, do, 1.5, False)
    dq_good = orig(q, k, v, do, 1.5, False)[0]
    assert np.abs(dq_bad - dq_good).max() > 1e-3


# ------------------------------------------- f and element sparsity pins ---

FSP = os.path.join(os.path.dirname(__file__), "golden", "f_and_sparsity.json")


def test_entmax_f_hand_values():
    """f at non-root points, solved by hand (tests/golden/f_and_sparsity.json):
    a dropped '- 1', a wrong exponent or a missing (alpha - 1) factor fails."""
    for c in json.load(open(FSP))["f_values"]:
        x = (c["alpha"] - 1.0) * np.asarray([c["s"]], dtype=np.float64)
        f = O.entmax_f(x, np.asarray([c["tau"]]), c["alpha"])
        assert f[0] == pytest.approx(_eval(c["f"]), abs=1e-12), c


def test_entmax_f_vanishes_at_golden_tau():
    """At the hand-derived tau of every closed-form example, f = 0."""
    for c in json.load(open(GOLDEN))["cases"]:
        x = (c["alpha"] - 1.0) * np.asarray([c["s"]], dtype=np.float64)
        f = O.entmax_f(x, np.asarray([_eval(c["tau"])]), c["alpha"])
        assert abs(f[0]) <= 1e-12, c["name"]


@pytest.mark.parametrize("alpha", [1.25, 1.5, 1.75, 2.0])
def test_entmax_f_bracket_signs(alpha):
    """f(max x - 1) >= 0 >= f(max x - n^(1-alpha)) (proved from the definition:
    the top term alone is 1 at the lower end, every term is at most 1/n at the
    upper end), and f decreases strictly between them."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 37)) * rng.uniform(0.1, 5.0, (64, 1))
    lo, hi = O.tau_bracket(x, alpha)
    assert np.all(O.entmax_f(x, lo, alpha) >= 0.0)
    assert np.all(O.entmax_f(x, hi, alpha) <= 1e-15)
    mid = 0.5 * (lo + hi)
    assert np.all(O.entmax_f(x, lo, alpha) > O.entmax_f(x, mid, alpha))
    assert np.all(O.entmax_f(x, mid, alpha) > O.entmax_f(x, hi, alpha))


def test_element_sparsity_hand_counts():
    """Hand counts of zero-probability visible entries on tiny d = 1 cases,
    with entries exactly on the threshold (which count as zeros: p = 0 there),
    causal and not, one and two heads."""
    for c in json.load(open(FSP))["element_sparsity"]:
        q, k, tau = (np.asarray(c[n], dtype=np.float64) for n in ("q", "k", "tau"))
        got = O.element_sparsity(q, k, c["alpha"], c["causal"], tau)
        assert got == pytest.approx(_eval(c["sparsity"]), abs=1e-15), c
