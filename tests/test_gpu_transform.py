"""GPU parity of the stand-alone row-wise entmax transform (entmax_rows,
called through the C ABI) against the float64 oracle: tau, p, the support and
sum p = 1, for row lengths held in registers (n <= 1024, n <= 4096) and
streamed (n > 4096), every alpha kind, the three tau modes, fp32 and bf16
scores and outputs, masked (-inf) entries, tied and one-hot rows."""
import numpy as np
import pytest
import torch

import adaptive_sparse_flash_amd as A
from gen import inputs as G
from oracle import entmax_oracle as O
from tests import parity as PT

pytestmark = pytest.mark.gpu


def run_rows(s, alpha, mode, out_dtype=torch.float32, in_dtype=torch.float32):
    st = torch.from_numpy(s).to(in_dtype).cuda()
    p, tau, it = A.entmax_transform(st, alpha, mode, out_dtype)
    torch.cuda.synchronize()
    return p.float().cpu().numpy(), tau.cpu().numpy(), it.cpu().numpy()


def check_rows(s, alpha, p, tau, it, tol):
    x = (alpha - 1.0) * s.astype(np.float64)
    tau_ref = O.tau_exact(x, alpha)
    p_ref = O.entmax_probs(x, tau_ref, alpha)
    PT.check_tau(tau, tau_ref)
    PT.check_close("p", p, p_ref, tol)
    diff = (x > tau[:, None]) != (x > tau_ref[:, None])
    assert np.all(np.abs(x - tau_ref[:, None])[diff] <= PT.SUPPORT_BAND), "support differs"
    assert np.all(np.abs(p.sum(axis=1) - 1.0) <= max(tol, 1e-5))
    assert np.all(it >= 1)
    return tau_ref


@pytest.mark.parametrize("n", [1, 3, 100, 1023, 1024, 1025, 4096, 5000, 20000])
@pytest.mark.parametrize("mode", ["hist", "halley", "bisect"])
def test_rows_lengths_and_modes(n, mode):
    rows = 64 if n <= 5000 else 16
    s = G.make_score_rows(rows, n, scale=2.0, seed=n)
    print(f"\n[rows] n={n} rows={rows} mode={mode}", flush=True)
    p, tau, it = run_rows(s, 1.5, mode)
    check_rows(s, 1.5, p, tau, it, 1e-4)
    print(f"  sweeps mean {it.mean():.2f} max {it.max()}", flush=True)


@pytest.mark.parametrize("alpha", [1.25, 1.5, 1.75, 2.0, 1.1])
def test_rows_alpha_kinds(alpha):
    for n in (700, 3000, 9000):
        s = G.make_score_rows(32, n, scale=3.0, seed=7)
        for mode in ("hist", "halley"):
            p, tau, it = run_rows(s, alpha, mode)
            check_rows(s, alpha, p, tau, it, 1e-4)


def test_rows_bf16_in_and_out():
    s = G.make_score_rows(64, 2048, scale=2.0, seed=3, dtype="bf16")
    p, tau, it = run_rows(s, 1.5, "hist", in_dtype=torch.bfloat16)
    check_rows(s, 1.5, p, tau, it, 1e-4)
    pb, taub, _ = run_rows(s, 1.5, "hist", out_dtype=torch.bfloat16, in_dtype=torch.bfloat16)
    np.testing.assert_array_equal(taub, tau)
    PT.check_close("p(bf16)", pb, p, 1e-2)


def test_rows_masked_tied_onehot():
    n = 1500
    s = G.make_score_rows(8, n, scale=2.0, seed=11, masked=0.3)
    s[1, :] = -np.inf                     # nothing visible: tau = +inf, p = 0
    s[2, :] = 0.25                        # all tied: p = 1/n
    s[3, :] = -np.inf
    s[3, 17] = 1.0                        # one visible entry: p = 1
    s[4, :] = -3.0
    s[4, 5] = 3.0                         # one-hot: the top leads by more than 1/(alpha-1)
    p, tau, it = run_rows(s, 1.5, "hist")
    assert np.isposinf(tau[1]) and np.all(p[1] == 0.0)
    np.testing.assert_allclose(p[2], 1.0 / n, rtol=1e-4)
    assert p[3, 17] == pytest.approx(1.0, abs=1e-6) and p[3].sum() == pytest.approx(1.0, abs=1e-6)
    assert p[4, 5] == pytest.approx(1.0, abs=1e-6)
    keep = [0, 2, 3, 4, 5, 6, 7]
    check_rows(s[keep], 1.5, p[keep], tau[keep], it[keep], 1e-4)


def test_rows_empty():
    s = np.zeros((0, 64), np.float32)
    p, tau, it = run_rows(s, 1.5, "hist")
    assert p.shape == (0, 64)


def test_rows_histogram_iterations():
    """On attention-like rows the histogram start leaves at most two sweeps,
    Halley-bisection from the lower end a few, bisection about twenty."""
    s = G.make_score_rows(256, 4096, scale=2.0, seed=5)
    its = {m: run_rows(s, 1.5, m)[2] for m in ("hist", "halley", "bisect")}
    print({m: (float(v.mean()), int(v.max())) for m, v in its.items()}, flush=True)
    assert its["hist"].max() <= 2
    assert its["halley"].mean() < its["bisect"].mean() / 3
    assert its["bisect"].mean() >= 15
