"""Seeded generators: reproducible, bf16-exact, and with the stated structure."""
import numpy as np
import torch

from gen import inputs as G


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    x[:4] = [0.0, -0.0, np.inf, -np.inf]
    ours = G.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_reproducible_and_subset():
    w = G.workload("iid_causal_4k", N=96, H=3, B=2)
    a = G.make_inputs(w)
    b = G.make_inputs(w)
    for key in a:
        assert np.array_equal(a[key], b[key])
        assert np.array_equal(G.bf16_round(a[key]), a[key])      # bf16-exact
    sub = G.make_inputs(w, heads=slice(2, 4))
    assert np.array_equal(sub["k"], a["k"].reshape(6, 96, 64)[2:4])


def test_planted_structure():
    w = G.workload("planted_16k", N=1024, H=2)
    x = G.make_inputs(w)
    q, k = x["q"][0, 0], x["k"][0, 0]
    same = np.sum(q[0] * k[1]) / np.sqrt(128)          # both in cluster 0
    other = np.sum(q[0] * k[300]) / np.sqrt(128)        # cluster 1
    assert same > 30 and abs(other) < same / 2
    span = G.workload("planted_32k", N=1100, H=1)
    assert span.span == 512


def test_reference_shapes():
    assert G.WORKLOADS["small_f32"].dtype == "f32"
    w = G.WORKLOADS["planted_16k"]
    assert (w.B, w.H, w.N, w.d, w.causal, w.alpha) == (1, 16, 16384, 128, True, 1.5)
    w = G.WORKLOADS["encoder_8k"]
    assert (w.B, w.H, w.N, w.d, w.causal) == (2, 32, 8192, 64, False)
    w = G.WORKLOADS["planted_32k"]
    assert (w.B, w.H, w.N, w.d, w.causal) == (1, 8, 32768, 128, True)
