"""Host-side pieces of bench.py: sparsity accounting, the dense-equivalent
flop count and the guard on recorded HBM traffic."""
import hashlib

import numpy as np

import bench
from gen import inputs as G


def test_dense_equivalent_flops():
    w = G.workload("planted_16k")
    # 3.5 x forward (4 B H N^2 d, halved when causal)
    assert bench.dense_equiv_flops(w) == 3.5 * 4 * 1 * 16 * 16384 ** 2 * 128 * 0.5
    e = G.workload("encoder_8k")
    assert bench.dense_equiv_flops(e) == 3.5 * 4 * 2 * 32 * 8192 ** 2 * 64


def test_block_sparsity_counts_visible_tiles_only():
    n = 256                     # 8 query tiles of 32, 4 key tiles of 64
    vis = bench.visible_fraction_tiles(n, 32, 64, True)
    assert vis.sum() == sum(min(qt * 32 + 31, n - 1) // 64 + 1 for qt in range(8))
    full = vis[None].astype(np.uint8)
    assert bench.block_sparsity(full, n, True, 1) == 0.0
    diag = np.zeros_like(full)
    for qt in range(8):
        diag[0, qt, (qt * 32) // 64] = 1
    assert np.isclose(bench.block_sparsity(diag, n, True, 1), 1 - 8 / vis.sum())
    # OR of 4 mask rows: 128x64 tiles
    vis4 = bench.visible_fraction_tiles(n, 128, 64, True)
    assert np.isclose(bench.block_sparsity(diag, n, True, 4), 1 - 4 / vis4.sum())


def test_recorded_traffic_requires_matching_source(tmp_path):
    src = tmp_path / "k.hip"
    src.write_bytes(b"kernel text")
    digest = hashlib.sha256(b"kernel text").hexdigest()
    summ = tmp_path / "s.md"
    summ.write_text(f"x\nkernel_source_sha256 = {digest}\ntraffic_bytes_per_launch = 1.5e8\n")
    assert bench.recorded_traffic(str(summ), str(src)) == 1.5e8
    src.write_bytes(b"changed kernel")
    assert bench.recorded_traffic(str(summ), str(src)) is None
    assert bench.recorded_traffic(str(tmp_path / "missing.md"), str(src)) is None


def test_cpu_baseline_sample_is_bounded():
    """The oracle is timed on whole heads, one after another, until the time
    floor is reached or the head cap is hit; the reported rate covers exactly
    the heads that ran."""
    w = G.workload("iid_causal_4k", B=1, H=3, N=96)
    x = G.make_inputs(w)
    one = bench.cpu_baseline(w, x, max_heads=4, min_seconds=0.0)
    assert "on 1 of 3 heads" in one["sample"] and one["kind"] == "oracle" and one["value"] > 0
    capped = bench.cpu_baseline(w, x, max_heads=2, min_seconds=1e9)
    assert "on 2 of 3 heads" in capped["sample"]
    every = bench.cpu_baseline(w, x, max_heads=10, min_seconds=1e9)
    assert "on 3 of 3 heads" in every["sample"]


def test_micro_sparsity_reads_half_bits():
    n = 128                      # 4 query rows of 32, 2 key tiles of 64 = 4 micro columns
    m = np.zeros((1, 4, 2), np.uint8)
    m[0, 0, 0] = 1 | 2           # row 0: keys 0-31 only
    m[0, 3, 1] = 1 | 2 | 4       # row 3: keys 64-127
    vis = bench.visible_fraction_tiles(n, 32, 32, True)
    assert vis.sum() == 1 + 2 + 3 + 4
    assert np.isclose(bench.micro_sparsity(m, n, True), 1 - 3 / 10)
    assert np.isclose(bench.block_sparsity(m, n, True, 1), 1 - 2 / bench.visible_fraction_tiles(n, 32, 64, True).sum())
