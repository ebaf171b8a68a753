#!/usr/bin/env python3
"""Benchmark: fused alpha-entmax attention, forward + backward, on one MI355X.

One step = the whole hot path over one batch: entmax_attn_fwd (row and tile
maxima, tau solve with block mask, P V) followed by entmax_attn_bwd (delta and
dQ, then dK/dV), inputs resident in HBM before timing starts.

Default workload (the one the headline metric is quoted on): B=1, H=16,
N=16384, d=128, bf16, causal, alpha=1.5, planted-cluster locality (64 random
centroids sqrt(d)*u_k, cluster of token i = (i // 256) % 64, Q = 3c + N(0,1),
K = c + 0.3 N(0,1), V, dO ~ N(0,1)), seed 0.

Reported value: dense-equivalent TFLOP/s = 3.5 * 4*B*H*N^2*d*(1/2 causal) per
step / step time.  The line also carries ms/step, the measured block sparsity
(32x64 and 128x64 tiles), per-stage times from HIP events recorded by the
library on the launch stream (for bf16 the "tau" stage includes P V, and "pv"
is empty), the roofline of the dominant kernel and the float64 CPU oracle
timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak
HBM_PEAK_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "adaptive_sparse_flash_amd", "csrc", "entmax_attn.hip")
COUNTER_SUMMARY = os.path.join(ROOT, "profiles", "k_rowmax16_planted_16k_hbm_counters.md")


def recorded_traffic(summary: str = COUNTER_SUMMARY, src: str = KERNEL_SRC):
    """HBM bytes per row-max launch from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE scaled by a plain copy), or None when the
    counters were taken on a different kernel source."""
    try:
        text = open(summary).read()
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    vals = dict(re.findall(r"^(\w+) = (\S+)$", text, re.M))
    if vals.get("kernel_source_sha256") != digest or "traffic_bytes_per_launch" not in vals:
        return None
    return float(vals["traffic_bytes_per_launch"])


def dense_equiv_flops(w) -> float:
    cf = 0.5 if w.causal else 1.0
    fwd = 4.0 * w.B * w.H * w.N * w.N * w.d * cf
    return 3.5 * fwd


def visible_fraction_tiles(n, bm, bn, causal):
    nq, nk = -(-n // bm), -(-n // bn)
    vis = np.ones((nq, nk), dtype=bool)
    if causal:
        for qt in range(nq):
            last = min(n - 1, qt * bm + bm - 1)
            vis[qt, last // bn + 1:] = False
    return vis


def block_sparsity(mask: np.ndarray, n: int, causal: bool, group: int):
    """Sparsity over causally visible tiles after OR-ing `group` mask rows."""
    nh, nq, nk = mask.shape
    m = mask.astype(bool)
    if group > 1:
        pad = (-nq) % group
        if pad:
            m = np.concatenate([m, np.zeros((nh, pad, nk), bool)], axis=1)
        m = m.reshape(nh, -1, group, nk).any(axis=2)
    vis = visible_fraction_tiles(n, 32 * group, 64, causal)
    act = m[:, :vis.shape[0], :] & vis[None]
    return 1.0 - act.sum() / (vis.sum() * nh)


class HipEvents:
    """hipEvent_t handles from the HIP runtime already loaded by torch."""

    def __init__(self, count: int):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(count):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(e.value)
        self.arr = (ctypes.c_void_p * count)(*self.ev)

    def block(self, i: int, n: int):
        return ctypes.cast(ctypes.byref(self.arr, i * n * ctypes.sizeof(ctypes.c_void_p)),
                           ctypes.POINTER(ctypes.c_void_p))

    def elapsed_ms(self, a: int, b: int) -> float:
        out = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(out), self.ev[a], self.ev[b]) != 0:
            return float("nan")
        return out.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


def cpu_baseline(w, x, max_heads: int, min_seconds: float = 10.0):
    """Time the float64 oracle (forward + backward) on whole heads of the
    workload, one after another on this host's cores, until at least
    `min_seconds` have been spent or `max_heads` heads are done, and scale to
    a dense-equivalent rate."""
    from oracle import entmax_oracle as O

    cores = len(os.sched_getaffinity(0))
    qa, ka, va, da = (x[n].reshape(-1, w.N, w.d) for n in ("q", "k", "v", "dout"))
    dt, heads = 0.0, 0
    while heads < min(max_heads, w.B * w.H) and (heads == 0 or dt < min_seconds):
        sl = slice(heads, heads + 1)
        t0 = time.perf_counter()
        _, tau = O.attention_forward(qa[sl], ka[sl], va[sl], w.alpha, w.causal, workers=cores)
        O.attention_backward(qa[sl], ka[sl], va[sl], da[sl], w.alpha, w.causal, tau=tau, workers=cores)
        dt += time.perf_counter() - t0
        heads += 1
    flops = dense_equiv_flops(w) * heads / (w.B * w.H)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"float64 oracle forward+backward on {heads} of {w.B * w.H} heads "
                      f"(full N={w.N}), {dt:.1f} s; rate scaled to the whole step"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="planted_16k")
    ap.add_argument("--tau-mode", default="hist", choices=["hist", "halley", "bisect"])
    ap.add_argument("--cpu-heads", type=int, default=4,
                    help="most heads the CPU oracle is timed on, one after another until 10 s are spent "
                         "(0 = skip)")
    ap.add_argument("--strength", type=float, default=None,
                    help="planted workloads: query strength a (Q = a*c + noise); sets the sparsity")
    ap.add_argument("--alpha", type=float, default=None, help="override the workload's alpha")
    ap.add_argument("--scale", type=float, default=None,
                    help="iid workloads: standard deviation c of Q and K (sets the sparsity)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one plain 512 MiB device copy first (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(every (batch, head) is independent; see the sharding notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    import adaptive_sparse_flash_amd as A
    from gen import inputs as G

    over = {}
    if args.strength is not None:
        over["strength"] = args.strength
    if args.alpha is not None:
        over["alpha"] = args.alpha
    if args.scale is not None:
        over["scale"] = args.scale
    w = G.workload(args.workload, **over)
    x = G.make_inputs(w)
    dt_in = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    q, k, v, do = (torch.from_numpy(x[n]).to(dt_in).to(dev) for n in ("q", "k", "v", "dout"))
    bufs = A.Buffers(w.B, w.H, w.N, w.d, dt_in, dt_in, args.tau_mode, device=dev)
    ns = A.binding.EA_NUM_STAGES if hasattr(A.binding, "EA_NUM_STAGES") else 6

    def step():
        bufs.forward(q, k, v, w.alpha, w.causal)
        bufs.backward(q, k, v, do, w.alpha, w.causal)

    if args.copy_calibration:
        # 512 MiB read + 512 MiB written by one elementwise copy kernel
        src = torch.ones(128 * 1024 * 1024, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = HipEvents(2 * ns * args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        bufs.desc.events = ev.block(s, 2 * ns)
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    bufs.desc.events = None
    ms = (t1 - t0) / args.steps * 1e3
    stage_ms = {}
    for si, name in enumerate(A.binding.STAGES):
        vals = [ev.elapsed_ms(s * 2 * ns + 2 * si, s * 2 * ns + 2 * si + 1) for s in range(args.steps)]
        stage_ms[name] = float(np.mean(vals))
    ev.close()

    mask = bufs.mask.cpu().numpy().reshape(w.B * w.H, *bufs.mask.shape[2:])
    iters = bufs.iters.cpu().numpy()
    sp32 = block_sparsity(mask, w.N, w.causal, 1)
    sp128 = block_sparsity(mask, w.N, w.causal, 4)
    flops = dense_equiv_flops(w)
    value = flops / (ms * 1e-3) / 1e12

    # Dominant kernel: the row-max sweep (k_rowmax16 for bf16), the one full
    # score sweep.  Its algorithmic work per launch is 2*d flops per visible
    # score: B*H*N*(N+1)/2 visible scores when causal, B*H*N^2 otherwise.
    vis = w.N * (w.N + 1) / 2 if w.causal else float(w.N) * w.N
    sweep_flops = 2.0 * w.d * vis * w.B * w.H
    rm_ms = stage_ms["rowmax"]
    achieved = sweep_flops / (rm_ms * 1e-3) / 1e12
    default_config = (args.workload == "planted_16k" and args.strength is None and args.alpha is None
                      and args.scale is None and args.tau_mode == "hist")
    roofline = {"bound": "mfma", "kernel": "k_rowmax16" if w.dtype == "bf16" else "k_rowmax",
                "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                "traffic": recorded_traffic() if default_config else None,
                "flops_per_launch": sweep_flops, "launch_ms": rm_ms}

    line = {
        "metric": "fwd+bwd dense-equivalent TFLOP/s (alpha=1.5 entmax attention, N=16k, 1 GPU)",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype} "
                        f"{'causal' if w.causal else 'non-causal'} alpha={w.alpha} {w.gen}"
                        + (f" span={w.span} strength={w.strength}" if w.gen == "planted" else f" scale={w.scale}"),
            "tau_mode": args.tau_mode,
            "block_sparsity_32x64": sp32,
            "block_sparsity_128x64": sp128,
            "tau_iters_mean": float(iters.mean()),
            "tau_iters_max": int(iters.max()),
            "stage_ms": stage_ms,
        },
        "roofline": roofline,
    }
    if args.cpu_heads > 0:
        line["cpu_baseline"] = cpu_baseline(w, x, args.cpu_heads)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
