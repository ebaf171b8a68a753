#!/usr/bin/env python3
"""Benchmark: fused alpha-entmax attention, forward + backward, on one MI355X.

One step = the whole hot path over one batch: entmax_attn_fwd (row maxima and
block codes, tau solve with block mask, P V) followed by entmax_attn_bwd (delta
and dQ, then dK/dV), inputs resident in HBM before timing starts.  The timed
steps replay one HIP graph that holds a step's kernels (checked bit for bit
against an eager step first); the stage times come from a separate eager pass.

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
TRACE_SUMMARY = os.path.join(ROOT, "profiles", "k_rowmax16_planted_16k_kernel_trace.md")


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


def micro_sparsity(mask: np.ndarray, n: int, causal: bool):
    """Sparsity over causally visible 32x32 micro-tiles, from the half bits of
    the mask bytes (bit 1: keys 0-31 of the 64-key tile, bit 2: keys 32-63)."""
    nh, nq, nk = mask.shape
    m = mask.astype(np.uint8)
    halves = np.stack([(m >> 1) & 1, (m >> 2) & 1], axis=-1).astype(bool) & (m != 0)[..., None]
    halves = halves.reshape(nh, nq, 2 * nk)[:, :, :-(-n // 32)]
    vis = visible_fraction_tiles(n, 32, 32, causal)
    return 1.0 - (halves & vis[None]).sum() / (vis.sum() * nh)


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


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def recorded_kernel_us(summary: str = TRACE_SUMMARY, src: str = KERNEL_SRC):
    """Average duration (us) of the row-max kernel in the committed rocprofv3
    kernel trace, or None when the trace was taken on a different source."""
    try:
        text = open(summary).read()
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    vals = dict(re.findall(r"^(\w+) = (\S+)$", text, re.M))
    if vals.get("kernel_source_sha256") != digest or "rowmax_avg_us" not in vals:
        return None
    return float(vals["rowmax_avg_us"])


def describe(w) -> str:
    return (f"{w.name}: B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype} "
            f"{'causal' if w.causal else 'non-causal'} alpha={w.alpha} {w.gen}"
            + (f" span={w.span} strength={w.strength}" if w.gen == "planted" else f" scale={w.scale}"))


def element_sparsity_gpu(q, k, tau, alpha, causal, rows=4096):
    """Share of visible score entries with zero probability (x <= tau), from
    float32 scores recomputed by torch on the GPU chunk by chunk (a statistic
    for the report, not part of the attention path)."""
    import torch

    B, H, N, d = q.shape
    nz, vis = 0, 0
    scale = (alpha - 1.0) / float(np.sqrt(d))
    for b in range(B):
        for h in range(H):
            kf = k[b, h].float()
            for r0 in range(0, N, rows):
                r1 = min(N, r0 + rows)
                x = (q[b, h, r0:r1].float() @ kf.T) * scale
                keep = x > tau[b, h, r0:r1, None]
                if causal:
                    ii = torch.arange(r0, r1, device=x.device)[:, None]
                    jj = torch.arange(N, device=x.device)[None, :]
                    keep &= jj <= ii
                    vis += (r1 - r0) * (r0 + r1 + 1) // 2
                else:
                    vis += (r1 - r0) * N
                nz += int(keep.sum().item())
    return 1.0 - nz / max(vis, 1)


class Runner:
    """One workload's device inputs and buffers; measure() times fwd+bwd steps
    with HIP events per stage."""

    def __init__(self, A, torch, w, x, tau_mode, dev):
        self.A, self.torch, self.w = A, torch, w
        dt_in = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.q, self.k, self.v, self.do = (torch.from_numpy(x[n]).to(dt_in).to(dev)
                                           for n in ("q", "k", "v", "dout"))
        self.bufs = A.Buffers(w.B, w.H, w.N, w.d, dt_in, dt_in, tau_mode, device=dev)

    def step(self):
        w = self.w
        self.bufs.forward(self.q, self.k, self.v, w.alpha, w.causal)
        self.bufs.backward(self.q, self.k, self.v, self.do, w.alpha, w.causal)

    def capture(self):
        """One step (forward + backward) captured as a HIP graph, or None if a
        replay differs from the eager step.  The replays are checked bit for
        bit against an eager step on zeroed outputs, with eager steps between
        them."""
        torch = self.torch
        b = self.bufs
        outs = (b.out, b.tau, b.dq, b.dk, b.dv)
        self.step()
        torch.cuda.synchronize()
        ref = [t.clone() for t in outs]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.step()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step()
        torch.cuda.synchronize()
        for _ in range(2):
            for t in outs:
                t.zero_()
            g.replay()
            torch.cuda.synchronize()
            if not all(torch.equal(u, v) for u, v in zip(ref, outs)):
                return None
            self.step()
            torch.cuda.synchronize()
        return g

    def measure(self, steps, warmup, graph=True):
        """`warmup` eager steps, then exactly `steps` timed steps, each one
        replay of a HIP graph holding the step's kernels (eager launches if
        graph is False or the replay check fails).  Stage times come from a
        separate eager pass with the library's events."""
        torch, A = self.torch, self.A
        ns = A.binding.EA_NUM_STAGES
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        g = self.capture() if graph else None
        run_step = g.replay if g is not None else self.step
        launch = "hip_graph" if g is not None else "eager"
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            run_step()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        del g
        n_ev = max(1, min(steps, 10))
        ev = HipEvents(2 * ns * n_ev)
        torch.cuda.synchronize()
        te0 = time.perf_counter()
        for s in range(n_ev):
            self.bufs.desc.events = ev.block(s, 2 * ns)
            self.step()
        torch.cuda.synchronize()
        te1 = time.perf_counter()
        self.bufs.desc.events = None
        stage_ms = {}
        for si, name in enumerate(A.binding.STAGES):
            vals = [ev.elapsed_ms(s * 2 * ns + 2 * si, s * 2 * ns + 2 * si + 1) for s in range(n_ev)]
            stage_ms[name] = float(np.mean(vals))
        ev.close()
        w = self.w
        mask = self.bufs.mask.cpu().numpy().reshape(w.B * w.H, *self.bufs.mask.shape[2:])
        iters = self.bufs.iters.cpu().numpy()
        ms = (t1 - t0) / steps * 1e3
        return {"ms_per_step": ms, "tflops": dense_equiv_flops(w) / (ms * 1e-3) / 1e12,
                "launch": launch,
                "ms_per_step_eager": (te1 - te0) / n_ev * 1e3,
                "block_sparsity_32x32": micro_sparsity(mask, w.N, w.causal),
                "block_sparsity_32x64": block_sparsity(mask, w.N, w.causal, 1),
                "block_sparsity_128x64": block_sparsity(mask, w.N, w.causal, 4),
                "tau_iters_mean": float(iters.mean()), "tau_iters_max": int(iters.max()),
                "stage_ms": stage_ms}

    def element_sparsity(self):
        return element_sparsity_gpu(self.q, self.k, self.bufs.tau, self.w.alpha, self.w.causal)

    def close(self):
        del self.q, self.k, self.v, self.do, self.bufs
        self.torch.cuda.empty_cache()


def bench_transform(A, torch, G, dev, alpha=1.5, reps=10):
    """Stand-alone row-wise entmax (entmax_rows) on fp32 score rows
    s ~ N(0, 2^2) (x ~ N(0, 1) at alpha = 1.5): per tau mode the time per
    launch (HIP events on the launch stream, `reps` launches after 2 warm-up
    ones), algorithmic HBM bytes per second (read s, write p, tau and the
    sweep counts once) against the 8 TB/s peak, and sweeps per row."""
    res = []
    for rows, n in ((16384, 4096), (4096, 16384)):
        s = torch.from_numpy(G.make_score_rows(rows, n, scale=2.0, seed=1)).to(dev)
        p = torch.empty_like(s)
        tau = torch.empty(rows, dtype=torch.float32, device=dev)
        it = torch.empty(rows, dtype=torch.uint8, device=dev)
        byt = rows * n * 8 + rows * 5
        point = {"rows": rows, "n": n, "path": "registers" if n <= 4096 else "streamed", "modes": {}}
        for mode in ("hist", "halley", "bisect"):
            desc = A.make_rows_desc(rows, n, torch.float32, torch.float32, mode)
            for _ in range(2):
                A.entmax_rows(s, alpha, p, tau, it, desc)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                A.entmax_rows(s, alpha, p, tau, it, desc)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            itc = it.cpu().numpy()
            point["modes"][mode] = {"ms": ms, "gbs": byt / (ms * 1e-3) / 1e9,
                                    "hbm_frac": byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                    "sweeps_mean": float(itc.mean()), "sweeps_max": int(itc.max())}
        b = point["modes"]["bisect"]
        for mode in ("hist", "halley"):
            point["modes"][mode]["speedup_vs_bisect"] = b["ms"] / point["modes"][mode]["ms"]
            point["modes"][mode]["sweep_ratio_vs_bisect"] = b["sweeps_mean"] / max(point["modes"][mode]["sweeps_mean"], 1e-9)
        res.append(point)
        del s, p
    return {"alpha": alpha, "scores": "fp32 s ~ N(0, 4), dense rows", "points": res}


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
    ap.add_argument("--n", type=int, default=None, help="override the sequence length")
    ap.add_argument("--heads", type=int, default=None, help="override the head count")
    ap.add_argument("--extras", type=int, default=1,
                    help="1: also measure the sparsity sweep, the long-context tau modes and the "
                         "sequence-length scaling (after the headline timing); 0: headline only")
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

    torch.backends.cuda.matmul.allow_tf32 = False
    over = {}
    for key, val in (("strength", args.strength), ("alpha", args.alpha), ("scale", args.scale),
                     ("N", args.n), ("H", args.heads)):
        if val is not None:
            over[key] = val
    w = G.workload(args.workload, **over)
    x = G.make_inputs(w)
    dev = torch.device("cuda:0")
    run = Runner(A, torch, w, x, args.tau_mode, dev)

    if args.copy_calibration:
        # 512 MiB read + 512 MiB written by one elementwise copy kernel
        src = torch.ones(128 * 1024 * 1024, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- headline: exactly `steps` timed steps after `warmup` untimed ones
    head = run.measure(args.steps, args.warmup)
    ms, stage_ms = head["ms_per_step"], head["stage_ms"]
    value = head["tflops"]
    elem_sp = run.element_sparsity()
    ws_bytes = int(run.bufs.ws.numel())

    # Dominant kernel: the row-max sweep (k_rowmax16 for bf16), the one full
    # score sweep.  Its algorithmic work per launch is 2*d flops per visible
    # score: B*H*N*(N+1)/2 visible scores when causal, B*H*N^2 otherwise.
    vis = w.N * (w.N + 1) / 2 if w.causal else float(w.N) * w.N
    sweep_flops = 2.0 * w.d * vis * w.B * w.H
    rm_ms = stage_ms["rowmax"]
    achieved = sweep_flops / (rm_ms * 1e-3) / 1e12
    default_config = (args.workload == "planted_16k" and not over and args.tau_mode == "hist")
    rec_us = recorded_kernel_us() if default_config else None
    roofline = {"bound": "mfma", "kernel": "k_rowmax16" if w.dtype == "bf16" else "k_rowmax",
                "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                "traffic": recorded_traffic() if default_config else None,
                "flops_per_launch": sweep_flops, "launch_ms": rm_ms,
                "rocprof_avg_us": rec_us,
                "frac_rocprof": (sweep_flops / (rec_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS) if rec_us else None}

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
            "workload": describe(w),
            "tau_mode": args.tau_mode,
            "block_sparsity_32x32": head["block_sparsity_32x32"],
            "block_sparsity_32x64": head["block_sparsity_32x64"],
            "block_sparsity_128x64": head["block_sparsity_128x64"],
            "element_sparsity": elem_sp,
            "tau_iters_mean": head["tau_iters_mean"],
            "tau_iters_max": head["tau_iters_max"],
            "stage_ms": stage_ms,
            "launch": head["launch"],
            "ms_per_step_eager": head["ms_per_step_eager"],
            "workspace_bytes": ws_bytes,
        },
        "roofline": roofline,
    }
    run.close()

    if args.extras and default_config:
        # ---- throughput vs block sparsity: the same generator at weaker query
        # strengths (5 timed steps each after 2 warm-up steps)
        sweep = [dict(strength=w.strength, **{k_: head[k_] for k_ in (
            "ms_per_step", "tflops", "block_sparsity_32x32", "block_sparsity_32x64", "block_sparsity_128x64",
            "tau_iters_mean", "tau_iters_max", "stage_ms")}, element_sparsity=elem_sp)]
        for a in (0.5, 0.4, 0.3):
            wa = w.with_(strength=a)
            r = Runner(A, torch, wa, G.make_inputs(wa), "hist", dev)
            m = r.measure(5, 2)
            m["element_sparsity"] = r.element_sparsity()
            m["strength"] = a
            sweep.append(m)
            r.close()
        line["sparsity_sweep"] = sweep

        # ---- long-context workload: the three tau modes (5 timed steps each)
        wl = G.workload("planted_32k")
        xl = G.make_inputs(wl)
        modes = {}
        for mode in ("hist", "halley", "bisect"):
            r = Runner(A, torch, wl, xl, mode, dev)
            m = r.measure(5, 2)
            modes[mode] = {k_: m[k_] for k_ in ("ms_per_step", "tflops", "tau_iters_mean", "tau_iters_max",
                                                "block_sparsity_32x64")}
            modes[mode]["tau_stage_ms"] = m["stage_ms"]["tau"]
            r.close()
        line["tau_modes"] = {"workload": describe(wl), **modes}
        del xl

        # ---- sequence-length scaling, one head (3 timed steps each)
        scal = []
        for n in (32768, 65536, 131072):
            wn = G.workload("planted_32k", H=1, N=n)
            r = Runner(A, torch, wn, G.make_inputs(wn), "hist", dev)
            m = r.measure(3, 1)
            scal.append({"N": n, "ms_per_step": m["ms_per_step"], "tflops": m["tflops"],
                         "block_sparsity_32x64": m["block_sparsity_32x64"],
                         "tau_iters_mean": m["tau_iters_mean"],
                         "workspace_bytes": int(r.bufs.ws.numel()),
                         "stage_ms": m["stage_ms"]})
            r.close()
        line["seq_scaling"] = {"workload": "planted span 512, B=1 H=1 d=128 bf16 causal alpha=1.5",
                               "points": scal}
        line["transform"] = bench_transform(A, torch, G, dev)

    if args.cpu_heads > 0:
        cb = cpu_baseline(w, x, args.cpu_heads)
        cb["cpu_model"] = cpu_model()
        line["cpu_baseline"] = cb
    print(json.dumps(line))


if __name__ == "__main__":
    main()
