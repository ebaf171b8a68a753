"""One forward + backward step captured as a HIP graph and replayed.

The library launches only kernels on the caller's stream (no allocation, no
memset, no host synchronisation), so a step can be captured with torch's
graph API and replayed.  Every replay runs on zeroed outputs, with eager
steps and synchronisations between the replays, and must reproduce the eager
step bit for bit (the kernels are deterministic: integer histogram atomics,
fixed reduction orders)."""
import pytest
import torch

import adaptive_sparse_flash_amd as A
from gen import inputs as G

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("strength", [0.4, 3.0])
def test_graph_replays_match_eager(strength):
    w = G.workload("planted_16k", H=2, N=4096, strength=strength)
    print(f"\n[graph] planted a={strength} B={w.B} H={w.H} N={w.N} d={w.d}", flush=True)
    x = G.make_inputs(w)
    q, k, v, do = (torch.from_numpy(x[n]).to(torch.bfloat16).cuda() for n in ("q", "k", "v", "dout"))
    bufs = A.Buffers(w.B, w.H, w.N, w.d, torch.bfloat16, torch.bfloat16, "hist")
    outs = (bufs.out, bufs.tau, bufs.mask, bufs.iters, bufs.dq, bufs.dk, bufs.dv)

    def step():
        bufs.forward(q, k, v, w.alpha, w.causal)
        bufs.backward(q, k, v, do, w.alpha, w.causal)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    names = ("out", "tau", "mask", "iters", "dq", "dk", "dv")
    for rep in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for nm, r, t in zip(names, ref, outs):
            assert torch.equal(r, t), f"replay {rep}: {nm} differs from the eager step"
        step()
        torch.cuda.synchronize()
        for nm, r, t in zip(names, ref, outs):
            assert torch.equal(r, t), f"eager step after replay {rep}: {nm} differs"
