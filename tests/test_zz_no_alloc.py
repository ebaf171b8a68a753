"""The forward entry point that allocates nothing (entmax_attn_fwd_static),
called through the C ABI: its results equal entmax_attn_fwd's bit for bit on
two calls in a row on one GPU, the second with a smaller input; a desc whose
forward workspace exceeds the fixed array is refused before any GPU work."""
import ctypes

import numpy as np
import pytest
import torch

import adaptive_sparse_flash_amd as A
from adaptive_sparse_flash_amd import binding as Bd
from gen import inputs as G


def test_static_forward_refuses_oversized_desc():
    # 64 heads at N = 65536 need 128 MiB of block codes: more than the 32 MiB array
    d = A.make_desc(1, 64, 65536, 128)
    lib = A.load_library()
    p = ctypes.c_void_p(256)     # never dereferenced: the size check comes first
    st = lib.entmax_attn_fwd_static(p, p, p, 1.5, 1, p, p, p, None, ctypes.byref(d), None)
    assert st == -6


@pytest.mark.gpu
def test_static_forward_equals_workspace_forward():
    for (name, H, N) in (("planted_16k", 4, 3000), ("iid_causal_4k", 2, 700)):
        w = G.workload(name, B=1, H=H, N=N)
        print(f"\n[no-alloc] {name} H={H} N={N} d={w.d}", flush=True)
        x = G.make_inputs(w)
        q, k, v = (torch.from_numpy(x[n]).to(torch.bfloat16).cuda() for n in ("q", "k", "v"))
        ref = A.Buffers(w.B, w.H, w.N, w.d, torch.bfloat16, torch.float32, "hist")
        ref.forward(q, k, v, w.alpha, w.causal)
        desc = A.make_desc(w.B, w.H, w.N, w.d, torch.bfloat16, torch.float32, "hist")
        out = torch.full_like(ref.out, float("nan"))
        tau = torch.full_like(ref.tau, float("nan"))
        mask = torch.full_like(ref.mask, 7)
        iters = torch.zeros_like(ref.iters)
        Bd.entmax_attn_fwd_static(q, k, v, w.alpha, w.causal, out, tau, mask, iters, desc)
        torch.cuda.synchronize()
        for a, b in ((out, ref.out), (tau, ref.tau), (mask, ref.mask), (iters, ref.iters)):
            np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy())
