"""Thin ctypes binding over the C ABI declared in include/entmax_attn.h.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libentmax_attn.so.  torch tensors provide device memory and the
current HIP stream.  There is no CPU fallback: if the library is missing,
the first call into it raises FileNotFoundError.
"""
from __future__ import annotations

import ctypes
import os

import torch

from .build import LIB

EA_OK = 0
EA_F32, EA_BF16 = 0, 1
EA_TAU_HIST_HALLEY, EA_TAU_HALLEY_BISECT, EA_TAU_BISECT = 0, 1, 2
EA_FLAG_FORCE_DENSE = 1
STAGES = ("fwd_prep", "rowmax", "tau", "pv", "bwd_prep", "dq", "dkdv")
EA_NUM_STAGES = len(STAGES)
TAU_MODES = {"hist": EA_TAU_HIST_HALLEY, "halley": EA_TAU_HALLEY_BISECT, "bisect": EA_TAU_BISECT}

EXPORTED = (
    "entmax_attn_workspace_bytes",
    "entmax_attn_mask_dims",
    "entmax_attn_fwd",
    "entmax_attn_fwd_static",
    "entmax_attn_bwd",
    "entmax_rows",
    "entmax_attn_strerror",
)


class EaDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32), ("d", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("tau_mode", ctypes.c_int32), ("max_iters", ctypes.c_int32),
        ("tol", ctypes.c_float), ("flags", ctypes.c_int32),
        ("events", ctypes.POINTER(ctypes.c_void_p)),
        ("key_lens", ctypes.POINTER(ctypes.c_int32)),
    ]


class EaRowsDesc(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int64), ("n", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32), ("tau_mode", ctypes.c_int32), ("max_iters", ctypes.c_int32),
        ("tol", ctypes.c_float),
    ]


class EntmaxAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {strerror(status)} (status {status})")
        self.status = status


_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load the built HIP library (raises FileNotFoundError if it was not built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB
    if not os.path.exists(p):
        raise FileNotFoundError(f"{p} not found: run `python -m adaptive_sparse_flash_amd.build`")
    lib = ctypes.CDLL(p)
    vp, sz, i32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_float
    dp = ctypes.POINTER(EaDesc)
    lib.entmax_attn_workspace_bytes.argtypes = [dp]
    lib.entmax_attn_workspace_bytes.restype = sz
    ip = ctypes.POINTER(ctypes.c_int)
    lib.entmax_attn_mask_dims.argtypes = [dp, ip, ip, ip, ip]
    lib.entmax_attn_mask_dims.restype = i32
    lib.entmax_attn_fwd.argtypes = [vp, vp, vp, f32, i32, vp, vp, vp, vp, dp, vp, sz, vp]
    lib.entmax_attn_fwd.restype = i32
    lib.entmax_attn_fwd_static.argtypes = [vp, vp, vp, f32, i32, vp, vp, vp, vp, dp, vp]
    lib.entmax_attn_fwd_static.restype = i32
    lib.entmax_attn_bwd.argtypes = [vp, vp, vp, f32, i32, vp, vp, vp, vp, vp, vp, dp, vp, sz, vp]
    lib.entmax_attn_bwd.restype = i32
    lib.entmax_rows.argtypes = [vp, f32, vp, vp, vp, ctypes.POINTER(EaRowsDesc), vp]
    lib.entmax_rows.restype = i32
    lib.entmax_attn_strerror.argtypes = [i32]
    lib.entmax_attn_strerror.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def strerror(status: int) -> str:
    return load_library().entmax_attn_strerror(int(status)).decode()


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return EA_F32
    if dt == torch.bfloat16:
        return EA_BF16
    raise TypeError(f"unsupported dtype {dt}")


def make_desc(B, H, N, d, in_dtype=torch.bfloat16, out_dtype=torch.float32, tau_mode="hist",
              max_iters=0, tol=0.0, force_dense=False, key_lens=None) -> EaDesc:
    """Descriptor; key_lens (B ints, or None) selects variable-length batches.
    The host array it points to is kept alive by the descriptor."""
    mode = TAU_MODES[tau_mode] if isinstance(tau_mode, str) else int(tau_mode)
    desc = EaDesc(B, H, N, d, _dtype_code(in_dtype) if isinstance(in_dtype, torch.dtype) else in_dtype,
                  _dtype_code(out_dtype) if isinstance(out_dtype, torch.dtype) else out_dtype,
                  mode, max_iters, tol, EA_FLAG_FORCE_DENSE if force_dense else 0, None, None)
    if key_lens is not None:
        if len(key_lens) != B:
            raise ValueError(f"key_lens has {len(key_lens)} entries, expected B = {B}")
        desc._key_lens = (ctypes.c_int32 * B)(*[int(x) for x in key_lens])
        desc.key_lens = ctypes.cast(desc._key_lens, ctypes.POINTER(ctypes.c_int32))
    return desc


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def entmax_attn_workspace_bytes(desc: EaDesc) -> int:
    return int(load_library().entmax_attn_workspace_bytes(ctypes.byref(desc)))


def entmax_attn_mask_dims(desc: EaDesc):
    vals = [ctypes.c_int() for _ in range(4)]
    st = load_library().entmax_attn_mask_dims(ctypes.byref(desc), *[ctypes.byref(v) for v in vals])
    if st != EA_OK:
        raise EntmaxAttnError(st, "entmax_attn_mask_dims")
    return tuple(v.value for v in vals)


_TORCH_DTYPE = {EA_F32: torch.float32, EA_BF16: torch.bfloat16}


def _check_tensors(desc: EaDesc, where: str, **spec) -> None:
    """Every tensor must hold exactly the elements the descriptor implies, in
    the descriptor's element type, contiguous, on a GPU: the library receives
    bare pointers and cannot check what they point to.  None is left to the
    library's own NULL check."""
    given = {name: v for name, v in spec.items() if v[0] is not None}
    for name, (t, numel, dtype) in given.items():
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{where}: {name} must be a torch.Tensor")
        if t.dtype != dtype:
            raise ValueError(f"{where}: {name} has dtype {t.dtype}, expected {dtype}")
        if t.numel() != numel:
            raise ValueError(f"{where}: {name} has {t.numel()} elements, expected {numel}")
        if not t.is_contiguous():
            raise ValueError(f"{where}: {name} must be contiguous")
    for name, (t, numel, _) in given.items():
        if numel and not t.is_cuda:
            raise ValueError(f"{where}: {name} must be a GPU tensor")


def _sizes(desc: EaDesc):
    n_qt, n_kt, _, _ = entmax_attn_mask_dims(desc)
    rows = desc.B * desc.H * desc.N
    return rows * desc.d, rows, desc.B * desc.H * n_qt * n_kt


def entmax_attn_fwd(q, k, v, alpha, causal, out, tau, block_mask, tau_iters, desc, ws,
                    stream=None) -> None:
    full, rows, mask = _sizes(desc)
    ti, to = _TORCH_DTYPE.get(desc.in_dtype), _TORCH_DTYPE.get(desc.out_dtype)
    _check_tensors(desc, "entmax_attn_fwd", q=(q, full, ti), k=(k, full, ti), v=(v, full, ti),
                   out=(out, full, to), tau=(tau, rows, torch.float32),
                   block_mask=(block_mask, mask, torch.uint8), tau_iters=(tau_iters, rows, torch.uint8))
    st = load_library().entmax_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), float(alpha), int(bool(causal)), _ptr(out), _ptr(tau),
        _ptr(block_mask), _ptr(tau_iters), ctypes.byref(desc), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    if st != EA_OK:
        raise EntmaxAttnError(st, "entmax_attn_fwd")


def entmax_attn_fwd_static(q, k, v, alpha, causal, out, tau, block_mask, tau_iters, desc, stream=None) -> None:
    """The forward on the library's fixed device scratch array (no workspace)."""
    full, rows, mask = _sizes(desc)
    ti, to = _TORCH_DTYPE.get(desc.in_dtype), _TORCH_DTYPE.get(desc.out_dtype)
    _check_tensors(desc, "entmax_attn_fwd_static", q=(q, full, ti), k=(k, full, ti), v=(v, full, ti),
                   out=(out, full, to), tau=(tau, rows, torch.float32),
                   block_mask=(block_mask, mask, torch.uint8), tau_iters=(tau_iters, rows, torch.uint8))
    st = load_library().entmax_attn_fwd_static(
        _ptr(q), _ptr(k), _ptr(v), float(alpha), int(bool(causal)), _ptr(out), _ptr(tau),
        _ptr(block_mask), _ptr(tau_iters), ctypes.byref(desc), _stream(stream))
    if st != EA_OK:
        raise EntmaxAttnError(st, "entmax_attn_fwd_static")


def entmax_attn_bwd(q, k, v, alpha, causal, dout, tau, block_mask, dq, dk, dv, desc, ws,
                    stream=None) -> None:
    full, rows, mask = _sizes(desc)
    ti, to = _TORCH_DTYPE.get(desc.in_dtype), _TORCH_DTYPE.get(desc.out_dtype)
    _check_tensors(desc, "entmax_attn_bwd", q=(q, full, ti), k=(k, full, ti), v=(v, full, ti),
                   dout=(dout, full, ti), tau=(tau, rows, torch.float32),
                   block_mask=(block_mask, mask, torch.uint8), dq=(dq, full, to), dk=(dk, full, to),
                   dv=(dv, full, to))
    st = load_library().entmax_attn_bwd(
        _ptr(q), _ptr(k), _ptr(v), float(alpha), int(bool(causal)), _ptr(dout), _ptr(tau),
        _ptr(block_mask), _ptr(dq), _ptr(dk), _ptr(dv), ctypes.byref(desc), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    if st != EA_OK:
        raise EntmaxAttnError(st, "entmax_attn_bwd")


def make_rows_desc(rows, n, in_dtype=torch.float32, out_dtype=torch.float32, tau_mode="hist", max_iters=0,
                   tol=0.0) -> EaRowsDesc:
    mode = TAU_MODES[tau_mode] if isinstance(tau_mode, str) else int(tau_mode)
    code = lambda dt: _dtype_code(dt) if isinstance(dt, torch.dtype) else int(dt)
    return EaRowsDesc(int(rows), int(n), code(in_dtype), code(out_dtype), mode, int(max_iters), float(tol))


def entmax_rows(s, alpha, p, tau, tau_iters, desc, stream=None) -> None:
    """Row-wise alpha-entmax of score rows s [rows, n] into p [rows, n], tau [rows]."""
    ti, to = _TORCH_DTYPE.get(desc.in_dtype), _TORCH_DTYPE.get(desc.out_dtype)
    full = desc.rows * desc.n
    _check_tensors(desc, "entmax_rows", s=(s, full, ti), p=(p, full, to), tau=(tau, desc.rows, torch.float32),
                   tau_iters=(tau_iters, desc.rows, torch.uint8))
    st = load_library().entmax_rows(_ptr(s), float(alpha), _ptr(p), _ptr(tau), _ptr(tau_iters),
                                    ctypes.byref(desc), _stream(stream))
    if st != EA_OK:
        raise EntmaxAttnError(st, "entmax_rows")


def entmax_transform(s, alpha=1.5, tau_mode="hist", out_dtype=None, max_iters=0, tol=0.0):
    """alpha-entmax over the last axis of s (any leading shape, -inf = masked):
    returns (p, tau, iterations) computed by the library's row kernel."""
    n = s.shape[-1]
    rows = s.numel() // max(n, 1)
    out_dtype = s.dtype if out_dtype is None else out_dtype
    desc = make_rows_desc(rows, n, s.dtype, out_dtype, tau_mode, max_iters, tol)
    s = s.contiguous()
    p = torch.empty(s.shape, dtype=out_dtype, device=s.device)
    tau = torch.empty(s.shape[:-1], dtype=torch.float32, device=s.device)
    iters = torch.empty(s.shape[:-1], dtype=torch.uint8, device=s.device)
    entmax_rows(s, alpha, p, tau, iters, desc)
    return p, tau, iters


# ------------------------------------------------------ convenience layer ---

class Buffers:
    """Device buffers for one problem shape (allocated once, reused by calls)."""

    def __init__(self, B, H, N, d, in_dtype=torch.bfloat16, out_dtype=torch.float32,
                 tau_mode="hist", max_iters=0, tol=0.0, force_dense=False, device="cuda", key_lens=None):
        self.desc = make_desc(B, H, N, d, in_dtype, out_dtype, tau_mode, max_iters, tol, force_dense, key_lens)
        n_qt, n_kt, self.bm, self.bn = entmax_attn_mask_dims(self.desc)
        dev = torch.device(device)
        self.out = torch.empty(B, H, N, d, dtype=out_dtype, device=dev)
        self.tau = torch.empty(B, H, N, dtype=torch.float32, device=dev)
        self.mask = torch.empty(B, H, n_qt, n_kt, dtype=torch.uint8, device=dev)
        self.iters = torch.empty(B, H, N, dtype=torch.uint8, device=dev)
        ws = entmax_attn_workspace_bytes(self.desc)
        self.ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
        self.dq = torch.empty(B, H, N, d, dtype=out_dtype, device=dev)
        self.dk = torch.empty_like(self.dq)
        self.dv = torch.empty_like(self.dq)

    def forward(self, q, k, v, alpha, causal, stream=None):
        entmax_attn_fwd(q, k, v, alpha, causal, self.out, self.tau, self.mask, self.iters,
                        self.desc, self.ws, stream)
        return self.out

    def backward(self, q, k, v, dout, alpha, causal, stream=None):
        entmax_attn_bwd(q, k, v, alpha, causal, dout, self.tau, self.mask, self.dq,
                        self.dk, self.dv, self.desc, self.ws, stream)
        return self.dq, self.dk, self.dv


class EntmaxAttention(torch.autograd.Function):
    """Autograd wrapper: y = entmax_alpha(Q K^T / sqrt(d)) V, gradients for Q, K, V."""

    @staticmethod
    def forward(ctx, q, k, v, alpha: float, causal: bool, tau_mode: str = "hist"):
        B, H, N, d = q.shape
        bufs = Buffers(B, H, N, d, q.dtype, q.dtype, tau_mode, device=q.device)
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        out = bufs.forward(q, k, v, alpha, causal).clone()
        ctx.save_for_backward(q, k, v)
        ctx.bufs, ctx.alpha, ctx.causal = bufs, alpha, causal
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v = ctx.saved_tensors
        dq, dk, dv = ctx.bufs.backward(q, k, v, dout.contiguous().to(q.dtype), ctx.alpha, ctx.causal)
        return dq.clone(), dk.clone(), dv.clone(), None, None, None


def entmax_attention(q, k, v, alpha: float = 1.5, causal: bool = False, tau_mode: str = "hist"):
    return EntmaxAttention.apply(q, k, v, alpha, causal, tau_mode)
