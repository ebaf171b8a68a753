"""C ABI checks that need no GPU: the library loads, exports every function
the header declares, plans a workspace the size of the block mask, and rejects invalid
arguments before touching the device."""
import ctypes
import os
import re

import pytest

import adaptive_sparse_flash_amd as A
from adaptive_sparse_flash_amd import binding as Bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "entmax_attn.h")


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:size_t|int|const char\*)\s+(entmax_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    lib = A.load_library()
    names = header_functions()
    assert set(names) == set(Bd.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define\s+(EA_\w+)\s+(-?\d+)", text))
    assert int(consts["EA_F32"]) == Bd.EA_F32 and int(consts["EA_BF16"]) == Bd.EA_BF16
    assert int(consts["EA_TAU_HIST_HALLEY"]) == Bd.EA_TAU_HIST_HALLEY
    assert int(consts["EA_TAU_BISECT"]) == Bd.EA_TAU_BISECT
    assert int(consts["EA_NUM_STAGES"]) == len(Bd.STAGES)
    assert int(consts["EA_MASK_BM"]) == 32 and int(consts["EA_MASK_BN"]) == 64


def test_desc_struct_layout():
    # int32 x 9 + float + two pointers, natural alignment
    assert ctypes.sizeof(Bd.EaDesc) == 56
    # int64 + int32 x 5 + float
    assert ctypes.sizeof(Bd.EaRowsDesc) == 32


@pytest.mark.parametrize("field,value,status", [
    ("rows", -1, -2), ("n", 0, -2), ("n", (1 << 20) + 1, -2), ("in_dtype", 3, -3), ("out_dtype", 9, -3),
    ("tau_mode", 4, -8), ("max_iters", 300, -8), ("tol", 2.0, -8)])
def test_rows_invalid_desc_rejected(field, value, status):
    d = A.make_rows_desc(4, 100)
    setattr(d, field, value)
    lib = A.load_library()
    assert lib.entmax_rows(None, 1.5, None, None, None, ctypes.byref(d), None) == status


def test_rows_argument_checks():
    lib = A.load_library()
    d = A.make_rows_desc(4, 100)
    assert lib.entmax_rows(None, 1.5, None, None, None, None, None) == -1        # no descriptor
    assert lib.entmax_rows(None, 1.0, None, None, None, ctypes.byref(d), None) == -4   # alpha
    assert lib.entmax_rows(None, 1.5, None, None, None, ctypes.byref(d), None) == -1   # null tensors
    assert lib.entmax_rows(ctypes.c_void_p(16 * 3 + 4), 1.5, ctypes.c_void_p(64), ctypes.c_void_p(128), None,
                           ctypes.byref(d), None) == -5                                   # misaligned s
    empty = A.make_rows_desc(0, 100)
    assert lib.entmax_rows(None, 1.5, None, None, None, ctypes.byref(empty), None) == 0  # nothing to do


def _align(x):
    return (x + 255) // 256 * 256


def test_workspace_is_rows_plus_mask_sized_codes():
    """Workspace = one float per row + one byte per (32-query block, 64-key
    tile), rows padded to 64 tiles (the size of the block mask), + 256 bytes
    of work-queue counters, + the transposed copies for fp32 inputs.  It grows
    like the block mask (about N^2 / 2048 bytes per head), never like a score
    matrix."""
    for n in (1000, 4096, 16384, 131072):
        bh = 16
        nk, nq = -(-n // 64), -(-n // 32)
        d = A.make_desc(1, bh, n, 128)
        ws = A.entmax_attn_workspace_bytes(d)
        codes = _align(bh * nq * (-(-nk // 64) * 64))
        assert ws == _align(bh * n * 4) + codes + 256
        assert ws <= bh * n * 4 + bh * nq * (nk + 63) + 1024
        f = A.make_desc(1, bh, n, 128, in_dtype=0)
        tr = _align(bh * 128 * nk * 64 * 4)
        mt = _align(bh * nk * ((nq + 3) // 4 * 4))      # transposed block mask
        assert A.entmax_attn_workspace_bytes(f) == max(tr + ws, 3 * tr + _align(bh * n * 4) + mt)
    # the largest accepted length: one head at N = 2^20 needs the 512 MiB of
    # its block mask plus 4 MiB of row maxima (and the queue counters)
    big = A.entmax_attn_workspace_bytes(A.make_desc(1, 1, 1 << 20, 128))
    assert big == (1 << 22) + (1 << 15) * (1 << 14) + 256
    d = A.make_desc(2, 3, 1000, 64, out_dtype=1)
    assert A.entmax_attn_mask_dims(d) == (32, 16, 32, 64)


@pytest.mark.parametrize("field,value,status", [
    ("d", 96, -2), ("N", -1, -2), ("B", 0, -2), ("in_dtype", 7, -3), ("out_dtype", -1, -3),
    ("tau_mode", 5, -8), ("max_iters", -1, -8), ("tol", -1.0, -8), ("flags", 8, -8)])
def test_invalid_desc_rejected(field, value, status):
    d = A.make_desc(1, 1, 128, 64)
    setattr(d, field, value)
    assert A.entmax_attn_workspace_bytes(d) == 0
    lib = A.load_library()
    st = lib.entmax_attn_fwd(None, None, None, 1.5, 0, None, None, None, None,
                             ctypes.byref(d), None, 0, None)
    assert st == status


def _fwd(lib, d, alpha=1.5, causal=0, ptr=16, ws_bytes=1 << 30, null=None):
    p = [ctypes.c_void_p(ptr)] * 8
    if null is not None:
        p[null] = None
    return lib.entmax_attn_fwd(p[0], p[1], p[2], alpha, causal, p[3], p[4], p[5], None,
                               ctypes.byref(d), p[6], ws_bytes, None)


def test_argument_errors_before_launch():
    lib = A.load_library()
    d = A.make_desc(1, 2, 256, 64)
    for alpha in (1.0, 0.5, 2.5, float("nan"), float("inf")):
        assert _fwd(lib, d, alpha=alpha) == -4
    assert _fwd(lib, d, causal=2) == -8
    for i in range(7):
        assert _fwd(lib, d, null=i) == -1
    assert _fwd(lib, d, ptr=8) == -5
    assert _fwd(lib, d, ws_bytes=16) == -6
    st = lib.entmax_attn_bwd(None, None, None, 1.5, 0, None, None, None, None, None, None,
                             ctypes.byref(d), None, 0, None)
    assert st == -1
    assert A.strerror(-6) == "workspace too small"
    assert A.strerror(12345) == "unknown status"


def test_empty_sequence_is_a_no_op():
    lib = A.load_library()
    d = A.make_desc(1, 1, 0, 64)
    st = lib.entmax_attn_fwd(None, None, None, 1.5, 1, None, None, None, None,
                             ctypes.byref(d), None, 0, None)
    assert st == 0


C_CALLER = r"""
#include <stdio.h>
#include <string.h>
#include "entmax_attn.h"

int main(void) {
  ea_desc d;
  size_t ws;
  int st, bad, nq = 0, nk = 0, bm = 0, bn = 0;
  memset(&d, 0, sizeof d);
  d.B = 1; d.H = 2; d.N = 1000; d.d = 128;
  d.in_dtype = EA_BF16; d.out_dtype = EA_F32; d.tau_mode = EA_TAU_HIST_HALLEY;
  ws = entmax_attn_workspace_bytes(&d);
  st = entmax_attn_mask_dims(&d, &nq, &nk, &bm, &bn);
  /* missing tensors: rejected before any device work */
  bad = entmax_attn_fwd(NULL, NULL, NULL, 1.5f, 0, NULL, NULL, NULL, NULL, &d, NULL, 0, NULL);
  printf("%lu %d %d %d %d %d %d %s\n", (unsigned long)ws, st, nq, nk, bm, bn, bad,
         entmax_attn_strerror(bad));
  return 0;
}
"""


def test_header_is_plain_c_and_links(tmp_path):
    """The header compiles as strict C99 and a C program links against the
    library and drives its host-side entry points (no GPU involved)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    lib = A.load_library()
    libdir = os.path.dirname(Bd.LIB)
    src = tmp_path / "caller.c"
    src.write_text(C_CALLER)
    exe = tmp_path / "caller"
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    str(src), "-L", libdir, "-lentmax_attn", "-Wl,-rpath," + libdir,
                    "-Wl,-rpath-link,/opt/rocm/lib", "-o", str(exe)], check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split(maxsplit=7)
    desc = Bd.make_desc(1, 2, 1000, 128)
    assert int(out[0]) == Bd.entmax_attn_workspace_bytes(desc)
    assert [int(v) for v in out[1:6]] == [0, 32, 16, 32, 64]
    assert int(out[6]) == -1 and out[7].strip() == lib.entmax_attn_strerror(-1).decode()


def test_binding_rejects_mismatched_tensors():
    """The Python entry points check every tensor against the descriptor
    (element type, element count, contiguity, device) before the library is
    called, since the library only sees bare pointers."""
    import torch
    d = A.make_desc(1, 2, 100, 64)                       # bf16 in, fp32 out
    n_qt, n_kt, _, _ = A.entmax_attn_mask_dims(d)
    full, rows = 2 * 100 * 64, 2 * 100
    q = torch.zeros(1, 2, 100, 64, dtype=torch.bfloat16)
    out = torch.zeros(full, dtype=torch.float32)
    tau = torch.zeros(rows, dtype=torch.float32)
    mask = torch.zeros(2 * n_qt * n_kt, dtype=torch.uint8)
    fwd = lambda **kw: Bd.entmax_attn_fwd(kw.get("q", q), q, q, 1.5, 1, kw.get("out", out), tau,
                                          kw.get("mask", mask), None, d, None)
    with pytest.raises(ValueError, match="dtype"):
        fwd(q=q.float())
    with pytest.raises(ValueError, match="elements"):
        fwd(out=torch.zeros(full - 1, dtype=torch.float32))
    with pytest.raises(ValueError, match="elements"):
        fwd(mask=torch.zeros(2 * n_qt * n_kt + 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="contiguous"):
        fwd(q=torch.zeros(1, 2, 64, 100, dtype=torch.bfloat16).transpose(2, 3))
    with pytest.raises(ValueError, match="GPU"):
        fwd()
    with pytest.raises(ValueError, match="dtype"):
        Bd.entmax_attn_bwd(q, q, q, 1.5, 1, q, tau, mask, out, out, out.to(torch.bfloat16), d, None)


def test_key_lens_checked_before_launch():
    """A key length outside [0, N] is refused with EA_ERR_SHAPE before any
    GPU work; valid lengths pass the descriptor checks."""
    lib = A.load_library()
    ok = A.make_desc(3, 2, 100, 64, key_lens=[100, 7, 0])
    assert A.entmax_attn_workspace_bytes(ok) > 0
    for bad in ([101, 5, 5], [5, -1, 5]):
        d = A.make_desc(3, 2, 100, 64, key_lens=bad)
        assert A.entmax_attn_workspace_bytes(d) == 0
        p = ctypes.c_void_p(256)
        assert lib.entmax_attn_fwd(p, p, p, 1.5, 1, p, p, p, None, ctypes.byref(d), p, 1 << 20, None) == -2
    with pytest.raises(ValueError):
        A.make_desc(3, 2, 100, 64, key_lens=[1, 2])
