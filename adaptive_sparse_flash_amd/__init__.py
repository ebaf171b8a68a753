"""Fused alpha-entmax attention for AMD Instinct MI355X (gfx950).

The computation lives in the HIP library built from csrc/ (see build.py); this
package only marshals arguments to its C ABI (include/entmax_attn.h).
"""
from .binding import (  # noqa: F401
    Buffers,
    EntmaxAttention,
    EntmaxAttnError,
    EaDesc,
    entmax_attention,
    entmax_attn_bwd,
    entmax_attn_fwd,
    entmax_attn_fwd_static,
    entmax_attn_mask_dims,
    entmax_attn_workspace_bytes,
    entmax_rows,
    entmax_transform,
    load_library,
    make_desc,
    make_rows_desc,
    strerror,
)
