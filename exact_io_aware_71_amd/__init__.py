"""Exact IO-aware attention for AMD Instinct MI355X (gfx950).

The compute lives in libexact_attn.so (hand-written HIP kernels behind the C ABI of
include/attn.h); `binding` marshals torch tensors into those calls.
"""
from .binding import (  # noqa: F401
    AttnError, attn_bwd, attn_bwd_workspace_bytes, attn_decode, attn_decode_auto_splits,
    attn_decode_workspace_bytes, attn_fwd, load,
)
