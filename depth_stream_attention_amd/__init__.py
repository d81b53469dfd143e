"""MoDA (Mixture-of-Depths Attention) fused forward for AMD Instinct MI355X (gfx950).

The compute path is libmoda.so (hand-written HIP kernels behind a C ABI,
include/moda.h); this package is its thin Python binding.
"""
from .api import (  # noqa: F401
    MODAError,
    moda_append_depth_slot,
    moda_attn_bwd,
    moda_attn_bwd_workspace,
    moda_attn_decode,
    moda_attn_decode_noalloc,
    moda_attn_decode_ring,
    moda_attn_decode_workspace,
    moda_attn_fwd,
    moda_attn_fwd_f32,
    moda_attn_fwd_ring,
    moda_block_span,
    moda_error_string,
    moda_kv_project,
    moda_pack_depth,
)
