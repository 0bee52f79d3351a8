"""MI355X-native fused causal scaled-dot-product attention, forward and backward.

The work runs in hand-written HIP kernels for gfx950 behind the C ABI in
include/attn_api.h (libcausal_attn.so, built in-tree by
``python -m causal_attention_amd.build``).  This package is the thin Python
binding: the same entry points, taking torch device tensors.
"""
from ._binding import (  # noqa: F401
    ATTN_DECODE_SCRATCH_BYTES,
    ATTN_DTYPE_BF16,
    ATTN_DTYPE_F16,
    ATTN_DTYPE_F32,
    ATTN_MASK_CAUSAL,
    ATTN_MASK_DOC_CAUSAL,
    AttnError,
    AttnParams,
    LIB_PATH,
    attn_bwd,
    attn_bwd_dkdv,
    attn_bwd_ex,
    attn_bwd_dq,
    attn_bwd_dq_delta,
    attn_bwd_preprocess,
    attn_bwd_rope,
    attn_decode,
    attn_decode_noalloc,
    attn_fwd,
    attn_fwd_ex,
    attn_fwd_rope,
    attn_rope,
    attn_rope_table,
    backward,
    build_id,
    bwd_workspace_bytes,
    clock_probe,
    decode,
    decode_workspace_bytes,
    forward,
    header_functions,
    load_library,
    rope_table,
    status_string,
)
