"""Flash-attention forward for AMD Instinct MI355X (gfx950).

The kernels live in ``libattn.so`` (C ABI in ``include/attn.h``); ``attn``
is its thin Python binding. Importing this package does not load the
library; the first call does, and fails loudly if it is missing.
"""
from .attn import (  # noqa: F401
    AttnError,
    DecodeWorkspace,
    attn_decode_combine,
    attn_decode_combine_ex,
    attn_decode_fwd,
    attn_decode_fwd_fp8kv,
    attn_decode_fwd_noalloc,
    attn_decode_validate_pages,
    attn_prefill_fwd,
    attn_prefill_fwd_ex,
    attn_prefill_fwd_fp8kv,
    attn_prefill_varlen_fwd,
    auto_split_len,
    decode,
    decode_heads_per_workgroup,
    lib,
    max_splits_for,
    prefill,
    prefill_kernel,
    prefill_varlen,
)
