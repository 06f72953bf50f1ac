"""Exact fused attention forward for MI355X (gfx950).

The compute lives in a HIP shared library with a C ABI (``include/attn.h``);
``exact_attention_89_amd.api`` marshals torch tensors into it.  The library is
loaded on first use and a missing library is an error: there is no CPU path.
"""
from .api import (  # noqa: F401
    AttnError,
    attn_fwd,
    attn_fwd_f32,
    attn_materialized,
    attn_materialized_workspace_bytes,
    library_path,
    load_library,
)
