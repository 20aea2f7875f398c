"""LION bidirectional masked linear attention on AMD Instinct MI355X (gfx950).

The computation lives in ``liblion_attn.so`` (hand-written HIP kernels behind the C ABI declared
in ``include/lion_attn.h``); this package only marshals torch tensors into that ABI.  There is
no CPU fallback: if the library is missing, every call raises.
"""
from .binding import (  # noqa: F401
    CAUSAL,
    FP32_ARITH,
    FORM_BIRNN,
    FORM_CHUNK,
    FORM_FULL,
    FORM_CHUNK2,
    FORM_CHUNK_BWD,
    FORM_FULL_BWD,
    MASK_D,
    MASK_LIT,
    MASK_S,
    LionArgumentError,
    LionError,
    lion_attn_abi_version,
    lion_attn_birnn,
    lion_attn_chunk,
    lion_attn_full,
    lion_attn_full2,
    lion_attn_full_bwd,
    lion_attn_chunk_bwd,
    lion_attn_chunk2,
    lion_attn_chunk_noalloc,
    lion_attn_workspace_bytes,
    lion_selectivity,
    lion_status_str,
    library,
)
