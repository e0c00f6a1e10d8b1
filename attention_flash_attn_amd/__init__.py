"""MI355X-native fused scaled-dot-product attention (prefill, paged / gathered decode, MLA decode tail).

The compute path is the C-ABI library libattn.so (hand-written HIP kernels for
gfx950); this package is its thin Python binding. Importing the package does
not load the library: the binding loads it on first use and raises if it is
missing.
"""

from .binding import (  # noqa: F401
    AttnError,
    attn_prefill_fwd,
    attn_prefill_fwd_ex,
    attn_decode_fwd,
    attn_decode_fwd_noalloc,
    attn_decode_workspace_bytes,
    attn_dequant_fp16,
    attn_mla_tail,
    attn_mla_tail_workspace_bytes,
    attn_status_string,
    attn_abi_version,
    library_path,
    load_library,
)
