"""Exact IO-aware tiled attention (forward and backward) for AMD MI355X (gfx950).

The compute lives in ``libattn.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/attn.h``).  This package is the thin Python binding:
``attn_fwd`` / ``attn_bwd`` / ``attn_bwd_noalloc`` / ``attn_fwd_splitkv`` marshal torch device
tensors into that ABI (block-sparse and rectangular calls through their
``block_mask`` / ``causal_offset`` arguments; ``attn_fwd_standard`` /
``attn_bwd_standard`` run standard attention, which materialises the score
and probability matrices, as the baseline), and ``forward`` /
``backward`` are conveniences that allocate the outputs.  The
library is loaded on first use; if it is missing every call raises.
"""

from ._lib import (  # noqa: F401
    AttnError,
    attn_fwd,
    attn_bwd,
    attn_bwd_noalloc,
    attn_bwd_workspace_bytes,
    attn_fwd_splitkv,
    attn_fwd_splitkv_workspace_bytes,
    attn_fwd_standard,
    attn_bwd_standard,
    attn_standard_workspace_bytes,
    standard_probs,
    forward,
    backward,
    library_path,
    load_library,
)
