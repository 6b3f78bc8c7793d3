"""libgdn: the Gated DeltaNet token mixer on AMD MI355X (gfx950).

Python entry points with the C ABI's names (include/gdn.h):
  gdn_chunk_fwd, gdn_chunk_fwd_noalloc, gdn_chunk_bwd, gdn_decode_step, gdn_decode_multi,
  gdn_chunk_fwd_workspace_bytes, gdn_chunk_bwd_workspace_bytes, gdn_chunk_fwd_workspace_layout.
The HIP library is loaded on first use and is required: there is no CPU
fallback. Build it with `python -m linear_attention_recurrence_delta_amd.build`.
"""
from .binding import (  # noqa: F401
    GdnDims,
    GdnError,
    LIBRARY_PATH,
    gdn_chunk_bwd,
    gdn_chunk_bwd_workspace_bytes,
    gdn_chunk_fwd,
    gdn_chunk_fwd_noalloc,
    gdn_chunk_fwd_workspace_bytes,
    gdn_chunk_fwd_workspace_layout,
    gdn_decode_multi,
    gdn_decode_step,
    load_library,
    make_dims,
)
