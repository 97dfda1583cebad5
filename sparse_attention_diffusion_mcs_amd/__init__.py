"""MC-Sparse (Meta-Cached Sparse Attention) on AMD Instinct MI355X (gfx950).

Python face of libmcs.so: `select` runs the selection step (exact dense
attention, query grouping, per-group top-k of kept KV tokens, residual) and
returns the cached metadata; `sparse_attn` runs a reuse step over it;
`dense_attn` is the library's exact dense attention.  The library must be
built (`python -m sparse_attention_diffusion_mcs_amd.build`); there is no
fallback implementation.
"""

from ._lib import LIB_PATH, McsError, lib  # noqa: F401
from .api import (MetaCache, dense_attn, desc_for, meta_init, meta_layout, select, sparse_attn,  # noqa: F401
                  topk_rows, workspace_bytes)
