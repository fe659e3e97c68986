"""gfx950 paged decode attention: a C-ABI library (libpagedattn.so) and its
thin Python binding.  Besides the decode call the library writes the cache
in its own layout (one appended token per sequence, whole-block copies for
copy-on-write sharing) and scores blocks for block-wise eviction.

``_lib`` mirrors the C ABI (include/pagedattn.h) name for name; ``api``
adds torch-tensor conveniences (descriptor from shapes, workspace and
output allocation through torch, the current HIP stream)."""
from ._lib import (  # noqa: F401
    EXPORTS,
    PA_BF16,
    PA_F16,
    PA_F32,
    PA_KERNEL_AUTO,
    PA_KERNEL_MFMA,
    PA_KERNEL_VALU,
    LIB_PATH,
    BlockManager,
    PaDesc,
    PagedAttnError,
    load,
    pa_blocks_for_len,
    pa_check_desc,
    pa_decode_grid,
    pa_dtype_size,
    pa_k_elem_offset,
    pa_pool_bytes,
    pa_v_elem_offset,
    pa_validate_append_host,
    pa_validate_copy_host,
    pa_validate_host,
    pa_validate_prefill_host,
    pa_workspace_bytes,
    paged_attn_decode,
    paged_attn_decode_noalloc,
    paged_attn_decode_shared,
    pa_decode_shared_grid,
    pa_shared_workspace_bytes,
    pa_validate_shared_host,
    paged_attn_prefill,
    paged_kv_append,
    paged_kv_block_scores,
    paged_kv_copy_blocks,
    status_str,
)
from .api import (  # noqa: F401
    append, block_scores, copy_blocks, decode, decode_shared, ensure_built, make_desc,
    new_shared_workspace, new_workspace, prefill)
