"""MI355X-native paged KV cache with single-token and multi-query decode attention.

The compute path is libpkv.so (hand-written HIP for gfx950 behind the C ABI
in include/pkv.h); this package is its Python binding. Importing it loads the
in-tree library and fails loudly if it has not been built.
"""

from ._lib import (  # noqa: F401
    BlockManager,
    CacheDesc,
    OutOfBlocks,
    PkvError,
    STATIC_SCRATCH_BYTES,
    cache_desc,
    cascade_decode_attention,
    cascade_schedule,
    cascade_suffix_partition,
    copy_blocks,
    debug_check,
    decode_schedule,
    decode_workspace_bytes,
    default_partition_size,
    gather_kv,
    kv_append,
    lib,
    make_workspace,
    multi_query_partition_size,
    paged_decode_attention,
    paged_decode_attention_static,
    paged_decode_partials,
    paged_multi_query_attention,
    partial_views,
    set_debug,
    slot_mapping,
    splitk_reduce,
    status_string,
    swap_bytes,
    swap_in,
    swap_out,
    version,
)

lib()
