"""libpagedattn: paged KV-cache attention for AMD Instinct MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
include/pagedattn.h (libpagedattn.so, built by `python
paged_kv_cache_109_amd/build.py`); this package is the thin Python binding
(argument marshalling only). Importing it fails if the library is not built.
"""
from ._binding import (  # noqa: F401
    BlockManager,
    EXPORTED,
    LIB_PATH,
    OutOfBlocks,
    STREAM_SINK_WORDS_PER_GROUP,
    SHARED_ALL,
    SHARED_COMBINE,
    SHARED_OWN,
    SHARED_PREFIX,
    PagedAttnError,
    abi_version,
    MAX_GROUP_MEMBERS,
    alloc_decode_shared_workspace,
    alloc_decode_workspace,
    copy_blocks,
    decode_default_workers,
    decode_workspace_bytes,
    paged_attention_decode,
    paged_attention_decode_append,
    paged_attention_decode_append_partitions,
    paged_attention_decode_append_reduce,
    paged_attention_decode_noalloc,
    NOALLOC_SCRATCH_BYTES,
    paged_attention_decode_partitions,
    paged_attention_decode_reduce,
    paged_attention_decode_shared,
    paged_attention_prefill_chunk,
    paged_attention_prefill_chunk_append,
    reshape_and_cache,
    shared_prefix_groups,
    slot_mapping,
    stream_read,
    swap_blocks,
)
