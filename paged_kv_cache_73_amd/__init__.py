"""paged_kv_cache_73_amd: paged attention over a block-table KV cache on MI355X.

The compute path is libpa.so (include/pa.h): hand-written HIP kernels for gfx950
plus a C++ host block manager.  This package is its thin binding; the entry points
keep their C names.  See :mod:`paged_kv_cache_73_amd._native`.
"""

from ._native import (  # noqa: F401
    EXPORTS, PA_DECODE_SCRATCH_BYTES, BlockManager, KVPool, OutOfBlocks, PaError, RefcountError, lib,
    pa_abi_version, pa_build_cu_seqlens, pa_build_slot_mapping, pa_copy_blocks, pa_decode,
    pa_decode_append, pa_decode_merge, pa_decode_noalloc, pa_decode_partials, pa_decode_workspace_bytes, pa_pool_bytes, pa_prefill_varlen,
    pa_prefill_varlen_contiguous, pa_prefill_varlen_splitk, pa_prefill_workspace_bytes,
    pa_prefix_block_hash,
    pa_probe_stream_read, pa_source_digest, pa_status_str,
    pa_validate_decode, pa_validate_slots, pa_validate_varlen, pa_write_kv,
)
