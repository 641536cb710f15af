"""Python binding of libpagedkv: paged KV-cache decode attention on MI355X.

Argument marshalling only.  Every step of the path runs in the HIP library
``lib/libpagedkv.so`` built from ``csrc/`` (see ``include/pagedkv.h`` for the
contract of each call).  torch provides device memory and the current stream;
nothing here computes on tensor contents.  If the library has not been built
the import fails loudly: there is no fallback.
"""

from ._lib import (  # noqa: F401
    BLOCK_SIZE, F32, BF16, FP8_E4M3, INT4, INT8, LIB_PATH, PagedKVError, lib,
)
from .api import (  # noqa: F401
    BlockManager, BlockTable, KVPool, block_table_upload, kv_bytes_per_token, kv_copy_blocks, kv_pool_bytes,
    kv_pool_create, paged_attention_append, paged_attention_decode, paged_attention_prefill, paged_attention_prefill_varlen,
    paged_attention_verify, paged_attention_verify_noalloc,
    paged_attention_workspace_bytes, reshape_and_cache, slot_mapping_compute, speculative_accept,
)
