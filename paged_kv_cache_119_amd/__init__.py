"""MI355X-native paged decode attention and paged KV-cache append.

The computation runs in ``libpagedkv.so`` (hand-written HIP for gfx950, C ABI
declared in ``include/pagedkv.h``); this package is a thin ctypes binding over
it plus byte accounting for the roofline.  Build the library with
``python -m paged_kv_cache_119_amd.build``.
"""

from ._binding import (EXPORTS, LIB_PATH, POOL_REUSE, PagedKVError, PoolDesc, alloc_workspace,  # noqa: F401
                       LaunchInfo, copy_blocks, decode_launch_info, decode_merge, decode_partition_size,
                       decode_merge_fp8, decode_partitions, decode_partitions_append, decode_partitions_fp8,
                       decode_workspace_bytes, fp8_decode_workspace_bytes, fp8_multi_workspace_bytes, fp8_pool_bytes,
                       load_library,
                       make_pool_desc, multi_workspace_bytes, paged_attention_decode, paged_attention_decode_append,
                       paged_attention_decode_noalloc, paged_attention_decode_shared,
                       shared_prefix_workspace_bytes,
                       paged_attention_decode_append_fp8, paged_attention_decode_fp8, paged_attention_multi,
                       paged_attention_multi_fp8,
                       pool_bytes, pool_desc_of, pool_index, reshape_and_cache, reshape_and_cache_fp8, slot_mapping,
                       status_string, version, workspace_views)
