"""Paged-KV-cache store and attention for MI355X (gfx950).

The compute lives in ``libpkv.so`` (hand-written HIP kernels behind the C ABI
of ``include/pkv.h``, and the C++ block pool of ``include/pkv_pool.h``); this package is its thin Python binding plus the seeded
workload generator used by the tests and the benchmark.

    from paged_kv_cache_pools_amd import pkv_store, pkv_decode_attn, pkv_prefill_attn
"""
from .binding import (PkvError, load, pkv_decode_attn, pkv_decode_partition_tokens,  # noqa: F401
                      pkv_decode_workspace_bytes, pkv_kv_bytes, pkv_last_error,
                      pkv_prefill_attn, pkv_status_string, pkv_store, pkv_store_decode_attn,
                      pkv_store_decode_attn_rope,
                      pkv_store_fp8, pkv_decode_attn_fp8, pkv_store_decode_attn_fp8,
                      pkv_decode_partition_tokens_fp8, BlockPool, pkv_copy_blocks, pkv_mixed_attn,
                      pkv_mixed_workspace_bytes, pkv_decode_attn_prefix,
                      pkv_decode_prefix_workspace_bytes, pkv_prefix_groups)

__all__ = ["pkv_store", "pkv_decode_attn", "pkv_store_decode_attn", "pkv_store_decode_attn_rope",
           "pkv_prefill_attn",
           "pkv_store_fp8", "pkv_decode_attn_fp8", "pkv_store_decode_attn_fp8",
           "pkv_decode_partition_tokens_fp8", "pkv_kv_bytes",
           "pkv_decode_workspace_bytes", "pkv_decode_partition_tokens", "pkv_status_string",
           "pkv_last_error", "PkvError", "load", "BlockPool", "pkv_copy_blocks", "pkv_mixed_attn",
           "pkv_mixed_workspace_bytes", "pkv_decode_attn_prefix",
           "pkv_decode_prefix_workspace_bytes", "pkv_prefix_groups"]
