"""Paged decode attention for MI355X (gfx950): HIP kernels behind a C ABI.

    pa_write_kv(k, v, slot_mapping, k_pool, v_pool)
    pa_decode(q, k_pool, v_pool, block_tables, context_lens, scale, out=None, *,
              max_context_len, workspace=None)
    pa_decode_partitioned(..., scale, partition_tokens, ...): fixed partitions
        merged by the log-sum-exp reduce kernel
    pa_append_decode(q, new_k, new_v, k_pool, v_pool, block_tables, context_lens, scale, ...)
    pa_decode_sliding(q, k_pool, v_pool, block_tables, context_lens, scale, window, ...)
    pa_prefill(q, k_pool, v_pool, block_tables, context_lens, query_start, scale, ...)
    pa_write_kv_fp8 / pa_decode_fp8 / pa_append_decode_fp8: the same over FP8 (E4M3)
    pools with per-pool scales
    pa_copy_blocks(pools, block_mapping): whole-block copies for copy-on-write
        (pools: a list of tensors or a PoolSet prepared once)
    pa_check_inputs(k_pool, slot_mapping, block_tables, context_lens): report
        device-side contract violations of those arrays
    BlockManager(num_blocks, block_size): the native host block manager (free
        queue, reference counts, chained prefix hashes, copy-on-write)

The functions marshal torch tensors into libpa.so (built in-tree by
``paged_kv_cache_75_amd.build``).  They raise RuntimeError when the library is
missing; nothing falls back to another implementation.
"""
from .binding import (BlockManager, OutOfBlocks, PoolSet, pa_check_inputs, pa_copy_blocks, pa_sha256, PA_BF16, PA_ERR_HIP, PA_ERR_INVALID_ARGUMENT, PA_ERR_UNSUPPORTED,
                      PA_ERR_WORKSPACE_TOO_SMALL, PA_F16, PA_F32, PA_OK, PaError, lib,
                      fp8_pool_desc, pa_append_decode, pa_append_decode_fp8, pa_decode, pa_decode_fp8,
                      pa_decode_noalloc, pa_decode_partitioned,
                      pa_decode_partitioned_workspace_bytes,
                      pa_decode_sliding, pa_decode_workspace_bytes, pa_pool_desc, pa_prefill,
                      pa_profile_start, pa_profile_stop, pa_status_string, pa_stream_read,
                      pa_write_kv,
                      pa_write_kv_fp8, pool_desc)

__all__ = ["BlockManager", "OutOfBlocks", "PoolSet", "pa_check_inputs", "pa_copy_blocks", "pa_sha256", "PA_BF16", "PA_ERR_HIP", "PA_ERR_INVALID_ARGUMENT", "PA_ERR_UNSUPPORTED",
           "PA_ERR_WORKSPACE_TOO_SMALL", "PA_F16", "PA_F32", "PA_OK", "PaError", "lib",
           "fp8_pool_desc", "pa_append_decode", "pa_append_decode_fp8", "pa_decode",
           "pa_decode_fp8", "pa_decode_noalloc", "pa_decode_partitioned", "pa_decode_partitioned_workspace_bytes",
           "pa_decode_sliding", "pa_decode_workspace_bytes", "pa_pool_desc", "pa_prefill",
           "pa_profile_start", "pa_profile_stop", "pa_status_string", "pa_stream_read",
           "pa_write_kv",
           "pa_write_kv_fp8", "pool_desc"]
