// Host-side argument checks and launch planning for libpa.  Plain C++ with no
// HIP dependency, so it also builds with g++ (and sanitizers) for host tests.
#pragma once

#include <cstddef>
#include <cstdint>

#include "paged_attention.h"

namespace pa {

// Tokens per compute tile: one 16-column MFMA tile of keys.
constexpr int32_t kTileTokens = 16;
// Largest context partition.
constexpr int32_t kMaxPartitionTokens = 8192;
// Balanced split: at most this many workgroups (shares of the work), at most
// this many sequences per call, and at least this many 16-token tiles per
// share (smaller batches use fewer workgroups).
constexpr int32_t kMaxSplits = 4096;
constexpr int32_t kMaxSplitSeqs = 1024;
constexpr int32_t kMinSplitTiles = 8;
// MI355X's Infinity Cache (the memory-side cache in front of HBM)
constexpr int64_t kInfinityCacheBytes = int64_t(256) << 20;
// Chunked prefill: 16-column query blocks per wave, and the XCDs whose L2s a
// launch spreads over (workgroup i runs on XCD i mod kXcds)
constexpr int32_t kPrefillColumnBlocks = 2;
constexpr int32_t kPrefillWaves = 4;          // waves per prefill workgroup
constexpr int32_t kXcds = 8;
inline int64_t prefill_workgroups(int32_t num_seqs, int32_t num_kv_heads, int32_t group,
                                  int32_t max_query_len) {
  const int64_t queries = int64_t(16 / group) * kPrefillColumnBlocks * kPrefillWaves;
  const int64_t blocks = (max_query_len + queries - 1) / queries;
  const int64_t pairs = (int64_t(num_seqs) * num_kv_heads + kXcds - 1) / kXcds * kXcds;
  return blocks * pairs;
}

int32_t dtype_bytes(int32_t dtype);   // 0 for an unknown dtype

pa_status check_pool(const pa_pool_desc* pool);

pa_status check_write(const void* k, const void* v, const int32_t* slot_mapping,
                      int32_t num_tokens, const void* k_pool, const void* v_pool,
                      const pa_pool_desc* pool);

struct DecodePlan {
  int32_t group = 0;              // query heads per kv head
  bool balanced = false;          // balanced split (else fixed partitions)
  int32_t partition_tokens = 0;   // fixed partitions: tokens per partition
  int32_t num_partitions = 0;     // fixed partitions: of the longest sequence
  int32_t log2_block = 0;
  size_t ws_bytes = 0;            // 0 when nothing needs merging
  size_t ws_hdr_offset = 0;       // byte offsets inside the workspace
  size_t ws_ml_offset = 0;
  size_t ws_o_offset = 0;
};

// Shape checks plus the launch plan.  max_blocks_per_seq < 0 skips the
// table-width check (used by the workspace query).
pa_status plan_decode(int32_t num_seqs, int32_t num_q_heads, const pa_pool_desc* pool,
                      int32_t max_context_len, int32_t max_blocks_per_seq,
                      int32_t partition_tokens, DecodePlan* plan);

// Shape checks for chunked prefill; sets the query heads per kv head.
pa_status check_prefill(int32_t num_seqs, int32_t num_q_heads, const pa_pool_desc* pool,
                        int32_t max_context_len, int32_t max_blocks_per_seq,
                        int32_t max_query_len, int32_t* group);

pa_status check_decode_pointers(const void* q, const void* k_pool, const void* v_pool,
                                const int32_t* block_tables, const int32_t* context_lens,
                                const void* out, int32_t num_seqs);

}  // namespace pa
