// Host-side argument checks and launch planning (no HIP calls).
#include "pa_plan.h"

#include <climits>

namespace pa {

namespace {

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int32_t ilog2(int64_t x) {
  int32_t n = 0;
  while ((int64_t{1} << n) < x) ++n;
  return n;
}

bool group_supported(int32_t g) { return (g >= 1 && g <= 8) || g == 16; }

// Context partition length when the caller leaves it to the library.  Long
// contexts are cut into 256-token partitions (16 tiles, four per wave of a
// 256-thread workgroup); a sequence that fits one partition needs no merge.
int32_t auto_partition(int32_t max_context_len) {
  const int32_t p = 256;
  if (max_context_len <= p) {
    const int32_t t = (max_context_len + kTileTokens - 1) / kTileTokens * kTileTokens;
    return t > 0 ? t : kTileTokens;
  }
  return p;
}

}  // namespace

int32_t dtype_bytes(int32_t dtype) {
  switch (dtype) {
    case PA_F32: return 4;
    case PA_F16: return 2;
    case PA_BF16: return 2;
    default: return 0;
  }
}

pa_status check_pool(const pa_pool_desc* pool) {
  if (!pool) return PA_ERR_INVALID_ARGUMENT;
  if (pool->num_blocks <= 0 || pool->num_kv_heads <= 0 || pool->head_dim <= 0 ||
      pool->block_size <= 0)
    return PA_ERR_INVALID_ARGUMENT;
  if (dtype_bytes(pool->dtype) == 0) return PA_ERR_INVALID_ARGUMENT;
  if (!is_pow2(pool->block_size) || pool->block_size > 256) return PA_ERR_UNSUPPORTED;
  if (pool->head_dim != 64 && pool->head_dim != 128) return PA_ERR_UNSUPPORTED;
  // slots are int32: num_blocks * block_size must stay below 2^31
  if (int64_t{pool->num_blocks} * pool->block_size >= (int64_t{1} << 31))
    return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

pa_status check_write(const void* k, const void* v, const int32_t* slot_mapping,
                      int32_t num_tokens, const void* k_pool, const void* v_pool,
                      const pa_pool_desc* pool) {
  pa_status s = check_pool(pool);
  if (s != PA_OK) return s;
  if (num_tokens < 0) return PA_ERR_INVALID_ARGUMENT;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_pool || !v_pool) return PA_ERR_INVALID_ARGUMENT;
  return PA_OK;
}

pa_status plan_decode(int32_t num_seqs, int32_t num_q_heads, const pa_pool_desc* pool,
                      int32_t max_context_len, int32_t max_blocks_per_seq,
                      int32_t partition_tokens, DecodePlan* plan) {
  pa_status s = check_pool(pool);
  if (s != PA_OK) return s;
  if (!plan || num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0)
    return PA_ERR_INVALID_ARGUMENT;
  if (num_q_heads % pool->num_kv_heads != 0) return PA_ERR_INVALID_ARGUMENT;
  // sequences and heads index grid dimensions y/z (at most 65535 each)
  if (num_seqs > 65535 || num_q_heads > 65535) return PA_ERR_UNSUPPORTED;
  const int32_t group = num_q_heads / pool->num_kv_heads;
  if (!group_supported(group)) return PA_ERR_UNSUPPORTED;
  if (max_blocks_per_seq >= 0 &&
      int64_t{max_context_len} > int64_t{max_blocks_per_seq} * pool->block_size)
    return PA_ERR_INVALID_ARGUMENT;
  if (partition_tokens < 0 || partition_tokens % kTileTokens != 0)
    return PA_ERR_INVALID_ARGUMENT;
  if (partition_tokens > kMaxPartitionTokens) return PA_ERR_UNSUPPORTED;

  DecodePlan p;
  p.group = group;
  p.log2_block = ilog2(pool->block_size);
  const size_t D = size_t(pool->head_dim);
  auto align = [](size_t x) { return (x + 255) / 256 * 256; };
  // balanced split: 16-bit elements (matrix-core P.V), blocks holding whole
  // 16-token tiles, and a batch whose lengths fit the kernel's LDS copy (the
  // kernel counts the whole batch's work, kv heads x (tiles + 1) per
  // sequence, in 32 bits)
  const int64_t batch_units = int64_t(num_seqs) * pool->num_kv_heads *
                              (int64_t(max_context_len) / kTileTokens + 2);
  if (partition_tokens == 0 && num_seqs <= kMaxSplitSeqs && pool->dtype != PA_F32 &&
      pool->block_size >= kTileTokens && batch_units < (int64_t{1} << 31)) {
    // two piece slots per workgroup share; an 8-int header per piece
    const size_t pieces = size_t(kMaxSplits) * 2;
    p.balanced = true;
    p.ws_hdr_offset = 0;
    p.ws_ml_offset = align(pieces * 8 * sizeof(int32_t));
    p.ws_o_offset = align(p.ws_ml_offset + pieces * size_t(group) * 2 * sizeof(float));
    p.ws_bytes = p.ws_o_offset + pieces * size_t(group) * D * sizeof(float);
  } else {
    const int32_t P = partition_tokens ? partition_tokens : auto_partition(max_context_len);
    p.partition_tokens = P;
    p.num_partitions = max_context_len > 0 ? (max_context_len + P - 1) / P : 1;
    if (p.num_partitions > 1) {
      const size_t rows = size_t(num_seqs) * size_t(num_q_heads) * size_t(p.num_partitions);
      p.ws_o_offset = 0;
      p.ws_ml_offset = align(rows * D * sizeof(float));
      p.ws_bytes = p.ws_ml_offset + rows * 2 * sizeof(float);
    }
  }
  *plan = p;
  return PA_OK;
}

pa_status check_prefill(int32_t num_seqs, int32_t num_q_heads, const pa_pool_desc* pool,
                        int32_t max_context_len, int32_t max_blocks_per_seq,
                        int32_t max_query_len, int32_t* group) {
  DecodePlan p;   // the decode's shape checks (any valid partition)
  const pa_status s = plan_decode(num_seqs, num_q_heads, pool, max_context_len,
                                  max_blocks_per_seq, kTileTokens, &p);
  if (s != PA_OK) return s;
  if (max_blocks_per_seq <= 0 && num_seqs > 0) return PA_ERR_INVALID_ARGUMENT;
  if (max_query_len < 0 || max_query_len > max_context_len) return PA_ERR_INVALID_ARGUMENT;
  if (pool->dtype == PA_F32) return PA_ERR_UNSUPPORTED;   // matrix-core tile math only
  if (prefill_workgroups(num_seqs, pool->num_kv_heads, p.group, max_query_len) > INT32_MAX)
    return PA_ERR_UNSUPPORTED;                             // one-dimensional grid
  *group = p.group;
  return PA_OK;
}

pa_status check_decode_pointers(const void* q, const void* k_pool, const void* v_pool,
                                const int32_t* block_tables, const int32_t* context_lens,
                                const void* out, int32_t num_seqs) {
  if (num_seqs == 0) return PA_OK;
  if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !out)
    return PA_ERR_INVALID_ARGUMENT;
  return PA_OK;
}

}  // namespace pa
