// C entry points of libpa: validate on the host, plan, launch on the
// caller's stream.  Nothing here allocates or synchronizes.
#include <algorithm>
#include <climits>
#include <cmath>

#include <hip/hip_runtime_api.h>

#include "paged_attention.h"
#include "pa_kernels.h"
#include "pa_plan.h"

extern "C" {

pa_status pa_write_kv(const void* k, const void* v, const int32_t* slot_mapping,
                      int32_t num_tokens, void* k_pool, void* v_pool,
                      const pa_pool_desc* pool, void* stream) {
  const pa_status s = pa::check_write(k, v, slot_mapping, num_tokens, k_pool, v_pool, pool);
  if (s != PA_OK || num_tokens == 0) return s;
  pa::WriteArgs a;
  a.k = k;
  a.v = v;
  a.slot_mapping = slot_mapping;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.num_tokens = num_tokens;
  a.num_slots = pool->num_blocks * pool->block_size;
  a.num_kv_heads = pool->num_kv_heads;
  a.row_bytes = pool->head_dim * pa::dtype_bytes(pool->dtype);
  int32_t lb = 0;
  while ((1 << lb) < pool->block_size) ++lb;
  a.log2_block = lb;
  return pa::launch_write_kv(a, static_cast<hipStream_t>(stream)) == hipSuccess ? PA_OK
                                                                                : PA_ERR_HIP;
}

pa_status pa_copy_blocks(void* const* pools, int32_t num_pools, int32_t num_blocks,
                         int64_t block_bytes, const int32_t* block_mapping, int32_t num_pairs,
                         void* stream) {
  if (!pools || num_pools < 1 || num_blocks < 0 || num_pairs < 0) return PA_ERR_INVALID_ARGUMENT;
  if (block_bytes <= 0 || block_bytes % 16 != 0 || block_bytes > (int64_t(1) << 30))
    return PA_ERR_INVALID_ARGUMENT;
  if (num_pairs > 0 && !block_mapping) return PA_ERR_INVALID_ARGUMENT;
  for (int32_t i = 0; i < num_pools; ++i)
    if (!pools[i] || reinterpret_cast<uintptr_t>(pools[i]) % 16 != 0)
      return PA_ERR_INVALID_ARGUMENT;
  const int64_t chunks = pa::copy_chunks_per_block(block_bytes);
  if (int64_t(num_pairs) * chunks > INT32_MAX) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0 || num_blocks == 0) return PA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int32_t done = 0; done < num_pools; done += pa::kCopyMaxPools) {
    pa::CopyArgs a{};
    const int32_t n = std::min<int32_t>(pa::kCopyMaxPools, num_pools - done);
    for (int32_t i = 0; i < n; ++i) a.pools[i] = static_cast<char*>(pools[done + i]);
    a.mapping = block_mapping;
    a.block_bytes = block_bytes;
    a.num_blocks = num_blocks;
    a.chunks = static_cast<int32_t>(chunks);
    if (pa::launch_copy_blocks(a, num_pairs, n, s) != hipSuccess) return PA_ERR_HIP;
  }
  return PA_OK;
}

size_t pa_check_scratch_bytes(const pa_pool_desc* pool) {
  if (pa::check_pool(pool) != PA_OK) return 0;
  const int64_t slots = int64_t(pool->num_blocks) * pool->block_size;
  return size_t((slots + 31) / 32) * 2 * sizeof(uint32_t);
}

pa_status pa_check_inputs(const int32_t* slot_mapping, int32_t num_tokens,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                          const pa_pool_desc* pool, int32_t* report, void* scratch,
                          void* stream) {
  if (pa::check_pool(pool) != PA_OK || !report) return PA_ERR_INVALID_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(report) % 8 != 0) return PA_ERR_INVALID_ARGUMENT;
  if (scratch && reinterpret_cast<uintptr_t>(scratch) % 4 != 0) return PA_ERR_INVALID_ARGUMENT;
  if (num_tokens < 0 || (num_tokens > 0 && !slot_mapping)) return PA_ERR_INVALID_ARGUMENT;
  if (num_seqs < 0) return PA_ERR_INVALID_ARGUMENT;
  if (num_seqs > 0) {
    if (!block_tables || !context_lens || max_blocks_per_seq <= 0 || max_context_len < 0)
      return PA_ERR_INVALID_ARGUMENT;
    if (int64_t(max_context_len) > int64_t(max_blocks_per_seq) * pool->block_size)
      return PA_ERR_INVALID_ARGUMENT;
    if (int64_t(num_seqs) * max_blocks_per_seq > INT32_MAX) return PA_ERR_UNSUPPORTED;
  }
  pa::CheckArgs a{};
  a.slots = num_tokens > 0 ? slot_mapping : nullptr;
  a.tables = num_seqs > 0 ? block_tables : nullptr;
  a.lens = num_seqs > 0 ? context_lens : nullptr;
  a.report = report;
  a.num_slots = int64_t(pool->num_blocks) * pool->block_size;
  a.bitmap_words = (a.num_slots + 31) / 32;
  if (scratch) {
    a.seen = static_cast<uint32_t*>(scratch);
    a.dup = a.seen + a.bitmap_words;
  }
  a.num_tokens = num_tokens;
  a.num_seqs = num_seqs;
  a.max_blocks = max_blocks_per_seq;
  a.max_len = max_context_len;
  a.num_blocks = pool->num_blocks;
  int32_t lb = 0;
  while ((1 << lb) < pool->block_size) ++lb;
  a.log2_block = lb;
  return pa::launch_check(a, static_cast<hipStream_t>(stream)) == hipSuccess ? PA_OK
                                                                             : PA_ERR_HIP;
}

size_t pa_decode_partitioned_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                             const pa_pool_desc* pool, int32_t max_context_len,
                                             int32_t partition_tokens) {
  pa::DecodePlan plan;
  if (pa::plan_decode(num_seqs, num_q_heads, pool, max_context_len, -1, partition_tokens,
                      &plan) != PA_OK)
    return 0;
  return plan.ws_bytes;
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                 const pa_pool_desc* pool, int32_t max_context_len) {
  return pa_decode_partitioned_workspace_bytes(num_seqs, num_q_heads, pool, max_context_len, 0);
}

}  // extern "C"

namespace {

// pa_decode and pa_append_decode: new_k == nullptr for a plain decode.
pa_status decode(const void* q, const void* new_k, const void* new_v, const void* k_pool,
                 const void* v_pool, const pa_pool_desc* pool, const int32_t* block_tables,
                 int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                 int32_t max_context_len, int32_t num_q_heads, float scale, void* out,
                 void* workspace, size_t workspace_bytes, int32_t partition_tokens,
                 int32_t window, void* stream, bool kv_fp8 = false, float k_scale = 1.0f,
                 float v_scale = 1.0f) {
  pa::DecodePlan plan;
  pa_status s = pa::plan_decode(num_seqs, num_q_heads, pool, max_context_len,
                                max_blocks_per_seq, partition_tokens, &plan);
  if (s != PA_OK) return s;
  if (max_blocks_per_seq <= 0 && num_seqs > 0) return PA_ERR_INVALID_ARGUMENT;
  s = pa::check_decode_pointers(q, k_pool, v_pool, block_tables, context_lens, out, num_seqs);
  if (s != PA_OK) return s;
  if (!std::isfinite(scale)) return PA_ERR_INVALID_ARGUMENT;
  if (num_seqs == 0) return PA_OK;
  if (plan.ws_bytes > 0) {
    if (!workspace) return PA_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < plan.ws_bytes) return PA_ERR_WORKSPACE_TOO_SMALL;
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return PA_ERR_INVALID_ARGUMENT;
  }

  if (kv_fp8) {
    // FP8 pools: the balanced split with 16-bit queries only
    if (!plan.balanced || pool->dtype == PA_F32) return PA_ERR_UNSUPPORTED;
    if (!(std::isfinite(k_scale) && k_scale > 0.0f && std::isfinite(v_scale) && v_scale > 0.0f))
      return PA_ERR_INVALID_ARGUMENT;
  }

  pa::DecodeArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.out = out;
  char* ws = static_cast<char*>(workspace);
  a.ws_o = plan.ws_bytes ? reinterpret_cast<float*>(ws + plan.ws_o_offset) : nullptr;
  a.ws_ml = plan.ws_bytes ? reinterpret_cast<float*>(ws + plan.ws_ml_offset) : nullptr;
  a.ws_hdr = plan.balanced ? reinterpret_cast<int32_t*>(ws + plan.ws_hdr_offset) : nullptr;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.num_blocks = pool->num_blocks;
  a.log2_block = plan.log2_block;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.partition_tokens = plan.partition_tokens;
  a.num_partitions = plan.balanced ? 0 : plan.num_partitions;
  a.min_split_tiles = pa::kMinSplitTiles;
  // FP8 pools: scores are taken on the codes, so the key scale joins the scale
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * (kv_fp8 ? k_scale : 1.0f) *
                                    1.4426950408889634);
  a.kv_fp8 = kv_fp8 ? 1 : 0;
  a.v_scale = kv_fp8 ? v_scale : 1.0f;
  a.k_scale = kv_fp8 ? k_scale : 1.0f;
  a.new_k = new_k;
  a.new_v = new_v;
  a.window = window;
  // keys and values stream past the caches when the batch may read more than
  // the 256 MB Infinity Cache holds (its KV bytes are at most num_seqs x
  // max_context_len rows of every kv head); smaller batches keep the default
  // policy, so blocks that sequences share are read once from memory
  const double kv_bound = double(num_seqs) * double(max_context_len) * 2.0 *
                          double(pool->num_kv_heads) * double(pool->head_dim) *
                          (kv_fp8 ? 1.0 : double(pa::dtype_bytes(pool->dtype)));
  a.kv_stream = kv_bound > double(pa::kInfinityCacheBytes) ? 1 : 0;
  const hipError_t e = pa::launch_decode(a, pool->dtype, pool->head_dim, plan.group,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

extern "C" {

pa_status pa_decode(const void* q, const void* k_pool, const void* v_pool,
                    const pa_pool_desc* pool, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* context_lens,
                    int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads,
                    float scale, void* out, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return decode(q, nullptr, nullptr, k_pool, v_pool, pool, block_tables, max_blocks_per_seq,
                context_lens, num_seqs, max_context_len, num_q_heads, scale, out, workspace,
                workspace_bytes, 0, 0, stream);
}

pa_status pa_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                            const pa_pool_desc* pool, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads,
                            float scale, void* out, void* stream) {
  pa::DecodePlan plan;
  const pa_status s = pa::plan_decode(num_seqs, num_q_heads, pool, max_context_len,
                                      max_blocks_per_seq, 0, &plan);
  if (s != PA_OK) return s;
  if (plan.ws_bytes > pa::kStaticScratchBytes) return PA_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (plan.ws_bytes > 0 && num_seqs > 0) {
    if (pa::static_scratch(&ws) != hipSuccess) return PA_ERR_HIP;
  }
  return decode(q, nullptr, nullptr, k_pool, v_pool, pool, block_tables, max_blocks_per_seq,
                context_lens, num_seqs, max_context_len, num_q_heads, scale, out, ws,
                pa::kStaticScratchBytes, 0, 0, stream);
}

pa_status pa_decode_partitioned(const void* q, const void* k_pool, const void* v_pool,
                                const pa_pool_desc* pool, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* context_lens,
                                int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads,
                                float scale, void* out, void* workspace, size_t workspace_bytes,
                                int32_t partition_tokens, void* stream) {
  if (partition_tokens <= 0) return PA_ERR_INVALID_ARGUMENT;
  return decode(q, nullptr, nullptr, k_pool, v_pool, pool, block_tables, max_blocks_per_seq,
                context_lens, num_seqs, max_context_len, num_q_heads, scale, out, workspace,
                workspace_bytes, partition_tokens, 0, stream);
}

pa_status pa_decode_sliding(const void* q, const void* k_pool, const void* v_pool,
                            const pa_pool_desc* pool, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads,
                            float scale, int32_t window, void* out, void* workspace,
                            size_t workspace_bytes, int32_t partition_tokens, void* stream) {
  if (window < 1) return PA_ERR_INVALID_ARGUMENT;
  return decode(q, nullptr, nullptr, k_pool, v_pool, pool, block_tables, max_blocks_per_seq,
                context_lens, num_seqs, max_context_len, num_q_heads, scale, out, workspace,
                workspace_bytes, partition_tokens, window, stream);
}

pa_status pa_write_kv_fp8(const void* k, const void* v, const int32_t* slot_mapping,
                          int32_t num_tokens, void* k_pool, void* v_pool,
                          const pa_pool_desc* pool, float k_scale, float v_scale, void* stream) {
  const pa_status s = pa::check_write(k, v, slot_mapping, num_tokens, k_pool, v_pool, pool);
  if (s != PA_OK) return s;
  if (!(std::isfinite(k_scale) && k_scale > 0.0f && std::isfinite(v_scale) && v_scale > 0.0f))
    return PA_ERR_INVALID_ARGUMENT;
  if (num_tokens == 0) return PA_OK;
  pa::WriteArgs a;
  a.k = k;
  a.v = v;
  a.slot_mapping = slot_mapping;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.num_tokens = num_tokens;
  a.num_slots = pool->num_blocks * pool->block_size;
  a.num_kv_heads = pool->num_kv_heads;
  a.row_bytes = pool->head_dim;                 // one byte per code
  int32_t lb = 0;
  while ((1 << lb) < pool->block_size) ++lb;
  a.log2_block = lb;
  return pa::launch_write_kv_fp8(a, pool->dtype, k_scale, v_scale,
                                 static_cast<hipStream_t>(stream)) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

pa_status pa_decode_fp8(const void* q, const void* k_pool, const void* v_pool,
                        const pa_pool_desc* pool, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                        int32_t max_context_len, int32_t num_q_heads, float scale, float k_scale,
                        float v_scale, void* out, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return decode(q, nullptr, nullptr, k_pool, v_pool, pool, block_tables, max_blocks_per_seq,
                context_lens, num_seqs, max_context_len, num_q_heads, scale, out, workspace,
                workspace_bytes, 0, 0, stream, true, k_scale, v_scale);
}

pa_status pa_append_decode_fp8(const void* q, const void* new_k, const void* new_v,
                               void* k_pool, void* v_pool, const pa_pool_desc* pool,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t num_seqs,
                               int32_t max_context_len, int32_t num_q_heads, float scale,
                               float k_scale, float v_scale, void* out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (num_seqs > 0 && (!new_k || !new_v)) return PA_ERR_INVALID_ARGUMENT;
  return decode(q, new_k, new_v, k_pool, v_pool, pool, block_tables, max_blocks_per_seq,
                context_lens, num_seqs, max_context_len, num_q_heads, scale, out, workspace,
                workspace_bytes, 0, 0, stream, true, k_scale, v_scale);
}

pa_status pa_append_decode(const void* q, const void* new_k, const void* new_v,
                           void* k_pool, void* v_pool, const pa_pool_desc* pool,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs,
                           int32_t max_context_len, int32_t num_q_heads, float scale,
                           void* out, void* workspace, size_t workspace_bytes,
                           int32_t partition_tokens, void* stream) {
  if (num_seqs > 0 && (!new_k || !new_v)) return PA_ERR_INVALID_ARGUMENT;
  return decode(q, new_k, new_v, k_pool, v_pool, pool, block_tables, max_blocks_per_seq,
                context_lens, num_seqs, max_context_len, num_q_heads, scale, out, workspace,
                workspace_bytes, partition_tokens, 0, stream);
}

pa_status pa_prefill(const void* q, const void* k_pool, const void* v_pool,
                     const pa_pool_desc* pool, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* context_lens,
                     const int32_t* query_start, int32_t num_seqs, int32_t max_context_len,
                     int32_t max_query_len, int32_t num_q_heads, float scale, void* out,
                     void* stream) {
  int32_t group = 0;
  pa_status s = pa::check_prefill(num_seqs, num_q_heads, pool, max_context_len,
                                  max_blocks_per_seq, max_query_len, &group);
  if (s != PA_OK) return s;
  s = pa::check_decode_pointers(q, k_pool, v_pool, block_tables, context_lens, out, num_seqs);
  if (s != PA_OK) return s;
  if (num_seqs > 0 && !query_start) return PA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(scale)) return PA_ERR_INVALID_ARGUMENT;
  if (num_seqs == 0 || max_query_len == 0) return PA_OK;
  pa::DecodeArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.out = out;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.num_blocks = pool->num_blocks;
  int32_t lb = 0;
  while ((1 << lb) < pool->block_size) ++lb;
  a.log2_block = lb;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  a.query_start = query_start;
  a.max_query_len = max_query_len;
  const hipError_t e = pa::launch_prefill(a, pool->dtype, pool->head_dim, group,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes == 0) return PA_OK;
  if (!buf || !sink || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return PA_ERR_INVALID_ARGUMENT;
  if (bytes > (size_t(1) << 40)) return PA_ERR_UNSUPPORTED;
  return pa::launch_stream_read(buf, static_cast<int64_t>(bytes), sink,
                                static_cast<hipStream_t>(stream)) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

pa_status pa_profile_start(void) {
  pa::profile_start();
  return PA_OK;
}

pa_status pa_profile_stop(int32_t* launches, double* mean_us) {
  if (!launches || !mean_us) return PA_ERR_INVALID_ARGUMENT;
  return pa::profile_stop(launches, mean_us) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

const char* pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARGUMENT: return "PA_ERR_INVALID_ARGUMENT";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_WORKSPACE_TOO_SMALL: return "PA_ERR_WORKSPACE_TOO_SMALL";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    case PA_ERR_OUT_OF_BLOCKS: return "PA_ERR_OUT_OF_BLOCKS";
    case PA_ERR_HOST_MEMORY: return "PA_ERR_HOST_MEMORY";
    default: return "PA_UNKNOWN_STATUS";
  }
}

}  // extern "C"
