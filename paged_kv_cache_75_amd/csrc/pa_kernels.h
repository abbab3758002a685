// Internal launch interface between the C entry points and the HIP kernels.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime_api.h>

#include "pa_plan.h"

namespace pa {

struct WriteArgs {
  const void* k;
  const void* v;
  const int32_t* slot_mapping;
  void* k_pool;
  void* v_pool;
  int32_t num_tokens;
  int32_t num_slots;        // num_blocks * block_size; larger slots are skipped
  int32_t num_kv_heads;
  int32_t row_bytes;        // head_dim * element bytes
  int32_t log2_block;
};

struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  // workspace.  Fixed partitions: ws_o [num_seqs][num_q_heads][num_partitions]
  // [head_dim], ws_ml [..][num_partitions][2] (max, sum).  Balanced split:
  // per piece (2 per workgroup) ws_hdr [4] = {valid, seq, kv head, flags},
  // ws_ml [group][2], ws_o [group][head_dim].
  float* ws_o;
  float* ws_ml;
  int32_t* ws_hdr;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t log2_block;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;  // lengths above it are clamped to it
  int32_t partition_tokens;
  int32_t num_partitions;   // 0 selects the balanced split
  int32_t min_split_tiles;  // balanced split: tiles per workgroup share, at least
  float scale_log2;         // scale * log2(e): scores live in the exp2 domain
  // Appending decode (nullptr otherwise): token T_i - 1 of sequence i is row i
  // of new_k / new_v ([num_seqs][num_kv_heads][head_dim]).  The decode reads it
  // from there, and it is copied to its slot (found through the block table):
  // by the wave that handles the pair's last tile (balanced split), or by a
  // copy kernel before the decode (fixed partitions).
  const void* new_k;
  const void* new_v;
  int32_t window;           // sliding window in tokens; 0: attend to every token
  // Chunked prefill: rows query_start[i] .. query_start[i+1]-1 of q (and of
  // out) are sequence i's queries, the last M_i of its T_i tokens.
  const int32_t* query_start;
  int32_t max_query_len;    // host bound on M_i (sizes the grid)
  // FP8 pools (balanced split only): codes times v_scale are the values; the
  // key scale is folded into scale_log2
  int32_t kv_fp8;
  float v_scale;
  float k_scale;            // FP8 pools: the key scale itself (appended rows are quantized)
  // Balanced split: load keys and values non-temporally (batches larger than
  // the Infinity Cache); 0 keeps the default cache policy
  int32_t kv_stream;
};

hipError_t launch_write_kv(const WriteArgs& a, hipStream_t stream);

// Block copy: pools travel by value in the kernel arguments, up to
// kCopyMaxPools per launch.  A workgroup moves one chunk of kCopyChunkBytes of
// one block of one pool.
constexpr int32_t kCopyMaxPools = 64;
constexpr int64_t kCopyChunkBytes = 16384;
inline int64_t copy_chunks_per_block(int64_t block_bytes) {
  return (block_bytes + kCopyChunkBytes - 1) / kCopyChunkBytes;
}
struct CopyArgs {
  char* pools[kCopyMaxPools];
  const int32_t* mapping;      // [num_pairs][2] (source, destination)
  int64_t block_bytes;         // multiple of 16
  int32_t num_blocks;
  int32_t chunks;              // copy_chunks_per_block(block_bytes)
};
hipError_t launch_copy_blocks(const CopyArgs& a, int32_t num_pairs, int32_t num_pools,
                              hipStream_t stream);

// Slot write into FP8 (E4M3) pools; a.row_bytes = head_dim (one byte per
// code); dtype = element type of k and v.
hipError_t launch_write_kv_fp8(const WriteArgs& a, int32_t dtype, float k_scale, float v_scale,
                               hipStream_t stream);

// Contract check of the device arrays (pa_check_inputs).  bitmap_words: 32-bit
// words of each of the two slot bitmaps (seen, duplicated) in the scratch.
struct CheckArgs {
  const int32_t* slots;
  const int32_t* tables;
  const int32_t* lens;
  int32_t* report;             // [0] count, [2..3] the first violation's key, then kind/index/value
  uint32_t* seen;              // nullptr: no duplicate test
  uint32_t* dup;
  int64_t num_slots;           // num_blocks * block_size
  int64_t bitmap_words;
  int32_t num_tokens;
  int32_t num_seqs;
  int32_t max_blocks;
  int32_t max_len;
  int32_t num_blocks;
  int32_t log2_block;
};
hipError_t launch_check(const CheckArgs& a, hipStream_t stream);

// Chunked prefill (16-bit pools): causal attention of each sequence's last
// M_i tokens; group as planned.
hipError_t launch_prefill(const DecodeArgs& a, int32_t dtype, int32_t head_dim, int32_t group,
                          hipStream_t stream);

// Streaming read of `bytes` (a multiple of 16) at `buf` (16-byte aligned);
// writes sink[0] only for data crafted to match a constant (measurement only).
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream);

// Kernel timing (measurement only): start attaching events to the attention
// kernel of each decode call; stop, wait for those events and report.
void profile_start();
hipError_t profile_stop(int32_t* launches, double* mean_us);

// Size of the library-held decode workspace (pa_decode_noalloc) and the
// current device's copy of it (its address is looked up once per device).
constexpr size_t kStaticScratchBytes = size_t(36) << 20;
hipError_t static_scratch(void** ptr);

// dtype is a pa_dtype value; head_dim 64/128; group as planned.
hipError_t launch_decode(const DecodeArgs& a, int32_t dtype, int32_t head_dim,
                         int32_t group, hipStream_t stream);

}  // namespace pa
