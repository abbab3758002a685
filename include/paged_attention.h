/*
 * paged_attention.h -- C ABI of the MI355X (gfx950) paged decode-attention
 * library (libpa.so).
 *
 * The library implements the two kernels on the hot path of PagedAttention:
 *
 *   pa_write_kv  copies each new token's key and value rows into its slot of a
 *                per-layer block pool (the slot write of "vLLM Framework and
 *                Inference Engine Design", section "How is vLLM's KV cache
 *                paged?": slot = block_table[floor(t/B)] * B + (t mod B)).
 *   pa_decode    computes, for every sequence i and query head h,
 *                  out[i][h] = softmax(scale * q[i][h] . K_i^T) . V_i
 *                over the T_i cached tokens of sequence i, reading token t
 *                from physical block block_tables[i][floor(t/B)] at offset
 *                t mod B (same page, section "What is the essence of vLLM's
 *                PagedAttention?").
 *
 * Conventions shared by every entry point:
 *
 *   - Every buffer argument is a DEVICE pointer owned by the caller.  The
 *     library never allocates, frees or keeps a reference to caller memory.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *     null stream) and the call returns without synchronizing.  Results are
 *     valid once the stream reaches that point.  A decode that must see a
 *     token written by pa_write_kv has to be enqueued after that write on the
 *     same stream (or be ordered after it by the caller).
 *   - Arguments are validated on the host from the scalar arguments only; on
 *     any error the call returns a status and enqueues nothing.  Device
 *     arrays (slot_mapping, block_tables, context_lens) are never read on the
 *     host; their contract is stated per entry point.  Breaking it gives
 *     unspecified output values but no access outside the buffers: the
 *     kernels skip slots outside the pool, clamp context lengths into
 *     [0, max_context_len] and clamp block-table entries into the pool.
 *   - Element types: the pool, the new k/v rows, q and out share one element
 *     type (pa_dtype).  Accumulation is in float32.
 *   - Pool layout (both pools): dense [num_blocks][num_kv_heads][block_size]
 *     [head_dim], row-major.  One (block, kv head) pair is one contiguous run
 *     of block_size * head_dim elements.
 *   - Integer arrays are int32.
 */
#ifndef PAGED_ATTENTION_H
#define PAGED_ATTENTION_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative or inconsistent size */
  PA_ERR_UNSUPPORTED = 2,        /* a valid shape the library does not handle */
  PA_ERR_WORKSPACE_TOO_SMALL = 3,
  PA_ERR_HIP = 4,                /* a HIP runtime call or a launch failed      */
  PA_ERR_OUT_OF_BLOCKS = 5,      /* block manager: not enough free blocks      */
  PA_ERR_HOST_MEMORY = 6         /* block manager: a host allocation failed    */
} pa_status;

typedef enum pa_dtype {
  PA_F32 = 0,
  PA_F16 = 1,
  PA_BF16 = 2
} pa_dtype;

/* One layer's block pool.  block_size must be a power of two in [1, 256];
 * head_dim is 64 or 128; num_blocks * block_size must stay below 2^31. */
typedef struct pa_pool_desc {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;                 /* a pa_dtype value */
} pa_pool_desc;

/*
 * pa_write_kv -- place new tokens' K and V rows into their pool slots.
 *
 *   k, v          [num_tokens][num_kv_heads][head_dim], pool element type.
 *   slot_mapping  int32 [num_tokens]; slot s >= 0 sends token n to physical
 *                 block s / block_size at offset s % block_size, for every kv
 *                 head.  s < 0 skips the token (padding).  Live slots must be
 *                 distinct and below num_blocks * block_size.
 *   k_pool, v_pool  pools described by *pool; only the addressed rows change.
 *
 * The copy is of raw element bits, so the pools match a host-side copy bit
 * for bit.  num_tokens == 0 is a no-op returning PA_OK.
 */
pa_status pa_write_kv(const void* k, const void* v, const int32_t* slot_mapping,
                      int32_t num_tokens, void* k_pool, void* v_pool,
                      const pa_pool_desc* pool, void* stream);

/*
 * pa_decode_workspace_bytes -- size in bytes of the scratch buffer pa_decode
 * needs for these sizes (see pa_decode).  For fp16/bf16 pools with
 * block_size >= 16 and num_seqs <= 1024 (the balanced split) the size depends
 * only on the query heads per kv head and head_dim; otherwise it is that of
 * fixed 256-token partitions.  0 means no workspace is needed, and workspace
 * may then be NULL.  Returns 0 also for invalid sizes (pa_decode reports
 * those).  Host scalars only; nothing is enqueued.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                 const pa_pool_desc* pool, int32_t max_context_len);

/*
 * pa_decode -- one decode step of paged attention for num_seqs sequences.
 *
 *   q             [num_seqs][num_q_heads][head_dim].
 *   k_pool, v_pool, pool   the layer's pools (see above).
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]; entry j of row i is
 *                 the physical block of tokens j*B .. j*B+B-1 of sequence i.
 *                 Only entries j < ceil(T_i / B) are read; each must lie in
 *                 [0, num_blocks).  Entries past them may hold anything.
 *   context_lens  int32 [num_seqs]; T_i counts the token being decoded, whose
 *                 K/V must already be in the pool.  0 <= T_i <= max_context_len.
 *                 T_i == 0 yields an all-zero output row.
 *   max_context_len  host-side upper bound on every T_i; sizes the launch.
 *                 Must be <= max_blocks_per_seq * block_size.
 *   num_q_heads   a multiple of num_kv_heads.  Query head h reads kv head
 *                 h / (num_q_heads / num_kv_heads) (contiguous groups).
 *   scale         multiplies q . k before the softmax (1/sqrt(head_dim) for
 *                 standard attention).
 *   out           [num_seqs][num_q_heads][head_dim], rounded to nearest even.
 *   workspace     scratch of at least pa_decode_workspace_bytes(...) bytes
 *                 for the same sizes, 16-byte aligned; its contents on entry
 *                 do not matter.  Calls sharing one workspace must be ordered
 *                 on one stream.
 *
 * How the context is split across workgroups is the library's choice: for
 * fp16/bf16 pools with a block size of at least 16, the flattened work of all
 * (sequence, kv head) pairs, in 16-token tiles, is cut into equal contiguous
 * shares, one per resident wave but none under 8 tiles (at most 1024
 * sequences); otherwise fixed
 * 256-token partitions (pa_decode_partitioned with 256).  Pieces of a pair
 * computed by different workgroups are merged by log-sum-exp in a second
 * kernel; the split depends only on the sizes and context_lens, so a call
 * repeated on the same inputs gives the same bits.
 *
 * Supported: head_dim 64 or 128; query heads per kv head 1..8 or 16.
 */
pa_status pa_decode(const void* q, const void* k_pool, const void* v_pool,
                    const pa_pool_desc* pool, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* context_lens,
                    int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads,
                    float scale, void* out, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops or harnesses that
 * forbid allocation).  Arguments, results and errors are pa_decode's, without
 * the workspace: the library keeps one fixed workspace of 36 MiB per GPU, in
 * device memory reserved when the library's code is loaded on that GPU and
 * held until the process ends, and the call allocates and frees nothing.
 * Sizes whose pa_decode_workspace_bytes exceeds 36 MiB (e.g. 16 query heads
 * per kv head at head_dim 128) return PA_ERR_UNSUPPORTED.  Every call on a GPU
 * uses that GPU's one workspace: calls that may overlap on one GPU (other
 * streams, other threads) race and must be ordered by the caller.  Nothing in
 * the workspace needs clearing between calls.  The kernel timing of
 * pa_profile_start creates events, so it must be off around these calls.
 */
pa_status pa_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                            const pa_pool_desc* pool, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads,
                            float scale, void* out, void* stream);

/*
 * pa_decode_partitioned -- pa_decode with fixed context partitions: every
 * sequence's context is cut into partitions of partition_tokens tokens (a
 * multiple of 16, 16 .. 8192); one workgroup attends over one partition of
 * one (sequence, kv head) pair, and a sequence longer than one partition is
 * merged by a log-sum-exp reduce kernel (split-K).  Same result as pa_decode
 * up to float32 rounding.  Every other argument and the error behaviour are
 * pa_decode's; partition_tokens <= 0 returns PA_ERR_INVALID_ARGUMENT, a value
 * not a multiple of 16 PA_ERR_INVALID_ARGUMENT, above 8192 PA_ERR_UNSUPPORTED.
 *
 * pa_decode_partitioned_workspace_bytes -- its workspace size: one float32
 * record of head_dim + 2 values per (sequence, query head, partition of the
 * longest context), 0 when max_context_len fits one partition.  Returns 0
 * for invalid sizes.  (With partition_tokens 0 it equals
 * pa_decode_workspace_bytes, which also sizes pa_append_decode and
 * pa_decode_sliding with partition_tokens 0.)
 */
pa_status pa_decode_partitioned(const void* q, const void* k_pool, const void* v_pool,
                                const pa_pool_desc* pool, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* context_lens,
                                int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads,
                                float scale, void* out, void* workspace, size_t workspace_bytes,
                                int32_t partition_tokens, void* stream);
size_t pa_decode_partitioned_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                             const pa_pool_desc* pool, int32_t max_context_len,
                                             int32_t partition_tokens);

/*
 * pa_decode_sliding -- pa_decode for a layer trained with sliding-window
 * attention ("vLLM Framework and Inference Engine Design", section "How does
 * it support prompts of arbitrary length? Does it have a sliding window?":
 * each token attends only to the last W tokens, so only the blocks inside the
 * window are needed and older ones may be released).
 *
 *   window        W >= 1 tokens: the token being decoded (position T_i - 1)
 *                 attends to positions max(0, T_i - W) .. T_i - 1.  W >= T_i
 *                 gives pa_decode's result bit for bit.
 *   block_tables  only entries of blocks holding those positions are read
 *                 (at most ceil(W / B) + 1 per sequence); entries before them
 *                 may hold anything, e.g. -1 for released blocks.
 *
 *   partition_tokens  0: the library's split, as pa_decode; > 0: fixed
 *                 partitions of that many tokens, as pa_decode_partitioned
 *                 (partitions start at the tile holding the window's first
 *                 position).  Workspace: pa_decode_partitioned_workspace_bytes
 *                 with the same partition_tokens.
 *
 * Every other argument and the error behaviour are those of pa_decode.
 * window < 1 returns PA_ERR_INVALID_ARGUMENT.
 */
pa_status pa_decode_sliding(const void* q, const void* k_pool, const void* v_pool,
                            const pa_pool_desc* pool, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads,
                            float scale, int32_t window, void* out, void* workspace,
                            size_t workspace_bytes, int32_t partition_tokens, void* stream);

/*
 * FP8 KV pools ("vLLM Framework and Inference Engine Design", engine
 * settings: kv_cache_dtype "fp8" halves the KV memory; "Inside vLLM"
 * (besthub), "Quantization: Reducing Weight & KV Precision": the KV cache
 * stored in FP8).  The pages fix neither format nor scale; here the pools
 * hold OCP E4M3 codes (1 byte per element, same [num_blocks][num_kv_heads]
 * [block_size][head_dim] layout) with one float32 scale for the key pool and
 * one for the value pool: code = E4M3(x / scale), rounded to nearest even and
 * saturated to +-448; value = code * scale.  pool->dtype names the element
 * type of the rows written (k, v) and of q and out.
 *
 * pa_write_kv_fp8 -- pa_write_kv into FP8 pools: k and v ([num_tokens]
 *                 [num_kv_heads][head_dim], pool->dtype, any of the three)
 *                 are quantized with k_scale / v_scale (finite, > 0).
 * pa_decode_fp8 -- pa_decode over FP8 pools (q and out fp16 or bf16).  The
 *                 codes are converted exactly to the compute type; the key
 *                 scale multiplies the scores and the value scale the output.
 *                 Always the balanced split: partition_tokens is 0 and fp32,
 *                 blocks under 16 tokens or over 1024 sequences return
 *                 PA_ERR_UNSUPPORTED.  Workspace: pa_decode_workspace_bytes
 *                 with the same desc and partition_tokens 0.
 */
pa_status pa_write_kv_fp8(const void* k, const void* v, const int32_t* slot_mapping,
                          int32_t num_tokens, void* k_pool, void* v_pool,
                          const pa_pool_desc* pool, float k_scale, float v_scale, void* stream);
pa_status pa_decode_fp8(const void* q, const void* k_pool, const void* v_pool,
                        const pa_pool_desc* pool, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                        int32_t max_context_len, int32_t num_q_heads, float scale, float k_scale,
                        float v_scale, void* out, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * pa_append_decode -- one whole decode step in one call: every sequence's
 * newest token is placed in the pools and then attended over, with the same
 * result as
 *   pa_write_kv(new_k, new_v, slot_mapping, num_seqs, ...), then pa_decode(...)
 * where slot_mapping[i] is the slot of token T_i - 1 of sequence i (the slot
 * write and the block-table lookup of the same page as above; the newest
 * token counts in T_i).  Arguments are those of pa_decode, plus
 *
 *   new_k, new_v  [num_seqs][num_kv_heads][head_dim], pool element type: the
 *                 K and V rows of token T_i - 1 of sequence i.  Rows of
 *                 sequences with T_i == 0 are ignored.
 *   k_pool, v_pool  written: token T_i - 1's rows go to block
 *                 block_tables[i][(T_i - 1) / B] at offset (T_i - 1) % B; an
 *                 entry outside [0, num_blocks) skips that write.
 *
 * Contract: the slot of token T_i - 1 is read by no other sequence of the
 * call (a block being appended to is private to its sequence).  On the
 * balanced split the decode takes the newest rows straight from new_k / new_v
 * and the workgroup that attends over a sequence's last tile also stores
 * them, so the step is two kernels instead of three; with fixed partitions
 * the rows are written first and the decode follows.  partition_tokens: 0
 * for the library's split (as pa_decode), > 0 for fixed partitions (as
 * pa_decode_partitioned).  Workspace: pa_decode_partitioned_workspace_bytes
 * with the same partition_tokens.
 */
pa_status pa_append_decode(const void* q, const void* new_k, const void* new_v,
                           void* k_pool, void* v_pool, const pa_pool_desc* pool,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs,
                           int32_t max_context_len, int32_t num_q_heads, float scale,
                           void* out, void* workspace, size_t workspace_bytes,
                           int32_t partition_tokens, void* stream);

/*
 * pa_append_decode_fp8 -- pa_append_decode over FP8 pools: every sequence's
 * newest token is quantized into the pools and attended over, with the same
 * bits as
 *   pa_write_kv_fp8(new_k, new_v, slot_mapping, num_seqs, ..., k_scale, v_scale),
 *   then pa_decode_fp8(...)
 * (slot_mapping as for pa_append_decode; the FP8 pool format of the vLLM-design
 * page's engine settings, kv_cache_dtype "fp8", as pa_write_kv_fp8 states it).
 * new_k, new_v are [num_seqs][num_kv_heads][head_dim] in pool->dtype (fp16 or
 * bf16, the type of q and out).  Other arguments, the contract on the newest
 * token's slot and the workspace are those of pa_append_decode and
 * pa_decode_fp8 (balanced split only, no partition argument).
 */
pa_status pa_append_decode_fp8(const void* q, const void* new_k, const void* new_v,
                               void* k_pool, void* v_pool, const pa_pool_desc* pool,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t num_seqs,
                               int32_t max_context_len, int32_t num_q_heads, float scale,
                               float k_scale, float v_scale, void* out, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * pa_prefill -- causal attention of a prompt chunk through the block table
 * (chunked prefill: "vLLM Framework and Inference Engine Design", scheduler
 * step and "How does it support prompts of arbitrary length?": a long prompt
 * is read in chunks that run in one batch with other requests' decode
 * tokens).  Sequence i brings M_i = query_start[i+1] - query_start[i] query
 * rows, its last M_i tokens (their K/V already written, e.g. by pa_write_kv);
 * query row r sits at position T_i - M_i + r and attends to positions
 * 0 .. T_i - M_i + r.  A decode token is M_i = 1; batches may mix both.
 *
 *   q, out        [query_start[num_seqs]][num_q_heads][head_dim], pool dtype;
 *                 rows query_start[i] .. query_start[i+1] - 1 belong to
 *                 sequence i.
 *   query_start   int32 [num_seqs + 1], non-decreasing, query_start[0] = 0.
 *   context_lens  T_i, counting the chunk; M_i <= T_i.
 *   max_query_len host bound on every M_i (sizes the grid), at most
 *                 max_context_len.
 *
 * Other arguments as pa_decode (no workspace).  16-bit pools only (fp32 pools
 * return PA_ERR_UNSUPPORTED).  Contract violations clamp: M_i into [0, T_i],
 * T_i into [0, max_context_len], table entries into the pool.
 */
pa_status pa_prefill(const void* q, const void* k_pool, const void* v_pool,
                     const pa_pool_desc* pool, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* context_lens,
                     const int32_t* query_start, int32_t num_seqs, int32_t max_context_len,
                     int32_t max_query_len, int32_t num_q_heads, float scale, void* out,
                     void* stream);

/*
 * pa_copy_blocks -- copy whole physical blocks, the copy behind copy-on-write
 * ("vLLM Framework and Inference Engine Design", section "What operations can
 * cause memory fragmentation, and how does vLLM avoid it?": a block shared
 * through reference counts is copied only when a sequence has to write into
 * it; bibekananda.in, "vLLM", section "The part that is easy to miss": the
 * writer gets a fresh block and the shared one stays untouched).  One call
 * copies the same block pairs in every given pool, e.g. the K and V pools of
 * every layer of a model, in one launch.
 *
 *   pools         HOST array of num_pools DEVICE pointers (16-byte aligned);
 *                 each pool is num_blocks blocks of block_bytes bytes (a
 *                 pa_pool_desc pool has block_bytes = num_kv_heads *
 *                 block_size * head_dim * element bytes, 1 byte for FP8).
 *   block_bytes   a positive multiple of 16, at most 2^30.
 *   block_mapping DEVICE int32 [num_pairs][2]: (source, destination).  For
 *                 every pool, destination block = source block, raw bytes.
 *                 A pair with an entry outside [0, num_blocks) is skipped.
 *                 Contract: destinations are distinct and none is a source
 *                 (a copy-on-write destination is always a fresh block);
 *                 otherwise the affected blocks are unspecified.
 *   num_pools     >= 1; num_pairs >= 0 (0: nothing is enqueued).
 *
 * The pool pointers are passed by value to the kernel (64 pools per launch;
 * more pools take more launches), so the call allocates nothing.
 */
pa_status pa_copy_blocks(void* const* pools, int32_t num_pools, int32_t num_blocks,
                         int64_t block_bytes, const int32_t* block_mapping, int32_t num_pairs,
                         void* stream);

/*
 * pa_check_inputs -- flag the device-side contract violations of the arrays a
 * write or decode call reads.  The kernels stay inside the pools whatever
 * these arrays hold (they skip or clamp), but silently; this call reports.
 * It never reads the pools.  The rules are those of the slot and table
 * definitions (vLLM-design page, "How is vLLM's KV cache paged?": one slot per
 * new token, slot = block * B + offset; "What is the essence of vLLM's
 * PagedAttention?": a sequence's table names the blocks of its first T tokens).
 *
 *   slot_mapping, num_tokens      as pa_write_kv (NULL / 0: not checked).
 *   block_tables, max_blocks_per_seq, context_lens, num_seqs, max_context_len
 *                                 as pa_decode (NULL / 0: not checked).
 *   pool                          the pool the arrays address.
 *   report        DEVICE int32 [4], written: [0] the number of violations;
 *                 [1] the kind of the first one, [2] its index, [3] its value
 *                 (all 0 when there is none).  Kinds, in the order "first"
 *                 follows (then by index):
 *                   PA_CHECK_SLOT_RANGE  slot_mapping[n] >= num_blocks * B
 *                                        (index n, value the slot);
 *                   PA_CHECK_SLOT_DUP    a live slot used by more than one
 *                                        token, every such token counted
 *                                        (index n, value the slot);
 *                   PA_CHECK_LENGTH      context_lens[i] outside
 *                                        [0, max_context_len] (index i);
 *                   PA_CHECK_TABLE       block_tables[i][j] outside
 *                                        [0, num_blocks) for j < ceil(T_i/B),
 *                                        T_i clamped as the kernels do
 *                                        (index i * max_blocks_per_seq + j).
 *   scratch       DEVICE buffer of pa_check_scratch_bytes(pool) bytes for the
 *                 duplicate test (two bits per slot); NULL skips that test.
 *
 * Work is enqueued on `stream` like the other calls; read `report` after the
 * stream reaches that point.  Invalid scalars return an error and enqueue
 * nothing.
 */
enum {
  PA_CHECK_SLOT_RANGE = 1,
  PA_CHECK_SLOT_DUP = 2,
  PA_CHECK_LENGTH = 3,
  PA_CHECK_TABLE = 4
};
size_t pa_check_scratch_bytes(const pa_pool_desc* pool);
pa_status pa_check_inputs(const int32_t* slot_mapping, int32_t num_tokens,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                          const pa_pool_desc* pool, int32_t* report, void* scratch, void* stream);

/*
 * pa_profile_start / pa_profile_stop -- kernel timing for measurements; not
 * needed to compute anything.  Between the two calls, every pa_decode,
 * pa_decode_partitioned, pa_append_decode, pa_decode_sliding, the FP8 decode
 * calls and pa_prefill launch their attention kernel (the balanced-split
 * stream kernel, the fixed-partition kernel, or the prefill kernel), and every
 * pa_copy_blocks and pa_stream_read launch, with a HIP start and stop event
 * attached to that dispatch; the piece merge is not included.  pa_profile_stop
 * turns timing off, waits for the recorded events, and returns how many
 * launches were timed and their mean duration in microseconds (0 launches:
 * mean 0).  The switch is process-wide; while it is on each call creates two
 * events, so it does not belong on a path that must not allocate.
 */
pa_status pa_profile_start(void);
pa_status pa_profile_stop(int32_t* launches, double* mean_us);

/*
 * pa_stream_read -- read `bytes` bytes of a device buffer once, 16 bytes per
 * load with several loads in flight per thread (a measurement helper, not part
 * of the computation: the read ceiling that the decode kernels' KV bandwidth is
 * set against).  buf is 16-byte aligned and bytes a multiple of 16 (else
 * PA_ERR_INVALID_ARGUMENT); sink is a device uint32, written only when the
 * data match a fixed 32-bit hash (it exists so that no load can be dropped).
 * Its launch is timed by pa_profile_start / pa_profile_stop like the attention
 * kernels.
 */
pa_status pa_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* pa_status_string(pa_status status);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTENTION_H */
