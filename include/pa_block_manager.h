/*
 * pa_block_manager.h -- C ABI of libpa's host-side block manager: the
 * bookkeeping that decides which physical block of the KV pools each token
 * of each sequence lives in.  Plain host code; no call touches the GPU.
 *
 * State and transitions (policies from "vLLM Framework and Inference Engine
 * Design", vineetganti.com, sections "How is vLLM's KV cache paged?" and
 * "What operations can cause memory fragmentation, and how does vLLM avoid
 * it?"; the hash from sudo.vn, "vLLM self-hosted LLM", section "Prefix
 * caching: reusing the KV of identical prefixes"):
 *
 *   - per block: a reference count, an optional digest, and a place in an
 *     LRU queue while its count is zero;
 *   - per sequence: its block list (the block table), token count and the
 *     token ids of its partial last block;
 *   - append: a token that starts a new block takes the queue's head block
 *     (dropping any digest it held); a token that completes a block gives the
 *     block its digest; no KV is ever moved to grow a sequence;
 *   - allocate with prefix caching: leading full prompt blocks whose digests
 *     are registered are taken with one more reference each (a hit on a
 *     queued block takes it out of the queue);
 *   - release: every block of the sequence drops one reference; blocks that
 *     reach zero join the queue's tail still holding their digest, so they
 *     remain hittable until reused;
 *   - copy-on-write: writing into a last block whose count is above one
 *     moves the writer to a fresh block and reports the (old, new) pair for
 *     pa_copy_blocks, which the caller runs before the write; fork is how
 *     partial blocks come to be shared;
 *   - digests: SHA-256 chained through the parent block's digest, over full
 *     blocks only, seeded by a per-request salt.
 *
 * Conventions:
 *
 *   - Block ids are in [0, num_blocks); a block holds block_size tokens; the
 *     slot of token t of a sequence is table[t / B] * B + t % B, the slot
 *     mapping pa_write_kv takes.
 *   - Hash of full block j of a sequence: SHA-256 over 32 + 4 * block_size
 *     bytes, the parent digest followed by the block's token ids as
 *     little-endian int32.  Block 0's parent is the SHA-256 of the salt
 *     bytes (of the empty string without a salt).  Only the first block to
 *     get a hash is registered under it (found by later prompts).
 *   - Prefix match: the longest run of leading full prompt blocks whose
 *     hashes are registered, leaving at least one prompt token unmatched.
 *     A prompt's full blocks are registered when it is admitted, before its
 *     KV is computed: a request that hits them must not read them before
 *     the prefill that writes them has run (e.g. admit it in a later step,
 *     or order its attention after that prefill on the stream).
 *   - Free queue: block ids ascending at creation.  Taking a block pops the
 *     head and drops the block's hash; a block whose count drops to zero
 *     joins the tail; a freed sequence releases its blocks last block first.
 *     A prefix hit on a block at count zero takes it out of the queue.
 *   - Every call either succeeds or returns an error and changes nothing.
 *     PA_ERR_OUT_OF_BLOCKS: not enough free blocks.  PA_ERR_INVALID_ARGUMENT:
 *     a null pointer, a negative size, an unknown sequence id, or an id that
 *     is already live where a new one is expected.  PA_ERR_HOST_MEMORY: a
 *     host allocation failed part way; the manager should then be destroyed.
 *   - Output arrays are HOST memory owned by the caller.  A manager is not
 *     thread-safe: one thread (the scheduler) drives it.
 */
#ifndef PA_BLOCK_MANAGER_H
#define PA_BLOCK_MANAGER_H

#include <stddef.h>
#include <stdint.h>

#include "paged_attention.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/* A manager for a pool of num_blocks blocks (>= 0) of block_size tokens
 * (>= 1); prefix_caching != 0 turns hashing and prefix hits on.  *out
 * receives the handle (NULL on error). */
pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, int32_t prefix_caching,
                       pa_block_manager** out);
void pa_bm_destroy(pa_block_manager* bm);

/* Admit sequence seq_id with its prompt (num_tokens >= 0 token ids).  Blocks
 * for every prompt token are held on return: prefix hits shared, the rest
 * taken from the free queue.  *cached_tokens (may be NULL) receives the
 * number of leading prompt tokens whose KV is already in the pools (a
 * multiple of block_size, below num_tokens). */
pa_status pa_bm_allocate(pa_block_manager* bm, int64_t seq_id, const int32_t* tokens,
                         int32_t num_tokens, const void* salt, int32_t salt_bytes,
                         int32_t* cached_tokens);

/* One decode step's tokens: token tokens[i] is appended to sequence
 * seq_ids[i], in order (an id may repeat).  slots[i] receives the token's
 * slot.  Copy-on-write pairs are written to cow_pairs as (source,
 * destination) int32 pairs, in order, and *num_cow receives their count (at
 * most n); copy them with pa_copy_blocks before writing the new tokens.
 * All n appends happen, or none (PA_ERR_OUT_OF_BLOCKS, checked up front). */
pa_status pa_bm_append(pa_block_manager* bm, const int64_t* seq_ids, const int32_t* tokens,
                       int32_t n, int32_t* slots, int32_t* cow_pairs, int32_t* num_cow);

/* A new sequence child sharing every block (and token) of parent. */
pa_status pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child);

/* End a sequence: each of its blocks loses one reference. */
pa_status pa_bm_free(pa_block_manager* bm, int64_t seq_id);

/* Block tables for a decode launch: row i of block_tables ([num_seqs]
 * [max_blocks_per_seq]) receives sequence seq_ids[i]'s blocks, padded with
 * -1, and context_lens[i] its token count.  A sequence holding more than
 * max_blocks_per_seq blocks is PA_ERR_INVALID_ARGUMENT. */
pa_status pa_bm_tables(const pa_block_manager* bm, const int64_t* seq_ids, int32_t num_seqs,
                       int32_t max_blocks_per_seq, int32_t* block_tables,
                       int32_t* context_lens);

/* Free blocks (cached ones included); -1 for a NULL handle. */
int32_t pa_bm_num_free(const pa_block_manager* bm);

/* Inspection, for tests and metrics.  pa_bm_block_info: reference count,
 * whether the block holds a hash, the hash (32 bytes, zero without one) and
 * whether it is the registered holder of that hash.  pa_bm_free_queue:
 * up to capacity free block ids in queue order, head first; *count receives
 * the queue length. */
pa_status pa_bm_block_info(const pa_block_manager* bm, int32_t block, int32_t* ref_count,
                           int32_t* has_digest, uint8_t* digest, int32_t* registered);
pa_status pa_bm_free_queue(const pa_block_manager* bm, int32_t* blocks, int32_t capacity,
                           int32_t* count);

/* SHA-256 (FIPS 180-4) of len bytes at data into digest[32]; the hash the
 * manager names blocks with, exported so callers can compute block names. */
pa_status pa_sha256(const void* data, size_t len, uint8_t* digest);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCK_MANAGER_H */
