// Host block manager: free queue, reference counts, chained prefix hashes and
// copy-on-write over one pool of physical blocks.  Plain C++ (no HIP), so it
// also builds with g++ and sanitizers for host tests.
//
// The free queue is an intrusive doubly linked list over block ids, so taking
// the head, adding at the tail and taking out a block hit by a prefix match
// are all O(1), as the pages ask of allocation and release.  A sequence keeps
// its block list, its token count, the token ids of its partial last block and
// the digest of its last full block: enough to hash the next block when it
// fills, without keeping the whole token history.
#include <algorithm>
#include <array>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_block_manager.h"
#include "pa_sha256.h"

namespace {

using Digest = std::array<uint8_t, 32>;

struct DigestHash {
  size_t operator()(const Digest& d) const {
    uint64_t h;
    std::memcpy(&h, d.data(), sizeof(h));
    return static_cast<size_t>(h);
  }
};

struct Seq {
  int32_t num_tokens = 0;
  std::vector<int32_t> blocks;
  std::vector<int32_t> tail;   // token ids of the partial last block
  Digest parent{};             // digest of the last full block (block 0: the salt's)
  // scratch of one pa_bm_append call's dry run, valid while mark == the call's epoch
  uint32_t mark = 0;
  int32_t extra = 0;           // tokens the batch added so far
  bool private_last = false;   // the batch gave the sequence a block of its own
};

Digest salt_digest(const void* salt, int32_t salt_bytes) {
  Digest d;
  pa::sha256(salt_bytes > 0 ? salt : "", static_cast<size_t>(salt_bytes), d.data());
  return d;
}

// SHA-256 of the parent digest followed by block_size little-endian int32 ids
Digest block_digest(const Digest& parent, const int32_t* tokens, int32_t block_size) {
  pa::Sha256 h;
  h.update(parent.data(), parent.size());
  uint8_t le[4 * 64];
  for (int32_t i = 0; i < block_size; i += 64) {
    const int32_t n = std::min<int32_t>(64, block_size - i);
    for (int32_t j = 0; j < n; ++j) {
      const uint32_t t = static_cast<uint32_t>(tokens[i + j]);
      le[4 * j] = uint8_t(t);
      le[4 * j + 1] = uint8_t(t >> 8);
      le[4 * j + 2] = uint8_t(t >> 16);
      le[4 * j + 3] = uint8_t(t >> 24);
    }
    h.update(le, 4 * size_t(n));
  }
  Digest d;
  h.finish(d.data());
  return d;
}

}  // namespace

struct pa_block_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 1;
  bool caching = true;
  std::vector<int32_t> ref, prev, next;
  std::vector<Digest> digest;
  std::vector<uint8_t> has_digest;
  int32_t head = -1, tail = -1, num_free = 0;
  std::unordered_map<Digest, int32_t, DigestHash> cached;
  std::unordered_map<int64_t, Seq> seqs;
  // pa_bm_append's dry run: references a batch gives up per block, valid while
  // drop_mark[b] == epoch
  uint32_t epoch = 0;
  std::vector<uint32_t> drop_mark;
  std::vector<int32_t> drop_count;
  std::vector<Seq*> batch;

  // -- free queue ------------------------------------------------------------
  void push_tail(int32_t b) {
    prev[b] = tail;
    next[b] = -1;
    if (tail >= 0) next[tail] = b; else head = b;
    tail = b;
    ++num_free;
  }
  void unlink(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
    prev[b] = next[b] = -1;
    --num_free;
  }
  // the head, for new tokens: it loses its hash and gets one reference
  int32_t take_free() {
    const int32_t b = head;
    unlink(b);
    if (has_digest[b]) {
      auto it = cached.find(digest[b]);
      if (it != cached.end() && it->second == b) cached.erase(it);
      has_digest[b] = 0;
      digest[b] = Digest{};
    }
    ref[b] = 1;
    return b;
  }
  void release(int32_t b) {
    if (--ref[b] == 0) push_tail(b);
  }
  void register_block(int32_t b, const Digest& d) {
    digest[b] = d;
    has_digest[b] = 1;
    cached.emplace(d, b);    // keeps an earlier holder of the same digest
  }
};

extern "C" {

pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, int32_t prefix_caching,
                       pa_block_manager** out) {
  if (!out) return PA_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  if (num_blocks < 0 || block_size < 1) return PA_ERR_INVALID_ARGUMENT;
  pa_block_manager* m = new (std::nothrow) pa_block_manager;
  if (!m) return PA_ERR_HOST_MEMORY;
  try {
    m->num_blocks = num_blocks;
    m->block_size = block_size;
    m->caching = prefix_caching != 0;
    m->ref.assign(num_blocks, 0);
    m->prev.assign(num_blocks, -1);
    m->next.assign(num_blocks, -1);
    m->digest.assign(num_blocks, Digest{});
    m->has_digest.assign(num_blocks, 0);
    m->drop_mark.assign(num_blocks, 0);
    m->drop_count.assign(num_blocks, 0);
  } catch (const std::bad_alloc&) {
    delete m;
    return PA_ERR_HOST_MEMORY;
  }
  for (int32_t b = 0; b < num_blocks; ++b) m->push_tail(b);
  *out = m;
  return PA_OK;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

pa_status pa_bm_allocate(pa_block_manager* bm, int64_t seq_id, const int32_t* tokens,
                         int32_t num_tokens, const void* salt, int32_t salt_bytes,
                         int32_t* cached_tokens) {
  if (!bm || num_tokens < 0 || (num_tokens > 0 && !tokens) || salt_bytes < 0 ||
      (salt_bytes > 0 && !salt))
    return PA_ERR_INVALID_ARGUMENT;
  if (bm->seqs.count(seq_id)) return PA_ERR_INVALID_ARGUMENT;
  const int32_t B = bm->block_size;
  const int32_t full = num_tokens / B;
  const int32_t needed = full + (num_tokens % B != 0);
  try {
    // digests of the full prompt blocks, then the longest registered run
    std::vector<Digest> chain;
    Digest parent{};
    if (bm->caching) {
      parent = salt_digest(salt, salt_bytes);
      chain.reserve(full);
      for (int32_t j = 0; j < full; ++j) {
        parent = block_digest(parent, tokens + int64_t(j) * B, B);
        chain.push_back(parent);
      }
    }
    const int32_t limit = num_tokens > 0 ? (num_tokens - 1) / B : 0;
    std::vector<int32_t> blocks;
    blocks.reserve(needed);
    int32_t revived = 0;
    for (int32_t j = 0; j < limit && j < int32_t(chain.size()); ++j) {
      auto it = bm->cached.find(chain[j]);
      if (it == bm->cached.end()) break;
      blocks.push_back(it->second);
      revived += bm->ref[it->second] == 0;
    }
    const int32_t hits = int32_t(blocks.size());
    if (needed - hits > bm->num_free - revived) return PA_ERR_OUT_OF_BLOCKS;

    Seq s;
    s.num_tokens = num_tokens;
    s.tail.assign(tokens + int64_t(full) * B, tokens + num_tokens);
    s.parent = full > 0 && bm->caching ? chain[full - 1] : parent;
    auto slot = bm->seqs.emplace(seq_id, std::move(s)).first;   // last allocation
    for (int32_t b : blocks) {
      if (bm->ref[b] == 0) bm->unlink(b);
      ++bm->ref[b];
    }
    for (int32_t j = hits; j < needed; ++j) {
      const int32_t b = bm->take_free();
      blocks.push_back(b);
      if (j < int32_t(chain.size())) bm->register_block(b, chain[j]);
    }
    slot->second.blocks = std::move(blocks);
    if (cached_tokens) *cached_tokens = hits * B;
    return PA_OK;
  } catch (const std::bad_alloc&) {
    return PA_ERR_HOST_MEMORY;
  }
}

pa_status pa_bm_append(pa_block_manager* bm, const int64_t* seq_ids, const int32_t* tokens,
                       int32_t n, int32_t* slots, int32_t* cow_pairs, int32_t* num_cow) {
  if (!bm || n < 0 || (n > 0 && (!seq_ids || !tokens || !slots || !cow_pairs)) || !num_cow)
    return PA_ERR_INVALID_ARGUMENT;
  *num_cow = 0;
  const int32_t B = bm->block_size;
  try {
    // dry run: every id known, and the blocks the whole batch takes, in order
    bm->batch.resize(n);
    if (++bm->epoch == 0) {                 // marks wrapped: clear them
      std::fill(bm->drop_mark.begin(), bm->drop_mark.end(), 0u);
      for (auto& kv : bm->seqs) kv.second.mark = 0;
      bm->epoch = 1;
    }
    const uint32_t epoch = bm->epoch;
    int32_t need = 0;
    for (int32_t i = 0; i < n; ++i) {
      auto it = bm->seqs.find(seq_ids[i]);
      if (it == bm->seqs.end()) return PA_ERR_INVALID_ARGUMENT;
      Seq& p = it->second;
      bm->batch[i] = &p;
      if (p.mark != epoch) {
        p.mark = epoch;
        p.extra = 0;
        p.private_last = false;
      }
      const int32_t t = p.num_tokens + p.extra;
      if (t % B == 0) {
        ++need;
        p.private_last = true;
      } else if (!p.private_last) {
        const int32_t last = p.blocks.back();
        if (bm->drop_mark[last] != epoch) {
          bm->drop_mark[last] = epoch;
          bm->drop_count[last] = 0;
        }
        if (bm->ref[last] - bm->drop_count[last] > 1) {
          ++need;
          ++bm->drop_count[last];
          p.private_last = true;
        }
      }
      ++p.extra;
    }
    if (need > bm->num_free) return PA_ERR_OUT_OF_BLOCKS;
    for (int32_t i = 0; i < n; ++i) {
      bm->batch[i]->tail.reserve(B);
      if (bm->batch[i]->num_tokens % B == 0) bm->batch[i]->blocks.reserve(bm->batch[i]->blocks.size() + 1);
    }

    for (int32_t i = 0; i < n; ++i) {
      Seq& s = *bm->batch[i];
      const int32_t t = s.num_tokens;
      if (t % B == 0) {
        s.blocks.push_back(bm->take_free());
      } else {
        const int32_t last = s.blocks.back();
        if (bm->ref[last] > 1) {
          const int32_t b = bm->take_free();
          --bm->ref[last];
          s.blocks.back() = b;
          cow_pairs[2 * *num_cow] = last;
          cow_pairs[2 * *num_cow + 1] = b;
          ++*num_cow;
        }
      }
      const int32_t b = s.blocks[t / B];
      s.num_tokens = t + 1;
      s.tail.push_back(tokens[i]);
      if (int32_t(s.tail.size()) == B) {
        if (bm->caching) {
          s.parent = block_digest(s.parent, s.tail.data(), B);
          bm->register_block(b, s.parent);
        }
        s.tail.clear();
      }
      slots[i] = b * B + t % B;
    }
    return PA_OK;
  } catch (const std::bad_alloc&) {
    return PA_ERR_HOST_MEMORY;
  }
}

pa_status pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child) {
  if (!bm) return PA_ERR_INVALID_ARGUMENT;
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end() || bm->seqs.count(child)) return PA_ERR_INVALID_ARGUMENT;
  try {
    Seq copy = it->second;
    for (int32_t b : copy.blocks) ++bm->ref[b];
    bm->seqs.emplace(child, std::move(copy));
    return PA_OK;
  } catch (const std::bad_alloc&) {
    return PA_ERR_HOST_MEMORY;
  }
}

pa_status pa_bm_free(pa_block_manager* bm, int64_t seq_id) {
  if (!bm) return PA_ERR_INVALID_ARGUMENT;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_INVALID_ARGUMENT;
  const std::vector<int32_t>& blocks = it->second.blocks;
  for (size_t j = blocks.size(); j-- > 0;) bm->release(blocks[j]);
  bm->seqs.erase(it);
  return PA_OK;
}

pa_status pa_bm_tables(const pa_block_manager* bm, const int64_t* seq_ids, int32_t num_seqs,
                       int32_t max_blocks_per_seq, int32_t* block_tables,
                       int32_t* context_lens) {
  if (!bm || num_seqs < 0 || max_blocks_per_seq < 0 ||
      (num_seqs > 0 && (!seq_ids || !context_lens || (max_blocks_per_seq > 0 && !block_tables))))
    return PA_ERR_INVALID_ARGUMENT;
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end() || int32_t(it->second.blocks.size()) > max_blocks_per_seq)
      return PA_ERR_INVALID_ARGUMENT;
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Seq& s = bm->seqs.find(seq_ids[i])->second;
    int32_t* row = block_tables + int64_t(i) * max_blocks_per_seq;
    const int32_t nb = int32_t(s.blocks.size());
    for (int32_t j = 0; j < max_blocks_per_seq; ++j) row[j] = j < nb ? s.blocks[j] : -1;
    context_lens[i] = s.num_tokens;
  }
  return PA_OK;
}

int32_t pa_bm_num_free(const pa_block_manager* bm) { return bm ? bm->num_free : -1; }

pa_status pa_bm_block_info(const pa_block_manager* bm, int32_t block, int32_t* ref_count,
                           int32_t* has_digest, uint8_t* digest, int32_t* registered) {
  if (!bm || block < 0 || block >= bm->num_blocks) return PA_ERR_INVALID_ARGUMENT;
  if (ref_count) *ref_count = bm->ref[block];
  if (has_digest) *has_digest = bm->has_digest[block];
  if (digest) std::memcpy(digest, bm->digest[block].data(), 32);
  if (registered) {
    int32_t r = 0;
    if (bm->has_digest[block]) {
      auto it = bm->cached.find(bm->digest[block]);
      r = it != bm->cached.end() && it->second == block;
    }
    *registered = r;
  }
  return PA_OK;
}

pa_status pa_bm_free_queue(const pa_block_manager* bm, int32_t* blocks, int32_t capacity,
                           int32_t* count) {
  if (!bm || capacity < 0 || (capacity > 0 && !blocks) || !count) return PA_ERR_INVALID_ARGUMENT;
  int32_t i = 0;
  for (int32_t b = bm->head; b >= 0 && i < capacity; b = bm->next[b]) blocks[i++] = b;
  *count = bm->num_free;
  return PA_OK;
}

pa_status pa_sha256(const void* data, size_t len, uint8_t* digest) {
  if (!digest || (len > 0 && !data)) return PA_ERR_INVALID_ARGUMENT;
  pa::sha256(len > 0 ? data : "", len, digest);
  return PA_OK;
}

}  // extern "C"
