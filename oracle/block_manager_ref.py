"""CPU oracle for the host side of the paged KV cache: the block manager
(free queue, reference counts, prefix hashes, copy-on-write) and the block
copy that copy-on-write asks for.

TEST INFRASTRUCTURE ONLY.  This module is an independent definition that the
library's native block manager and its block-copy kernel are checked against.
Only the test suite, the smoke check in ``__graft_entry__`` and the
CPU-baseline leg of ``bench.py`` may import it; the library never imports it
and it imports nothing from the library.  Plain Python lists and dicts, with
``hashlib.sha256`` as the one library primitive; pools are NumPy arrays.

What it follows, page by page:

* "vLLM Framework and Inference Engine Design" (vineetganti.com), section
  "How is vLLM's KV cache paged?": a sequence grows by taking a block from a
  free list when its last block is full and appending it to its block table,
  copying nothing; every block carries a reference count; with prefix caching
  a full block is also named by a hash of its own tokens and of all tokens
  before it, so a request whose prompt begins the same way reuses the blocks
  and skips that much prefill; when a request ends each of its blocks loses a
  reference, a block at zero goes back to the free list but keeps its hash
  and can still be hit until its space is needed, and the least recently
  used blocks are reused first.
* Same page, section "What operations can cause memory fragmentation, and how
  does vLLM avoid it?": every block has the same size, so any free block
  serves any request; reference counts let requests with a common prefix
  share blocks; the original design copies a shared block only when a
  sequence has to write into it (copy-on-write), while the V1 engine shares
  only full blocks, which are never written again.
* sudo.vn, "vLLM self-hosted LLM", section "Prefix caching: reusing the KV of
  identical prefixes": only full blocks are cached; a block's hash is made
  from the previous block's hash, the block's token ids and extra values such
  as a cache salt, so it stands for the whole prefix; SHA-256 is the default
  hash; blocks nobody references sit in a free queue and are evicted least
  recently used first; a salt restricts sharing to requests with that salt.
* bibekananda.in, "vLLM", section "The part that is easy to miss": requests
  with a common prefix point at the same blocks and the engine counts the
  references; a request that writes past the shared region gets fresh blocks
  of its own and the shared ones are left untouched.

Readings taken where the pages leave a step open:

* Hash input: the parent's 32-byte digest followed by the block's token ids
  as little-endian int32.  The first block's parent is the SHA-256 of the
  salt bytes (the empty string when there is no salt), so every hashed
  message has the same length and two prefixes collide only through a
  SHA-256 collision.
* Only full blocks get a hash, when they become full: at allocation for the
  full blocks of a prompt, on the append that fills a block.  The first
  block registered under a hash keeps the name; a later block with an equal
  hash holds the hash but is not registered (it can be hit only by its own
  sequence's table).
* Prefix match: the longest run of leading full prompt blocks whose hashes
  are registered, capped so that at least one prompt token is left to
  compute (the step must still produce the last prompt token's output).
* Free queue: block ids in ascending order at start; allocation takes the
  head; a block whose count drops to zero joins the tail.  A request's blocks
  are released last block first, so its later blocks are reused before its
  earlier ones (a hit on a block needs hits on every block before it).  A
  hit on a block with count zero takes it out of the queue; a block taken
  from the head for new tokens loses its hash (eviction).
* Fork (the original design's sharing, e.g. parallel samples of one prompt):
  the child shares every block of the parent, the partial last block too.
* Append: a token that starts a new block takes a free block.  Otherwise, if
  the last block is shared (count > 1), copy-on-write: a free block is taken,
  the whole old block is copied into it (reported as a (source, destination)
  pair for the copy kernel) and the old block loses one reference.
* An operation that needs more free blocks than there are fails and changes
  nothing.  Unknown or duplicate sequence ids are errors.
* Block copy: ``pool[dst] = pool[src]`` for every pair, all pools, whole
  blocks, raw bytes, every source read before any destination is written.
  Destinations are distinct and are not sources (a copy-on-write destination
  is always a fresh block).

Parity pins (tests/test_oracle_pins.py): the pages' worked examples (three
prompts sharing a system prompt match 0, 10 and 10 blocks of 16 tokens; the
fragmentation example's 2,016 paged slots; twelve requests sharing an
1,800-token prefix), brute-force invariants over random operation sequences,
the chain property of the hash, salt isolation, LRU reuse after free, and the
decode-through-a-copied-block invariance.  No function here is "parity
unpinned".
"""

from __future__ import annotations

import hashlib
import struct

import numpy as np


class OutOfBlocks(RuntimeError):
    """Raised when an operation needs more free blocks than the queue holds."""


def salt_digest(salt: bytes = b"") -> bytes:
    """Parent digest of a sequence's first block: SHA-256 of the salt."""
    return hashlib.sha256(bytes(salt)).digest()


def block_digest(parent: bytes, tokens) -> bytes:
    """SHA-256 of the parent digest followed by the block's token ids
    (little-endian int32)."""
    if len(parent) != 32:
        raise ValueError("parent digest must be 32 bytes")
    body = b"".join(struct.pack("<i", int(t)) for t in tokens)
    return hashlib.sha256(parent + body).digest()


def chain_digests(tokens, block_size: int, salt: bytes = b"") -> list[bytes]:
    """Digests of the full blocks of a token list, each chained on the one
    before it; a trailing partial block has none."""
    out = []
    parent = salt_digest(salt)
    for j in range(len(tokens) // block_size):
        parent = block_digest(parent, tokens[j * block_size:(j + 1) * block_size])
        out.append(parent)
    return out


class BlockManagerRef:
    """The block manager written as plain Python state.

    ``free`` is a list in queue order (head first); ``ref`` and ``digest`` are
    per-block lists; ``cached`` maps a registered digest to its block;
    ``seqs`` maps a sequence id to its tokens, its blocks and its salt.
    """

    def __init__(self, num_blocks: int, block_size: int, prefix_caching: bool = True):
        if num_blocks < 0 or block_size < 1:
            raise ValueError("bad pool size")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.prefix_caching = prefix_caching
        self.free = list(range(num_blocks))
        self.ref = [0] * num_blocks
        self.digest: list[bytes | None] = [None] * num_blocks
        self.cached: dict[bytes, int] = {}
        self.seqs: dict[int, dict] = {}

    # -- free queue ---------------------------------------------------------
    def _take_free(self) -> int:
        """Pop the queue's head for new tokens; it loses its hash."""
        b = self.free.pop(0)
        d = self.digest[b]
        if d is not None:
            if self.cached.get(d) == b:
                del self.cached[d]
            self.digest[b] = None
        self.ref[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)

    def _register(self, b: int, d: bytes) -> None:
        self.digest[b] = d
        if d not in self.cached:
            self.cached[d] = b

    # -- requests -----------------------------------------------------------
    def allocate(self, seq: int, prompt, salt: bytes = b"") -> int:
        """Admit a sequence with its prompt; returns the number of prompt
        tokens whose KV is already in the pool (prefix hits)."""
        if seq in self.seqs:
            raise KeyError(f"sequence {seq} exists")
        prompt = [int(t) for t in prompt]
        bs = self.block_size
        digests = chain_digests(prompt, bs, salt) if self.prefix_caching else []
        hits = []
        limit = (len(prompt) - 1) // bs if prompt else 0   # leave one token to compute
        for j in range(min(limit, len(digests))):
            b = self.cached.get(digests[j])
            if b is None:
                break
            hits.append(b)
        fresh_needed = -(-len(prompt) // bs) - len(hits)
        revived = sum(1 for b in hits if self.ref[b] == 0)
        if fresh_needed > len(self.free) - revived:
            raise OutOfBlocks(f"sequence {seq} needs {fresh_needed} free blocks")
        for b in hits:
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
        blocks = list(hits)
        for j in range(len(hits), len(hits) + fresh_needed):
            b = self._take_free()
            blocks.append(b)
            if j < len(digests):
                self._register(b, digests[j])
        self.seqs[seq] = {"tokens": prompt, "blocks": blocks, "salt": bytes(salt)}
        return len(hits) * bs

    def append(self, seq: int, token: int):
        """Add one token; returns (slot, cow) where cow is the (source,
        destination) block pair to copy first, or None."""
        s = self.seqs[seq]
        bs = self.block_size
        t = len(s["tokens"])
        cow = None
        if t % bs == 0:
            if not self.free:
                raise OutOfBlocks(f"sequence {seq} needs a block")
            s["blocks"].append(self._take_free())
        else:
            last = s["blocks"][-1]
            if self.ref[last] > 1:
                if not self.free:
                    raise OutOfBlocks(f"sequence {seq} needs a block for copy-on-write")
                b = self._take_free()
                self.ref[last] -= 1
                s["blocks"][-1] = b
                cow = (last, b)
        s["tokens"].append(int(token))
        b = s["blocks"][t // bs]
        if self.prefix_caching and (t + 1) % bs == 0:
            self._register(b, chain_digests(s["tokens"], bs, s["salt"])[-1])
        return b * bs + t % bs, cow

    def fork(self, parent: int, child: int) -> None:
        """The child shares all of the parent's blocks."""
        if child in self.seqs:
            raise KeyError(f"sequence {child} exists")
        p = self.seqs[parent]
        for b in p["blocks"]:
            self.ref[b] += 1
        self.seqs[child] = {"tokens": list(p["tokens"]), "blocks": list(p["blocks"]),
                            "salt": p["salt"]}

    def free_seq(self, seq: int) -> None:
        """End a sequence: one reference less per block, last block first."""
        s = self.seqs.pop(seq)
        for b in reversed(s["blocks"]):
            self._release(b)

    # -- views --------------------------------------------------------------
    def block_table(self, seq: int) -> list[int]:
        return list(self.seqs[seq]["blocks"])

    def num_tokens(self, seq: int) -> int:
        return len(self.seqs[seq]["tokens"])

    def num_free(self) -> int:
        return len(self.free)

    def slot(self, seq: int, t: int) -> int:
        """block_table[floor(t/B)] * B + (t mod B) for a held token."""
        s = self.seqs[seq]
        if not 0 <= t < len(s["tokens"]):
            raise IndexError("token not held by the sequence")
        return s["blocks"][t // self.block_size] * self.block_size + t % self.block_size

    def tables(self, seqs, max_blocks: int):
        """int32 block tables [len(seqs)][max_blocks] (unused entries -1) and
        context lengths, for a decode launch."""
        tab = np.full((len(seqs), max_blocks), -1, dtype=np.int32)
        lens = np.zeros(len(seqs), dtype=np.int32)
        for i, q in enumerate(seqs):
            blocks = self.seqs[q]["blocks"]
            if len(blocks) > max_blocks:
                raise ValueError("table row too short")
            tab[i, :len(blocks)] = blocks
            lens[i] = len(self.seqs[q]["tokens"])
        return tab, lens


def copy_blocks(pools, pairs, inplace: bool = False):
    """Copy whole blocks: for every (src, dst) pair, ``pool[dst] = pool[src]``
    in every pool (axis 0 is the block).  All sources are read before any
    destination is written; destinations must be distinct and not sources."""
    pairs = [(int(s), int(d)) for s, d in pairs]
    dsts = [d for _, d in pairs]
    if len(set(dsts)) != len(dsts) or set(dsts) & {s for s, _ in pairs}:
        raise ValueError("copy destinations must be distinct and not sources")
    out = []
    for pool in pools:
        n = pool.shape[0]
        if any(not (0 <= s < n and 0 <= d < n) for s, d in pairs):
            raise ValueError("block outside the pool")
        src_rows = [pool[s].copy() for s, _ in pairs]
        new = pool if inplace else pool.copy()
        for (_, d), rows in zip(pairs, src_rows):
            new[d] = rows
        out.append(new)
    return out
