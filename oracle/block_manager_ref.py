"""CPU oracle for the host side of the paged KV cache: the block manager
(free queue, reference counts, prefix hashes, copy-on-write) and the block
copy that copy-on-write asks for.

TEST INFRASTRUCTURE ONLY.  This module is an independent definition that the
library's native block manager and its block-copy kernel are checked against.
Only the test suite, the smoke check in ``__graft_entry__`` and the
CPU-baseline leg of ``bench.py`` may import it; the library never imports it
and it imports nothing from the library.  Plain Python lists and dicts, with
``hashlib.sha256`` as the one library primitive; pools are NumPy arrays.

What it follows (the pages fix the policies; the byte layout of a hash and the
tie-breaking orders are readings, listed below):

* "vLLM Framework and Inference Engine Design" (vineetganti.com), section
  "How is vLLM's KV cache paged?": growth by whole blocks from a free list,
  with nothing copied; reference counts on blocks; prefix caching that names
  a full block by a hash covering its tokens and every token before them;
  release that decrements counts and parks zero-count blocks, digest intact,
  for least-recently-used reuse.
* Same page, section "What operations can cause memory fragmentation, and how
  does vLLM avoid it?": equal-size blocks (any free block serves any
  request), sharing through reference counts, and copy-on-write of a shared
  block at the first write into it (the V1 engine shares only full blocks).
* sudo.vn, "vLLM self-hosted LLM", section "Prefix caching: reusing the KV of
  identical prefixes": hashes over full blocks only, each chained on its
  parent's and including extra keys such as a salt; SHA-256; an LRU queue
  of unreferenced blocks; sharing limited to requests with the same salt.
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
