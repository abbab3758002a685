"""Checks that tie the block-manager oracle (oracle/block_manager_ref.py) to
something other than itself.

Each ``pin_*`` function takes the oracle module and raises when it disagrees
with what the pages fix.  tests/test_block_manager_oracle.py runs them on the
real oracle and on planted mistakes.

Sources of truth, none of which is the oracle's own code:

* the pages' worked examples (tests/golden/page_figures.json): three prompts
  sharing a system prompt ("Prefix caching: reusing the KV of identical
  prefixes"), the fragmentation example ("What operations can cause memory
  fragmentation, and how does vLLM avoid it?") and twelve requests sharing an
  1,800-token prefix ("The part that is easy to miss");
* a content model kept beside the manager: a list of token ids per physical
  block, written as a model would write KV.  Every sequence read back through
  its block table must equal the tokens it was given, and a prefix hit must
  land on blocks that already hold the hit tokens;
* brute-force counts: a block's reference count is the number of live tables
  that name it, the free queue holds exactly the blocks nobody references;
* the hash's chain property, salt isolation, and the free queue's order
  derived by hand from the rule stated on the pages.
"""

from __future__ import annotations

import copy
import hashlib
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)

from oracle_pins import load_golden  # noqa: E402


# ---------------------------------------------------------------------------
# the content model: what the pool would hold if every written slot got the
# token id as its "KV"
# ---------------------------------------------------------------------------
class ContentModel:
    def __init__(self, m):
        self.m = m
        self.B = m.block_size
        self.blocks = {}          # physical block -> list of B token ids (None: unwritten)
        self.tokens = {}          # sequence -> the tokens it was given

    def _block(self, b):
        return self.blocks.setdefault(b, [None] * self.B)

    def allocate(self, seq, prompt, salt=b""):
        hit = self.m.allocate(seq, prompt, salt)
        table = self.m.block_table(seq)
        assert hit % self.B == 0 and 0 <= hit <= max(0, len(prompt) - 1)
        for t, tok in enumerate(prompt):
            blk = self._block(table[t // self.B])
            if t < hit:
                assert blk[t % self.B] == tok, "prefix hit on a block holding other tokens"
            else:
                blk[t % self.B] = tok
        self.tokens[seq] = list(prompt)
        return hit

    def append(self, seq, tok):
        slot, cow = self.m.append(seq, tok)
        if cow is not None:
            src, dst = cow
            self.blocks[dst] = list(self._block(src))
        self._block(slot // self.B)[slot % self.B] = tok
        self.tokens[seq].append(tok)
        return slot, cow

    def fork(self, parent, child):
        self.m.fork(parent, child)
        self.tokens[child] = list(self.tokens[parent])

    def free(self, seq):
        self.m.free_seq(seq)
        del self.tokens[seq]

    def check(self, o):
        """Every live sequence reads back its own tokens; counts and the
        queue agree with brute force; digests are the chain's."""
        m = self.m
        refs = [0] * m.num_blocks
        for seq, toks in self.tokens.items():
            table = m.block_table(seq)
            assert len(table) == -(-len(toks) // self.B)
            for t, tok in enumerate(toks):
                assert self.blocks[table[t // self.B]][t % self.B] == tok, "sequence reads foreign KV"
            for b in table:
                refs[b] += 1
        assert refs == m.ref
        assert sorted(m.free) == [b for b in range(m.num_blocks) if refs[b] == 0]
        assert len(set(m.free)) == len(m.free)
        for d, b in m.cached.items():
            assert m.digest[b] == d
        for seq, toks in self.tokens.items():
            chain = o.chain_digests(toks, self.B, m.seqs[seq]["salt"]) if m.prefix_caching else []
            for j, b in enumerate(m.block_table(seq)[:len(chain)]):
                assert m.digest[b] == chain[j], "full block without its chain digest"


def _prompt(rng, n, vocab=50):
    return [int(x) for x in rng.integers(0, vocab, n)]


# ---------------------------------------------------------------------------
# the pages' worked examples
# ---------------------------------------------------------------------------
def pin_prefix_caching_example(o):
    """Three prompts after one system prompt match 0, 10 and 10 blocks of 16
    tokens (160 tokens skipped).  A prompt that repeats a cached one whole
    still leaves its last block to compute."""
    g = load_golden()["prefix_caching_example"]
    B = g["block_size"]
    rng = np.random.default_rng(11)
    system = _prompt(rng, g["shared_prefix_tokens"], vocab=30000)
    m = o.BlockManagerRef(256, B)
    cm = ContentModel(m)
    for i, (n, full, matched, skipped) in enumerate(zip(g["lens"], g["full_blocks"],
                                                        g["matched_blocks"], g["skipped_tokens"])):
        question = [30000 + 1000 * i + x for x in _prompt(rng, n - len(system), vocab=1000)]
        prompt = system + question
        assert len(prompt) // B == full
        hit = cm.allocate(i, prompt)
        assert hit == skipped and hit // B == matched
        cm.check(o)
    assert m.num_free() == 256 - (12 + 2 + 2)
    # 176 tokens = 11 full blocks, all cached: 10 hit, the last is recomputed
    again = cm.tokens[0][:176]
    assert cm.allocate(10, again) == 160
    assert m.block_table(10)[:10] == m.block_table(0)[:10]
    assert m.block_table(10)[10] != m.block_table(0)[10]
    cm.check(o)


def pin_fragmentation_example(o):
    """300, 1,100 and 600 tokens in blocks of 16 take 2,016 slots (the
    contiguous reservation takes 6,144)."""
    f = load_golden()["fragmentation"]
    B = f["block_size"]
    m = o.BlockManagerRef(1000, B)
    rng = np.random.default_rng(12)
    for i, n in enumerate(f["lens"]):
        m.allocate(i, [10000 * (i + 1) + x for x in _prompt(rng, n, vocab=9999)])
    used = m.num_blocks - m.num_free()
    assert used * B == f["paged_slots"]
    assert len(f["lens"]) * f["max_len"] == f["contiguous_slots"]
    for i in range(len(f["lens"])):
        m.free_seq(i)
    assert m.num_free() == 1000 and all(r == 0 for r in m.ref)


def pin_shared_prefix_twelve(o):
    """Twelve requests on an 1,800-token prefix: shared, the prefix takes the
    space of one copy (up to block rounding).  Fork-style sharing copies the
    partial last block for eleven of them when they write past it; prefix
    caching shares the 112 full blocks and gives each its own last block."""
    p = load_golden()["prefix_sharing"]
    B = 16
    per_block = B * p["bytes_per_token"]
    prefix = list(range(p["prefix_tokens"]))
    n = p["requests"]
    # fork: one request, eleven children, all blocks shared
    m = o.BlockManagerRef(4096, B)
    cm = ContentModel(m)
    cm.allocate(0, prefix)
    for c in range(1, n):
        cm.fork(0, c)
    shared_bytes = (m.num_blocks - m.num_free()) * per_block
    printed_shared = p["printed_shared_gb"] * 1e9
    assert printed_shared - 0.0005e9 <= shared_bytes <= printed_shared + 0.0005e9 + per_block
    partial = m.block_table(0)[-1]
    cows = []
    for c in range(n):
        _, cow = cm.append(c, 100000 + c)
        if cow is not None:
            assert cow[0] == partial
            cows.append(cow)
        cm.check(o)
    assert len(cows) == n - 1
    assert m.block_table(n - 1)[-1] == partial     # the last writer owns the original
    assert m.num_blocks - m.num_free() == 113 + (n - 1)
    # prefix caching: each prompt is the prefix plus a token of its own
    m = o.BlockManagerRef(4096, B)
    cm = ContentModel(m)
    held = []
    for c in range(n):
        hit = cm.allocate(c, prefix + [200000 + c])
        assert hit == (0 if c == 0 else 112 * B)
        held.append(len(m.block_table(c)))
        cm.check(o)
    assert m.num_blocks - m.num_free() == 113 + (n - 1)
    copies = sum(held) * per_block
    printed_copies = p["printed_copies_gb"] * 1e9
    assert printed_copies - 0.005e9 <= copies <= printed_copies + 0.005e9 + n * per_block


# ---------------------------------------------------------------------------
# hash, salt, free queue
# ---------------------------------------------------------------------------
def pin_chain_property(o):
    """Digest j is equal for two token lists exactly when their first (j+1)
    blocks are equal; a block equal in content after a different block does
    not match.  The byte encoding is rebuilt here with NumPy."""
    B = 4
    rng = np.random.default_rng(13)
    base = _prompt(rng, 24)
    for cut in range(24):
        other = list(base)
        other[cut] += 1
        a, b = o.chain_digests(base, B), o.chain_digests(other, B)
        for j in range(6):
            assert (a[j] == b[j]) == ((j + 1) * B <= cut)
    d0 = hashlib.sha256(hashlib.sha256(b"").digest()
                        + np.asarray(base[:B], dtype="<i4").tobytes()).digest()
    d1 = hashlib.sha256(d0 + np.asarray(base[B:2 * B], dtype="<i4").tobytes()).digest()
    assert o.chain_digests(base, B)[:2] == [d0, d1]
    assert len(o.chain_digests(base[:7], B)) == 1
    # identical second block, different first block: no hit on either
    m = o.BlockManagerRef(16, B)
    m.allocate(0, [1, 2, 3, 4, 5, 6, 7, 8, 9])
    assert m.allocate(1, [0, 2, 3, 4, 5, 6, 7, 8, 9]) == 0


def pin_salt_isolation(o):
    """A salt limits sharing to requests with the same salt."""
    B = 4
    prompt = list(range(13))
    m = o.BlockManagerRef(32, B)
    assert m.allocate(0, prompt, b"tenant-a") == 0
    assert m.allocate(1, prompt, b"tenant-b") == 0
    assert m.allocate(2, prompt) == 0
    assert m.allocate(3, prompt, b"tenant-a") == 12
    assert m.allocate(4, prompt) == 12
    assert o.salt_digest(b"") == hashlib.sha256(b"").digest()


def pin_free_queue_order(o):
    """Allocation takes the least recently used free block: never-used blocks
    in id order first, then released blocks in release order, a request's
    last block first.  A released block keeps its hash until it is taken."""
    B = 2
    m = o.BlockManagerRef(8, B)
    m.allocate(0, [1, 2, 3, 4, 5])        # blocks 0 1 2, hashes on 0 and 1
    m.allocate(1, [9, 9, 9])              # blocks 3 4, hash on 3
    assert m.block_table(0) == [0, 1, 2] and m.block_table(1) == [3, 4]
    m.free_seq(0)                         # queue: 5 6 7 2 1 0
    m.free_seq(1)                         # queue: 5 6 7 2 1 0 4 3
    assert m.free == [5, 6, 7, 2, 1, 0, 4, 3]
    # a hit still finds the released blocks
    assert m.allocate(2, [1, 2, 3, 4, 6]) == 4
    assert m.block_table(2) == [0, 1, 5]
    m.free_seq(2)                         # releases 5, 1, 0 onto the tail
    assert m.free == [6, 7, 2, 4, 3, 5, 1, 0]
    # new tokens take the head; taking block 3 evicts its hash
    m.allocate(3, [7] * 10)
    assert m.block_table(3) == [6, 7, 2, 4, 3]
    assert m.allocate(4, [9, 9, 9]) == 0
    assert m.block_table(4) == [5, 1]


def pin_out_of_blocks(o):
    """An operation that needs more free blocks than exist fails and leaves
    the state as it was."""
    B = 4
    m = o.BlockManagerRef(6, B)
    m.allocate(0, list(range(10)))        # 3 blocks
    m.fork(0, 1)
    m.allocate(2, list(range(100, 111)))  # 3 blocks, queue empty
    m.append(2, 1)                        # the 12th token fits the private last block
    assert m.num_tokens(2) == 12 and m.num_free() == 0
    before = copy.deepcopy(m.__dict__)
    # a new prompt, a write into a shared partial block, a token that starts a block
    for op in (lambda: m.allocate(3, [1]), lambda: m.append(0, 5), lambda: m.append(2, 5)):
        try:
            op()
        except o.OutOfBlocks:
            pass
        else:
            raise AssertionError("operation without free blocks succeeded")
        assert m.__dict__ == before
    m.allocate(3, [])                     # an empty prompt holds no block
    assert m.block_table(3) == []


def pin_growth_copies_nothing(o):
    """Growing a sequence only takes free blocks; with prefix caching and no
    forks no block is ever copied (only full blocks are shared)."""
    rng = np.random.default_rng(14)
    m = o.BlockManagerRef(2000, 4)
    cm = ContentModel(m)
    sys_prompt = _prompt(rng, 9)
    live = []
    for step in range(300):
        r = rng.random()
        if r < 0.25 or not live:
            seq = step
            cm.allocate(seq, sys_prompt[:int(rng.integers(0, 10))] + _prompt(rng, int(rng.integers(0, 7))))
            live.append(seq)
        elif r < 0.9:
            seq = live[int(rng.integers(len(live)))]
            _, cow = cm.append(seq, int(rng.integers(50)))
            assert cow is None
        else:
            cm.free(live.pop(int(rng.integers(len(live)))))
        cm.check(o)


def pin_random_operations(o):
    """Random allocate / append / fork / free on small pools, with shared
    prompt prefixes and salts: after every step each sequence reads back its
    own tokens, hits land on blocks that hold the hit tokens, and counts,
    queue and digests agree with brute force.  Failed operations change
    nothing."""
    for seed, (nb, B, caching) in enumerate([(24, 4, True), (40, 2, True), (30, 4, False),
                                              (64, 8, True)]):
        rng = np.random.default_rng(100 + seed)
        m = o.BlockManagerRef(nb, B, prefix_caching=caching)
        cm = ContentModel(m)
        bases = [_prompt(rng, 3 * B + 1) for _ in range(3)]
        salts = [b"", b"", b"x"]
        live, next_id, cows = [], 0, 0
        for step in range(400):
            r = rng.random()
            before = copy.deepcopy(m.__dict__)
            try:
                if r < 0.2 or not live:
                    base = bases[int(rng.integers(3))]
                    prompt = base[:int(rng.integers(0, len(base) + 1))] + _prompt(rng, int(rng.integers(0, B + 2)))
                    cm.allocate(next_id, prompt, salts[int(rng.integers(3))])
                    live.append(next_id)
                    next_id += 1
                elif r < 0.75:
                    _, cow = cm.append(live[int(rng.integers(len(live)))], int(rng.integers(50)))
                    cows += cow is not None
                elif r < 0.87:
                    cm.fork(live[int(rng.integers(len(live)))], next_id)
                    live.append(next_id)
                    next_id += 1
                else:
                    cm.free(live.pop(int(rng.integers(len(live)))))
            except o.OutOfBlocks:
                assert m.__dict__ == before
                if live:
                    cm.free(live.pop(0))
            cm.check(o)
        assert cows > 0


# ---------------------------------------------------------------------------
# the block copy
# ---------------------------------------------------------------------------
def pin_copy_blocks(o):
    """copy_blocks against element loops; untouched blocks stay as they were;
    a sequence read through a copied block decodes exactly as through the
    original, and writing into the copy leaves the original's readers alone."""
    import oracle.paged_attention_ref as ref
    rng = np.random.default_rng(15)
    NB, Hkv, B, D = 9, 2, 4, 8
    k = rng.standard_normal((NB, Hkv, B, D)).astype(np.float32)
    v = rng.standard_normal((NB, Hkv, B, D)).astype(np.float32)
    (k4,) = o.copy_blocks([k], [(2, 6)])
    assert np.array_equal(k4[6], k[2]) and np.array_equal(k4[2], k[2])
    assert np.array_equal(np.delete(k4, 6, axis=0), np.delete(k, 6, axis=0))
    pairs = [(1, 7), (4, 0), (1, 5)]
    k2, v2 = o.copy_blocks([k, v], pairs)
    for pool, new in ((k, k2), (v, v2)):
        for b in range(NB):
            src = {d: s for s, d in pairs}.get(b, b)
            for h in range(Hkv):
                for r in range(B):
                    for x in range(D):
                        assert new[b, h, r, x] == pool[src, h, r, x]
    for bad in ([(1, 2), (3, 2)], [(1, 2), (2, 3)], [(0, NB)]):
        try:
            o.copy_blocks([k], bad)
        except ValueError:
            continue
        raise AssertionError(f"copy_blocks accepted {bad}")
    # decode through the copy equals decode through the original
    q = rng.standard_normal((2, 4, D)).astype(np.float32)
    tab = np.array([[2, 1, 3], [2, 7, 3]], np.int32)
    lens = np.array([10, 10], np.int32)
    out = ref.decode(q[[0, 0]], k2, v2, tab, lens, 0.3, "f32")
    assert np.array_equal(out[0], out[1])
    # copy-on-write: the second reader appends position 6 (block 7, offset 2)
    new_k = rng.standard_normal((1, Hkv, D)).astype(np.float32)
    k3, v3 = ref.write_kv(k2, v2, new_k, -new_k, np.array([7 * B + 2]), B)
    lens = np.array([6, 7], np.int32)
    a = ref.decode(q[[0, 0]], k2, v2, tab, np.array([6, 6], np.int32), 0.3, "f32")
    b = ref.decode(q[[0, 0]], k3, v3, tab, lens, 0.3, "f32")
    assert np.array_equal(a[0], b[0]) and not np.array_equal(a[1], b[1])
    assert np.array_equal(k3[1], k[1]) and np.array_equal(v3[1], v[1])


ALL_BM_PINS = [
    pin_prefix_caching_example,
    pin_fragmentation_example,
    pin_shared_prefix_twelve,
    pin_chain_property,
    pin_salt_isolation,
    pin_free_queue_order,
    pin_out_of_blocks,
    pin_growth_copies_nothing,
    pin_random_operations,
    pin_copy_blocks,
]
