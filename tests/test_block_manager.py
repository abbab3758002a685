"""The library's native block manager (pa_bm_* through the C ABI) against the
block-manager oracle, in lockstep: every operation is applied to both and
the whole visible state is compared after each one (return values, block
tables, token counts, reference counts, digests, which block holds a
registered digest, and the free queue in order).  Host code only: no GPU."""
import copy
import hashlib
import os

import numpy as np
import pytest

import oracle.block_manager_ref as bm
from paged_kv_cache_75_amd import binding as B

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="libpa.so not built")


class Lockstep:
    def __init__(self, num_blocks, block_size, caching=True):
        self.ref = bm.BlockManagerRef(num_blocks, block_size, prefix_caching=caching)
        self.lib = B.BlockManager(num_blocks, block_size, prefix_caching=caching)

    def check(self):
        r, n = self.ref, self.lib
        assert n.num_free() == r.num_free()
        assert n.free_queue() == r.free
        for seq in r.seqs:
            assert n.block_table(seq) == r.block_table(seq)
            assert n.num_tokens(seq) == r.num_tokens(seq)
        for b in range(r.num_blocks):
            ref_count, digest, registered = n.block_info(b)
            assert ref_count == r.ref[b]
            assert digest == r.digest[b]
            assert registered == (r.digest[b] is not None and r.cached.get(r.digest[b]) == b)
        if r.seqs:
            ids = sorted(r.seqs)
            width = max(len(r.block_table(s)) for s in ids) + 2
            got = n.tables(ids, width)
            want = r.tables(ids, width)
            assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])

    def allocate(self, seq, prompt, salt=b""):
        try:
            want = self.ref.allocate(seq, prompt, salt)
        except bm.OutOfBlocks:
            with pytest.raises(B.OutOfBlocks):
                self.lib.allocate(seq, prompt, salt)
            return None
        assert self.lib.allocate(seq, prompt, salt) == want
        return want

    def append(self, seqs, tokens):
        """A batch on the library; the same appends one by one on the oracle
        (all of them, or none when the oracle runs out part way)."""
        trial = copy.deepcopy(self.ref)
        try:
            res = [trial.append(s, t) for s, t in zip(seqs, tokens)]
        except bm.OutOfBlocks:
            with pytest.raises(B.OutOfBlocks):
                self.lib.append(seqs, tokens)
            return None
        self.ref = trial
        slots, pairs = self.lib.append(seqs, tokens)
        assert slots.tolist() == [s for s, _ in res]
        assert [tuple(p) for p in pairs.tolist()] == [c for _, c in res if c is not None]
        return slots, pairs

    def fork(self, parent, child):
        self.ref.fork(parent, child)
        self.lib.fork(parent, child)

    def free(self, seq):
        self.ref.free_seq(seq)
        self.lib.free_seq(seq)


def test_sha256_matches_hashlib():
    rng = np.random.default_rng(0)
    for n in list(range(0, 130)) + [1000, 4096, 65537]:
        data = rng.integers(0, 256, n, dtype=np.uint8).tobytes()
        assert B.pa_sha256(data) == hashlib.sha256(data).digest()


def test_block_digest_matches_oracle():
    m = B.BlockManager(8, 4)
    toks = [5, -1, 2**31 - 1, -2**31, 7, 8, 9, 10, 11]
    m.allocate(0, toks, b"salt")
    chain = bm.chain_digests(toks, 4, b"salt")
    table = m.block_table(0)
    assert [m.block_info(b)[1] for b in table[:2]] == chain
    assert m.block_info(table[2])[1] is None


def test_pages_worked_examples_lockstep():
    # three prompts after one system prompt: 0, 10 and 10 blocks matched
    rng = np.random.default_rng(1)
    L = Lockstep(64, 16)
    system = [int(x) for x in rng.integers(0, 30000, 165)]
    for i, n in enumerate((183, 182, 177)):
        q = [30000 + 1000 * i + int(x) for x in rng.integers(0, 1000, n - 165)]
        assert L.allocate(i, system + q) == (0, 160, 160)[i]
        L.check()
    # twelve requests on an 1,800-token prefix, shared by fork: 11 copies
    L = Lockstep(200, 16)
    L.allocate(0, list(range(1800)))
    for c in range(1, 12):
        L.fork(0, c)
    L.check()
    _, pairs = L.append(list(range(12)), [7] * 12)
    assert len(pairs) == 11
    L.check()


@pytest.mark.parametrize("cfg", [(24, 4, True), (40, 2, True), (30, 4, False), (64, 8, True),
                                 (12, 1, True)])
def test_random_operations_lockstep(cfg):
    nb, bs, caching = cfg
    rng = np.random.default_rng(nb * 100 + bs)
    L = Lockstep(nb, bs, caching)
    bases = [[int(x) for x in rng.integers(0, 50, 3 * bs + 1)] for _ in range(3)]
    salts = [b"", b"", b"tenant"]
    live, next_id = [], 0
    for step in range(500):
        r = rng.random()
        if r < 0.2 or not live:
            base = bases[int(rng.integers(3))]
            prompt = base[:int(rng.integers(0, len(base) + 1))] + \
                [int(x) for x in rng.integers(0, 50, int(rng.integers(0, bs + 2)))]
            if L.allocate(next_id, prompt, salts[int(rng.integers(3))]) is not None:
                live.append(next_id)
            next_id += 1
        elif r < 0.75:
            k = int(rng.integers(1, 4))
            seqs = [live[int(i)] for i in rng.integers(0, len(live), k)]   # repeats allowed
            if L.append(seqs, [int(x) for x in rng.integers(0, 50, k)]) is None and live:
                L.free(live.pop(0))
        elif r < 0.87:
            L.fork(live[int(rng.integers(len(live)))], next_id)
            live.append(next_id)
            next_id += 1
        else:
            L.free(live.pop(int(rng.integers(len(live)))))
        L.check()


def test_batch_append_is_all_or_nothing():
    L = Lockstep(6, 4)
    L.allocate(0, list(range(10)))      # 3 blocks
    L.fork(0, 1)
    L.allocate(2, list(range(100, 108)))  # 2 blocks, 1 free left
    L.check()
    # seq 0 needs a copy-on-write block, seq 2 a new block: 2 > 1 free
    assert L.append([0, 2], [1, 2]) is None
    L.check()
    # seq 0 copies (1 block); then seq 1 owns the original: no second copy
    slots, pairs = L.append([0, 1], [1, 2])
    assert len(pairs) == 1
    L.check()


def test_errors_change_nothing():
    L = Lockstep(8, 4)
    L.allocate(0, [1, 2, 3, 4, 5])
    L.check()
    n = L.lib
    for call in (lambda: n.allocate(0, [1]),          # live id
                 lambda: n.append([9], [1]),          # unknown id
                 lambda: n.append([0, 9], [1, 2]),    # unknown id after a known one
                 lambda: n.fork(9, 10),
                 lambda: n.fork(0, 0),
                 lambda: n.free_seq(9),
                 lambda: n.tables([0], 1)):           # row too short for 2 blocks
        with pytest.raises(B.PaError) as e:
            call()
        assert e.value.status == B.PA_ERR_INVALID_ARGUMENT
        L.check()
    with pytest.raises(B.PaError):
        B.BlockManager(-1, 4)
    with pytest.raises(B.PaError):
        B.BlockManager(4, 0)
    L2 = B.lib()
    assert L2.pa_bm_num_free(None) == -1
    assert L2.pa_bm_free(None, 0) == B.PA_ERR_INVALID_ARGUMENT
    assert L2.pa_bm_block_info(n._h, 8, None, None, None, None) == B.PA_ERR_INVALID_ARGUMENT


def test_empty_pool_and_empty_prompt():
    L = Lockstep(0, 16)
    assert L.allocate(0, []) == 0
    assert L.allocate(1, [1]) is None
    assert L.append([0], [3]) is None
    L.check()
