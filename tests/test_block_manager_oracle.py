"""The block-manager oracle against the pages' worked examples and brute
force, and planted mistakes that the pins must catch (no GPU)."""
import pytest

import oracle.block_manager_ref as bm
from block_manager_pins import ALL_BM_PINS


@pytest.mark.parametrize("pin", ALL_BM_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(bm)


def _release_to_head(self, b):
    self.ref[b] -= 1
    if self.ref[b] == 0:
        self.free.insert(0, b)


def _free_forward(self, seq):
    s = self.seqs.pop(seq)
    for b in s["blocks"]:
        self._release(b)


def _take_keeps_hash(self):
    b = self.free.pop(0)
    self.ref[b] = 1
    return b


def _append_in_place(self, seq, token):
    s = self.seqs[seq]
    t = len(s["tokens"])
    if t % self.block_size == 0:
        if not self.free:
            raise bm.OutOfBlocks("no block")
        s["blocks"].append(self._take_free())
    s["tokens"].append(int(token))
    b = s["blocks"][t // self.block_size]
    if self.prefix_caching and (t + 1) % self.block_size == 0:
        self._register(b, bm.chain_digests(s["tokens"], self.block_size, s["salt"])[-1])
    return b * self.block_size + t % self.block_size, None


def _fork_no_ref(self, parent, child):
    p = self.seqs[parent]
    self.seqs[child] = {"tokens": list(p["tokens"]), "blocks": list(p["blocks"]),
                        "salt": p["salt"]}


def _chain_unchained(tokens, block_size, salt=b""):
    parent = bm.salt_digest(salt)
    return [bm.block_digest(parent, tokens[j * block_size:(j + 1) * block_size])
            for j in range(len(tokens) // block_size)]


def _chain_no_salt(tokens, block_size, salt=b""):
    return _ORIG["chain"](tokens, block_size, b"")


def _copy_reversed(pools, pairs, inplace=False):
    return _ORIG["copy"](pools, [(d, s) for s, d in pairs], inplace)


def _allocate_no_cap(self, seq, prompt, salt=b""):
    # the match may take every full block, leaving nothing to compute
    prompt = [int(t) for t in prompt]
    digests = bm.chain_digests(prompt, self.block_size, salt)
    hits = []
    for d in digests:
        b = self.cached.get(d)
        if b is None:
            break
        hits.append(b)
    for b in hits:
        if self.ref[b] == 0:
            self.free.remove(b)
        self.ref[b] += 1
    blocks = list(hits)
    for j in range(len(hits), -(-len(prompt) // self.block_size)):
        b = self._take_free()
        blocks.append(b)
        if j < len(digests):
            self._register(b, digests[j])
    self.seqs[seq] = {"tokens": prompt, "blocks": blocks, "salt": bytes(salt)}
    return len(hits) * self.block_size


def _copy_next_block(pools, pairs, inplace=False):
    return _ORIG["copy"](pools, [(s + 1, d) for s, d in pairs], inplace)


_ORIG = {"chain": bm.chain_digests, "copy": bm.copy_blocks}

MUTANTS = {
    "free block joins the head (MRU reuse)": ("BlockManagerRef", "_release", _release_to_head),
    "request released first block first": ("BlockManagerRef", "free_seq", _free_forward),
    "eviction keeps the hash": ("BlockManagerRef", "_take_free", _take_keeps_hash),
    "no copy-on-write": ("BlockManagerRef", "append", _append_in_place),
    "fork without references": ("BlockManagerRef", "fork", _fork_no_ref),
    "hash not chained": (None, "chain_digests", _chain_unchained),
    "salt ignored": (None, "chain_digests", _chain_no_salt),
    "copy direction swapped": (None, "copy_blocks", _copy_reversed),
    "copy reads the next block": (None, "copy_blocks", _copy_next_block),
    "prefix match takes the whole prompt": ("BlockManagerRef", "allocate", _allocate_no_cap),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_caught(name, monkeypatch):
    owner, attr, fn = MUTANTS[name]
    target = getattr(bm, owner) if owner else bm
    monkeypatch.setattr(target, attr, fn)
    failed = []
    for pin in ALL_BM_PINS:
        try:
            pin(bm)
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake: {name}"
