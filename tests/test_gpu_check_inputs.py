"""pa_check_inputs on the GPU against the contract written out on the host:
the slots must be below num_blocks * B and distinct, the lengths within
[0, max_context_len], and the table entries a sequence's clamped length
reaches inside the pool.  The expected report is computed here by plain
loops over the same arrays."""
import collections

import numpy as np
import pytest

import workloads
from gpu_util import say, to_device

pytestmark = pytest.mark.gpu

DEV = "cuda"


def expected(slots, tables, lens, nb, bs, max_len, duplicates=True):
    found = []                                   # (kind, index, value)
    if slots is not None:
        live = collections.Counter(int(s) for s in slots if 0 <= s < nb * bs)
        for n, s in enumerate(int(x) for x in slots):
            if s < 0:
                continue
            if s >= nb * bs:
                found.append((1, n, s))
            elif duplicates and live[s] > 1:
                found.append((2, n, s))
    if tables is not None:
        mb = tables.shape[1]
        for i, T in enumerate(int(x) for x in lens):
            if T < 0 or T > max_len:
                found.append((3, i, T))
            tc = min(max(T, 0), max_len)
            for j in range(min(mb, -(-tc // bs))):
                e = int(tables[i, j])
                if e < 0 or e >= nb:
                    found.append((4, i * mb + j, e))
    if not found:
        return (0, 0, 0, 0)
    return (len(found),) + min(found, key=lambda f: (f[0], f[1]))


def _run(w, slots, tables, lens, duplicates=True, pool_shape=None):
    import torch
    from paged_kv_cache_75_amd import pa_check_inputs
    shape = pool_shape or (w.k_pool.shape[0], w.num_kv_heads, w.block_size, w.head_dim)
    k_pool = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
    got = pa_check_inputs(
        k_pool,
        slot_mapping=None if slots is None else to_device(np.asarray(slots, np.int32), None, DEV),
        block_tables=None if tables is None else to_device(tables.astype(np.int32), None, DEV),
        context_lens=None if lens is None else to_device(np.asarray(lens, np.int32), None, DEV),
        max_context_len=w.max_context_len, duplicates=duplicates)
    want = expected(slots, tables, lens, shape[0], shape[2], w.max_context_len, duplicates)
    say(f"  report {got}, expected {want}")
    assert got == want


@pytest.fixture(scope="module")
def batch():
    return workloads.make(3, seed=4500, poison=False)


def test_valid_batch_reports_nothing(batch):
    w = batch
    _run(w, w.slot_mapping, w.block_tables, w.context_lens)


def test_each_kind(batch):
    w = batch
    nb = w.k_pool.shape[0]
    slots = w.slot_mapping.astype(np.int64).copy()
    slots[7] = nb * w.block_size + 5
    _run(w, slots, None, None)                                   # slot past the pool
    slots = w.slot_mapping.astype(np.int64).copy()
    slots[10] = slots[3]
    _run(w, slots, None, None)                                   # two tokens, one slot
    lens = w.context_lens.astype(np.int64).copy()
    lens[4] = -3
    _run(w, None, w.block_tables, lens)                          # negative length
    lens[2] = w.max_context_len + 1
    _run(w, None, w.block_tables, lens)                          # length past the bound
    tables = w.block_tables.copy()
    i = int(np.argmax(w.context_lens))
    tables[i, 2] = -5
    tables[3, 0] = nb + 3
    _run(w, None, tables, w.context_lens)                        # entries outside the pool
    tables = w.block_tables.copy()
    T = int(w.context_lens[0])
    tables[0, -(-T // w.block_size):] = -7                       # past ceil(T / B): not read
    _run(w, None, tables, w.context_lens)


def test_mixed_violations_and_no_duplicate_test(batch):
    w = batch
    nb = w.k_pool.shape[0]
    slots = w.slot_mapping.astype(np.int64).copy()
    slots[[3, 10, 20]] = slots[3]
    slots[50] = nb * w.block_size
    lens = w.context_lens.astype(np.int64).copy()
    lens[9] = w.max_context_len + 7
    tables = w.block_tables.copy()
    tables[5, 0] = -1
    _run(w, slots, tables, lens)
    _run(w, slots, tables, lens, duplicates=False)


def test_many_workgroups_count_exactly(batch):
    """200,000 tokens over a 320,000-slot pool (many workgroups): 50,000 share
    one slot, 1,000 point past the pool, 5,000 are skipped, the rest are
    distinct; every violation is counted."""
    w = batch
    nb, bs = 20_000, 16
    rng = np.random.default_rng(4501)
    n = 200_000
    slots = rng.permutation(nb * bs)[:n].astype(np.int64)
    slots[rng.choice(n, 50_000, replace=False)] = 77
    slots[rng.choice(n, 1_000, replace=False)] = nb * bs + 3
    slots[rng.choice(n, 5_000, replace=False)] = -1
    _run(w, slots, None, None, pool_shape=(nb, 1, bs, 64))
