"""Pools larger than 4 GiB: every byte offset the kernels form from a block
id must be 64-bit.  A small decode batch is placed at the top of two 4.6 GB
pools (140,000 blocks of 32 KiB); the slot write, the one-call decode step
and a block copy there are compared with the oracle on the same batch in a
compact pool (block relabelling does not change the result)."""
import numpy as np
import pytest

import workloads
from gpu_util import compare, oracle_step, say, to_device, to_f64, to_host

pytestmark = pytest.mark.gpu

DEV = "cuda"
NB_BIG = 140_000                # x 8 heads x 16 rows x 128 x 2 bytes = 4.59 GB per pool


def _bytes(a):
    return np.ascontiguousarray(a).view(np.uint8)


def test_pools_beyond_4gib():
    import torch
    from paged_kv_cache_75_amd import pa_append_decode, pa_copy_blocks
    say("[big pools] generate")
    w = workloads.random_paged("big-pool", "bf16", 32, 8, 128, 16, [1, 40, 300, 17, 1000, 129],
                               seed=4400)
    nb = w.k_pool.shape[0]
    # compact block j lives at block NB_BIG - 1 - j of the big pools
    high = (NB_BIG - 1 - np.arange(nb)).astype(np.int64)
    tables = np.where(w.block_tables >= 0, high[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    assert int(high[-1]) * 16 * 8 * 128 * 2 > (1 << 32)
    say(f"[big pools] allocate 2 x {NB_BIG} blocks")
    k_big = torch.empty((NB_BIG, 8, 16, 128), dtype=torch.bfloat16, device=DEV)
    v_big = torch.empty_like(k_big)
    idx = torch.from_numpy(high).to(DEV)
    k_big[idx] = to_device(w.k_pool, "bf16", DEV)
    v_big[idx] = to_device(w.v_pool, "bf16", DEV)
    q = to_device(w.q, "bf16", DEV)
    say("[big pools] pa_append_decode")
    out = pa_append_decode(q, to_device(w.new_k, "bf16", DEV), to_device(w.new_v, "bf16", DEV),
                           k_big, v_big, to_device(tables, None, DEV),
                           to_device(w.context_lens.astype(np.int32), None, DEV), w.scale,
                           max_context_len=w.max_context_len)
    torch.cuda.synchronize()
    want, k_ref, v_ref = oracle_step(w)
    compare(to_f64(out), want, "bf16", label="decode at the top of 4.6 GB pools")
    assert np.array_equal(_bytes(to_host(k_big[idx], "bf16")), _bytes(k_ref))
    assert np.array_equal(_bytes(to_host(v_big[idx], "bf16")), _bytes(v_ref))
    say("[big pools] pa_copy_blocks between blocks above 4 GiB")
    live = sorted({int(b) for b in w.block_tables.ravel() if b >= 0})[:4]
    pairs = [(int(high[j]), int(high[-1]) - 1000 - i) for i, j in enumerate(live)]
    pa_copy_blocks([k_big, v_big], torch.tensor(pairs, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    # destination = source bit for bit (the oracle's block copy; unused rows
    # hold NaN, so bits are compared), and source = the oracle's written block
    bits = lambda t: t.view(torch.int16)
    for (src, dst), j in zip(pairs, live):
        assert torch.equal(bits(k_big[dst]), bits(k_big[src]))
        assert torch.equal(bits(v_big[dst]), bits(v_big[src]))
        assert np.array_equal(_bytes(to_host(k_big[dst], "bf16")), _bytes(k_ref[j]))
