"""Checks that tie the CPU oracle to something other than itself.

Each ``pin_*`` function takes the oracle module and raises AssertionError (or
any exception) when the oracle disagrees with what the pages or mathematics
fix.  tests/test_oracle_pins.py runs them on the real oracle;
tests/test_oracle_mutants.py plants mistakes in the oracle and checks that at
least one pin fails for each.

Sources of truth used here, none of which is the oracle's own code:

* brute force over a contiguous (unpaged) copy of the same tokens, with plain
  Python loops and ``math.exp``;
* a torch float64 rendering of the paged-attention sketch on "vLLM Framework
  and Inference Engine Design", section "What is the essence of vLLM's
  PagedAttention?" (token-major pool view, gather by block table, softmax);
* invariances: relabelling physical blocks, sharing versus copying prefix
  blocks;
* closed forms: one token, zero query or zero scale, equal keys, a hard
  maximum, empty context;
* known bit patterns of bfloat16 and float16;
* the numbers the pages print (tests/golden/page_figures.json).
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def load_golden():
    with open(os.path.join(HERE, "golden", "page_figures.json")) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# small hand-built paged problem (independent of the workload generator)
# ---------------------------------------------------------------------------
def _tiny_problem(seed, lens, Hq, Hkv, D, B, spare=3):
    """Contiguous per-sequence K/V plus the same tokens placed into a shuffled
    paged pool by explicit loops (slot of token t: table[t // B], offset t % B)."""
    rng = np.random.default_rng(seed)
    need = [-(-T // B) for T in lens]
    NB = sum(need) + spare
    perm = rng.permutation(NB)
    MB = max(need + [1]) + 1
    tables = np.full((len(lens), MB), -1, dtype=np.int64)
    at = 0
    for i, n in enumerate(need):
        tables[i, :n] = perm[at:at + n]
        at += n
    q = rng.standard_normal((len(lens), Hq, D)).astype(np.float32)
    k_pool = np.full((NB, Hkv, B, D), np.nan, dtype=np.float32)
    v_pool = np.full((NB, Hkv, B, D), np.nan, dtype=np.float32)
    contig_k, contig_v = [], []
    for i, T in enumerate(lens):
        kc = rng.standard_normal((T, Hkv, D)).astype(np.float32)
        vc = rng.standard_normal((T, Hkv, D)).astype(np.float32)
        contig_k.append(kc)
        contig_v.append(vc)
        for t in range(T):
            blk = tables[i, t // B]
            off = t % B
            for g in range(Hkv):
                k_pool[blk, g, off, :] = kc[t, g]
                v_pool[blk, g, off, :] = vc[t, g]
    return q, k_pool, v_pool, tables, np.array(lens), contig_k, contig_v


def _brute(qv, kc, vc, scale, G):
    """Pure-Python softmax attention for every query head, contiguous K/V."""
    Hq, D = len(qv), len(qv[0])
    T = len(kc)
    out = [[0.0] * D for _ in range(Hq)]
    if T == 0:
        return out
    for h in range(Hq):
        g = h // G
        s = [scale * sum(float(qv[h][d]) * float(kc[t][g][d]) for d in range(D))
             for t in range(T)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = sum(w)
        for d in range(D):
            out[h][d] = sum(w[t] * float(vc[t][g][d]) for t in range(T)) / z
    return out


def pin_contiguous_bruteforce(o):
    cases = [
        dict(seed=11, lens=[1, 5, 11, 16, 17], Hq=4, Hkv=2, D=8, B=4),
        dict(seed=12, lens=[3, 8, 2], Hq=3, Hkv=3, D=6, B=2),
        dict(seed=13, lens=[33, 7], Hq=8, Hkv=1, D=4, B=8),
    ]
    for c in cases:
        q, kp, vp, bt, lens, ck, cv = _tiny_problem(c["seed"], c["lens"], c["Hq"], c["Hkv"], c["D"], c["B"])
        scale = float(np.float32(0.37))
        got = o.decode(q, kp, vp, bt, lens, scale, "f32")
        G = c["Hq"] // c["Hkv"]
        for i in range(len(lens)):
            ref = np.array(_brute(q[i].tolist(), ck[i].tolist(), cv[i].tolist(), scale, G))
            np.testing.assert_allclose(got[i], ref, rtol=1e-12, atol=1e-13)


def pin_page_sketch_torch(o):
    """The pages' sketch in torch float64: view the pool token-major, gather the
    first ceil(T/B) blocks of the table, keep T rows, softmax over scores."""
    import torch
    cases = [
        dict(seed=21, lens=[9, 4, 13], Hq=4, Hkv=4, D=16, B=4),     # MHA, as on the page
        dict(seed=22, lens=[17, 32, 1], Hq=6, Hkv=2, D=8, B=16),    # GQA by kv-head expansion
    ]
    for c in cases:
        q, kp, vp, bt, lens, _, _ = _tiny_problem(c["seed"], c["lens"], c["Hq"], c["Hkv"], c["D"], c["B"])
        scale = float(np.float32(1.0 / math.sqrt(c["D"])))
        got = o.decode(q, kp, vp, bt, lens, scale, "f32")
        G = c["Hq"] // c["Hkv"]
        ktm = torch.from_numpy(kp).double().permute(0, 2, 1, 3)      # [NB][B][Hkv][D]
        vtm = torch.from_numpy(vp).double().permute(0, 2, 1, 3)
        for i, T in enumerate(lens):
            nb = -(-int(T) // c["B"])
            ids = torch.from_numpy(bt[i, :nb].astype(np.int64))
            keys = torch.index_select(ktm, 0, ids).reshape(nb * c["B"], c["Hkv"], c["D"])[:T]
            vals = torch.index_select(vtm, 0, ids).reshape(nb * c["B"], c["Hkv"], c["D"])[:T]
            keys = keys.repeat_interleave(G, dim=1).permute(1, 0, 2)  # [Hq][T][D]
            vals = vals.repeat_interleave(G, dim=1).permute(1, 0, 2)
            qi = torch.from_numpy(q[i]).double().unsqueeze(-1)        # [Hq][D][1]
            scores = torch.bmm(keys, qi).squeeze(-1) * scale          # [Hq][T]
            probs = torch.softmax(scores, dim=-1)
            ref = torch.bmm(probs.unsqueeze(1), vals).squeeze(1).numpy()
            np.testing.assert_allclose(got[i], ref, rtol=1e-12, atol=1e-13)


def pin_placement_invariance(o, w=None):
    import workloads
    w = w or workloads.make(1)
    rng = np.random.default_rng(99)
    perm = rng.permutation(w.num_blocks)
    w2 = workloads.relabel_blocks(w, perm)
    a = _decode_after_write(o, w)
    b = _decode_after_write(o, w2)
    assert np.array_equal(a, b), "relabelling physical blocks changed the oracle output"


def _decode_after_write(o, w):
    k, v = o.write_kv(w.k_pool, w.v_pool, w.new_k, w.new_v, w.slot_mapping, w.block_size)
    return o.decode(w.q, k, v, w.block_tables, w.context_lens, w.scale, w.dtype)


def pin_prefix_sharing(o):
    import workloads
    kw = dict(num_seqs=4, prefix_len=40, max_suffix=20)
    shared = workloads.prefix_shared(seed=5, **kw)
    private = workloads.prefix_shared(seed=5, share=False, **kw)
    assert shared.refcount.max() == 4 and private.refcount.max() == 1
    a = _decode_after_write(o, shared)
    b = _decode_after_write(o, private)
    assert np.array_equal(a, b), "shared prefix blocks and private copies disagree"
    assert np.isfinite(a).all()


def pin_closed_forms(o):
    rng = np.random.default_rng(31)
    Hkv, D, B = 2, 8, 4
    # T = 1: the output is the single value row, exactly
    kp = rng.standard_normal((3, Hkv, B, D)).astype(np.float32)
    vp = rng.standard_normal((3, Hkv, B, D)).astype(np.float32)
    q = rng.standard_normal((1, 4, D)).astype(np.float32)
    bt = np.array([[2, -1]])
    out = o.decode(q, kp, vp, bt, np.array([1]), 0.5, "f32")
    for h in range(4):
        assert np.array_equal(out[0, h], vp[2, h // 2, 0].astype(np.float64))
    # q = 0 (and scale = 0): uniform weights, the mean of V over t < T
    T = 7
    bt = np.array([[1, 0]])
    for qq, sc in ((np.zeros((1, 4, D), np.float32), 0.3), (q, 0.0)):
        out = o.decode(qq, kp, vp, bt, np.array([T]), sc, "f32")
        for h in range(4):
            rows = [vp[bt[0, t // B], h // 2, t % B] for t in range(T)]
            np.testing.assert_allclose(out[0, h], np.mean(np.array(rows, np.float64), axis=0), rtol=0, atol=1e-14)
    # equal keys: uniform weights whatever q is
    ke = kp.copy()
    ke[:, :, :, :] = kp[0, 0, 0]
    out = o.decode(q, ke, vp, bt, np.array([T]), 0.9, "f32")
    for h in range(4):
        rows = [vp[bt[0, t // B], h // 2, t % B] for t in range(T)]
        np.testing.assert_allclose(out[0, h], np.mean(np.array(rows, np.float64), axis=0), rtol=0, atol=1e-14)
    # empty context: zeros
    out = o.decode(q, kp, vp, np.array([[-1, -1]]), np.array([0]), 0.5, "f32")
    assert np.array_equal(out, np.zeros_like(out))


def pin_hard_max(o):
    """One key aligned with q and a scale so large that every other weight
    underflows to zero: the output is that token's value row, bit for bit."""
    rng = np.random.default_rng(41)
    Hq, Hkv, D, B, T = 2, 1, 8, 4, 10
    kp = rng.standard_normal((4, Hkv, B, D)).astype(np.float32) * 0.01
    vp = rng.standard_normal((4, Hkv, B, D)).astype(np.float32)
    bt = np.array([[3, 1, 0]])
    q = np.zeros((1, Hq, D), np.float32)
    q[0, :, 0] = 1.0
    for star in (0, 5, 9):
        k2 = kp.copy()
        k2[bt[0, star // B], 0, star % B, 0] = 4.0
        out = o.decode(q, k2, vp, bt, np.array([T]), 1000.0, "f32")
        want = vp[bt[0, star // B], 0, star % B].astype(np.float64)
        for h in range(Hq):
            assert np.array_equal(out[0, h], want), f"hard max at token {star}"


def pin_element_decoding(o):
    bits = np.array([0x3F80, 0xC000, 0x3FC0, 0x0000, 0x8000, 0x4049, 0x0001], dtype=np.uint16)
    want = [1.0, -2.0, 1.5, 0.0, -0.0, 3.140625, 2.0 ** -133]
    got = o.to_float64(bits, "bf16")
    assert got.tolist() == want
    h = np.array([0x3C00, 0xC000, 0x3E00, 0x0001], dtype=np.uint16).view(np.float16)
    assert o.to_float64(h, "f16").tolist() == [1.0, -2.0, 1.5, 2.0 ** -24]


def pin_write_roundtrip(o):
    """After the write, reading each sequence through its table returns the new
    token's K and V at position T - 1 and the earlier tokens unchanged."""
    import workloads
    for cfg in (1, 5):
        w = workloads.make(cfg) if cfg == 1 else workloads.prefix_shared(num_seqs=3, prefix_len=20, max_suffix=9)
        k, v = o.write_kv(w.k_pool, w.v_pool, w.new_k, w.new_v, w.slot_mapping, w.block_size)
        for i in range(w.num_seqs):
            T = int(w.context_lens[i])
            kg = o.gather_tokens(k, w.block_tables[i], T, w.block_size, w.dtype)
            vg = o.gather_tokens(v, w.block_tables[i], T, w.block_size, w.dtype)
            assert np.array_equal(kg[T - 1], o.to_float64(w.new_k[i], w.dtype))
            assert np.array_equal(vg[T - 1], o.to_float64(w.new_v[i], w.dtype))
            assert np.isfinite(kg).all() and np.isfinite(vg).all()
        # nothing but the target slots changed
        changed = np.nonzero(np.any(k.view(np.uint8).reshape(k.shape[0], k.shape[1], k.shape[2], -1)
                                    != w.k_pool.view(np.uint8).reshape(k.shape[0], k.shape[1], k.shape[2], -1),
                                    axis=(1, 3)))
        got = sorted(int(p) * w.block_size + int(r) for p, r in zip(*changed))
        assert got == sorted(int(s) for s in w.slot_mapping if s >= 0)


def pin_slot_formula(o):
    """The generator's slot mapping equals table[floor(t/B)]*B + t mod B at
    t = T - 1, and the pages' block-table example maps as printed."""
    import workloads
    for cfg in (1, 2, 5):
        w = workloads.make(cfg)
        for i in range(w.num_seqs):
            T = int(w.context_lens[i])
            assert w.slot_mapping[i] == o.slot_of_token(w.block_tables[i], T - 1, w.block_size)
    g = load_golden()["block_table_example"]
    table, B = g["logical_to_physical"], g["block_size"]
    assert o.token_location(table, 0, B) == (42, 0)
    assert o.token_location(table, 20, B) == (109, 4)
    assert o.token_location(table, 47, B) == (12, 15)
    assert o.slot_of_token(table, 20, B) == 109 * 16 + 4
    assert o.slot_location(109 * 16 + 4, B) == (109, 4)


def pin_block_counts(o):
    """ceil(T/B) blocks per sequence, fewer than B wasted slots, in every
    generated workload and in the pages' worked examples."""
    import workloads
    for cfg in (1, 2, 3, 5):
        w = workloads.make(cfg, poison=False) if cfg != 3 else workloads.llama3_8b(num_seqs=64, poison=False)
        for i in range(w.num_seqs):
            T = int(w.context_lens[i])
            n = int((w.block_tables[i] >= 0).sum())
            assert n == o.blocks_for_tokens(T, w.block_size)
            assert 0 <= n * w.block_size - T < w.block_size
        assert o.wasted_slots_paged(w.context_lens, w.block_size) < w.num_seqs * w.block_size
    g = load_golden()
    for e in g["blocks_per_request"]:
        if "blocks" in e:
            assert o.blocks_for_tokens(e["tokens"], e["block_size"]) == e["blocks"]
        else:
            assert e["tokens"] // e["block_size"] == e["full_blocks"]
            assert o.blocks_for_tokens(e["tokens"], e["block_size"]) == e["full_blocks"] + 1
    s = g["sliding_window"]
    assert o.blocks_for_tokens(s["window"], s["block_size"]) + 1 == s["max_blocks"]
    f = g["fragmentation"]
    assert o.wasted_slots_contiguous(f["lens"], f["max_len"]) + f["tokens"] == f["contiguous_slots"]
    assert o.wasted_slots_paged(f["lens"], f["block_size"]) + f["tokens"] == f["paged_slots"]
    assert round(100 * f["tokens"] / f["contiguous_slots"]) == 33
    assert round(100 * f["tokens"] / f["paged_slots"]) == 99


def pin_byte_accounting(o):
    g = load_golden()
    for e in g["kv_bytes_per_token"]:
        assert o.kv_bytes_per_token(e["layers"], e["kv_heads"], e["head_dim"], e["dtype_bytes"]) == e["expected"]
    for e in g["kv_bytes_measured"]:
        per = o.kv_bytes_per_token(e["layers"], e["kv_heads"], e["head_dim"], e["dtype_bytes"])
        assert per * e["tokens"] == e["expected"]
        # the per-step reader: one layer, these tokens, times the layer count
        assert o.kv_bytes_read([e["tokens"]], e["kv_heads"], e["head_dim"], e["dtype_bytes"]) * e["layers"] == e["expected"]
    for e in g["block_bytes"]:
        assert o.block_bytes(e["layers"], e["block_size"], e["kv_heads"], e["head_dim"], e["dtype_bytes"]) == e["expected"]
    c = g["pool_capacity"]
    blocks = (c["pool_gib"] << 30) // (c["block_mib"] << 20)
    tokens = blocks * c["block_size"]
    assert abs(blocks - c["printed_blocks"]) <= c["tolerance_rel"] * c["printed_blocks"]
    assert abs(tokens - c["printed_tokens"]) <= c["tolerance_rel"] * c["printed_tokens"]
    assert tokens // c["full_context"] == c["printed_full_requests"]
    assert abs(tokens // 512 - c["printed_512_requests"]) <= c["tolerance_rel"] * c["printed_512_requests"]
    k = g["concurrency"]
    reserve = k["bytes_per_token"] * k["reserve_tokens"]
    assert round(reserve / 1e6) == k["printed_reservation_mb"]
    assert int(k["free_bytes"] // reserve) == k["printed_contiguous_requests"]
    req = o.blocks_for_tokens(k["typical_tokens"], k["block_size"]) * k["block_size"] * k["bytes_per_token"]
    assert round(req / 1e6, 1) == k["printed_request_mb"]
    assert int(k["free_bytes"] // req) == k["printed_paged_requests"]
    assert round(1 - k["typical_tokens"] / k["reserve_tokens"], 3) == k["printed_untouched"]
    assert round(k["printed_paged_requests"] / k["printed_contiguous_requests"], 1) == k["printed_gain"]
    p = g["prefix_sharing"]
    copies = p["requests"] * p["prefix_tokens"] * p["bytes_per_token"]
    shared = p["prefix_tokens"] * p["bytes_per_token"]
    assert round(copies / 1e9, 2) == p["printed_copies_gb"]
    assert round(shared / 1e9, 3) == p["printed_shared_gb"]
    assert round((copies - shared) / 1e9, 2) == p["printed_freed_gb"]
    assert int((copies - shared) // req) == p["printed_more_requests"]
    b = g["static_batch"]
    frac = o.static_batch_useful_fraction(b["prompts"], b["outputs"])
    assert frac == b["numerator"] / b["denominator"]
    assert round(100 * frac) == 62


def pin_toy_batch_config(o):
    """Config 1's lengths are prompt + output of the toy batch: 7, 8, 9, 8."""
    import workloads
    w = workloads.make(1)
    g = load_golden()["static_batch"]
    assert w.context_lens.tolist() == [p + q for p, q in zip(g["prompts"], g["outputs"])]
    assert int(w.context_lens.sum()) == g["numerator"]
    assert o.kv_bytes_read(w.context_lens, 4, 64, 4) == 65536


def pin_poison_isolated(o):
    """NaN in unused slots never reaches the output once the new token is
    written; decoding before the write does see the NaN of the empty slot."""
    import workloads
    w = workloads.make(1)
    after = _decode_after_write(o, w)
    assert np.isfinite(after).all()
    before = o.decode(w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale, w.dtype)
    assert np.isnan(before).all(axis=(1, 2)).all()


# ---------------------------------------------------------------------------
# sliding window ("vLLM Framework and Inference Engine Design", section "How
# does it support prompts of arbitrary length? Does it have a sliding window?")
# ---------------------------------------------------------------------------
def _release_before_window(bt, lens, window, B, k_pool, v_pool):
    """Blocks wholly before each sequence's window may be released: their
    table entries become -1 and their contents NaN (private blocks here)."""
    bt, kp, vp = bt.copy(), k_pool.copy(), v_pool.copy()
    for i, T in enumerate(lens):
        for j in range(max(0, int(T) - window) // B):
            kp[bt[i, j]] = np.nan
            vp[bt[i, j]] = np.nan
            bt[i, j] = -1
    return bt, kp, vp


WINDOW_CASES = [
    dict(seed=31, lens=[1, 5, 11, 16, 17, 40], Hq=4, Hkv=2, D=8, B=4),
    dict(seed=32, lens=[3, 33, 2, 0], Hq=6, Hkv=3, D=6, B=2),
    dict(seed=33, lens=[37, 64], Hq=8, Hkv=1, D=4, B=8),
]


def pin_window_bruteforce(o):
    """Each query attends to exactly the last W tokens: the contiguous brute
    force over those tokens, with the blocks before the window released."""
    for c in WINDOW_CASES:
        q, kp, vp, bt, lens, ck, cv = _tiny_problem(c["seed"], c["lens"], c["Hq"], c["Hkv"],
                                                    c["D"], c["B"])
        scale = float(np.float32(0.41))
        G = c["Hq"] // c["Hkv"]
        for W in (1, 2, 3, 5, 16, 21):
            bt_r, kp_r, vp_r = _release_before_window(bt, lens, W, c["B"], kp, vp)
            got = o.decode(q, kp_r, vp_r, bt_r, lens, scale, "f32", window=W)
            for i, T in enumerate(lens):
                first = max(0, int(T) - W)
                want = np.array(_brute(q[i].tolist(), ck[i][first:].tolist(),
                                       cv[i][first:].tolist(), scale, G))
                np.testing.assert_allclose(got[i], want, rtol=1e-12, atol=1e-13)


def pin_window_closed_forms(o):
    """W >= T is full attention (the same numbers, bit for bit); W = 1 returns
    the newest token's value row exactly; T = 0 stays zero."""
    c = WINDOW_CASES[0]
    q, kp, vp, bt, lens, ck, cv = _tiny_problem(c["seed"], c["lens"], c["Hq"], c["Hkv"],
                                                c["D"], c["B"])
    full = o.decode(q, kp, vp, bt, lens, 0.3, "f32")
    for W in (int(max(lens)), 10 ** 9):
        assert np.array_equal(o.decode(q, kp, vp, bt, lens, 0.3, "f32", window=W), full)
    one = o.decode(q, kp, vp, bt, lens, 0.3, "f32", window=1)
    G = c["Hq"] // c["Hkv"]
    for i, T in enumerate(lens):
        for h in range(c["Hq"]):
            want = cv[i][T - 1][h // G] if T else np.zeros(c["D"])
            assert np.array_equal(one[i, h], np.asarray(want, dtype=np.float64))
    z = o.decode(q[:1], kp, vp, bt[:1], np.array([0]), 0.3, "f32", window=4)
    assert np.array_equal(z, np.zeros_like(z))


def pin_window_blocks(o):
    """Blocks a windowed sequence needs: exactly the distinct blocks of its
    last W positions; at most ceil((W-1)/B) + 1 over all lengths, which is
    within the page's bound ceil(W/B) + 1 and equals it unless B divides
    W - 1, as in the page's Mistral example (W = 4,096, B = 16: at most 257)."""
    s = load_golden()["sliding_window"]
    worst = max(o.window_blocks(T, s["window"], s["block_size"])
                for T in range(1, 3 * s["window"]))
    assert worst == s["max_blocks"]
    for B in (1, 4, 16):
        for W in (1, 5, 16, 17, 64):
            bound = -(-W // B) + 1
            seen = 0
            for T in range(0, 3 * W + 2 * B):
                first = o.window_start(T, W)
                distinct = len({t // B for t in range(first, T)})
                n = o.window_blocks(T, W, B)
                assert n == distinct and n <= bound
                seen = max(seen, n)
            assert seen == -(-(W - 1) // B) + 1
            assert (seen == bound) == ((W - 1) % B != 0)


# ---------------------------------------------------------------------------
# chunked prefill (a prompt chunk attends causally through the block table)
# ---------------------------------------------------------------------------
PREFILL_CASES = [
    dict(seed=41, lens=[1, 5, 11, 16, 17, 40], mq=[1, 5, 3, 16, 1, 9], Hq=4, Hkv=2, D=8, B=4),
    dict(seed=42, lens=[3, 33, 2, 6], mq=[2, 0, 2, 6], Hq=6, Hkv=3, D=6, B=2),
    dict(seed=43, lens=[37, 64], mq=[20, 3], Hq=8, Hkv=1, D=4, B=8),
]


def _prefill_q(seed, mq, Hq, D):
    return np.random.default_rng(seed + 1000).standard_normal((sum(mq), Hq, D)).astype(np.float32)


def pin_prefill_bruteforce(o):
    """Row r of a chunk of M rows ending at T attends to the first T - M + r + 1
    tokens: the contiguous brute force over exactly those."""
    for c in PREFILL_CASES:
        q0, kp, vp, bt, lens, ck, cv = _tiny_problem(c["seed"], c["lens"], c["Hq"], c["Hkv"],
                                                     c["D"], c["B"])
        q = _prefill_q(c["seed"], c["mq"], c["Hq"], c["D"])
        scale = float(np.float32(0.29))
        got = o.prefill(q, kp, vp, bt, lens, c["mq"], scale, "f32")
        G = c["Hq"] // c["Hkv"]
        row = 0
        for i, (T, M) in enumerate(zip(c["lens"], c["mq"])):
            for r in range(M):
                n = T - M + r + 1
                want = np.array(_brute(q[row + r].tolist(), ck[i][:n].tolist(),
                                       cv[i][:n].tolist(), scale, G))
                np.testing.assert_allclose(got[row + r], want, rtol=1e-12, atol=1e-13)
            row += M


def pin_prefill_special_cases(o):
    """One query per sequence is the decode step, bit for bit; a chunk's rows
    do not depend on how the prompt was chunked; the first position of a
    sequence returns its value row exactly; NaN in positions after a row's own
    never reaches it (causality)."""
    c = PREFILL_CASES[0]
    q0, kp, vp, bt, lens, ck, cv = _tiny_problem(c["seed"], c["lens"], c["Hq"], c["Hkv"],
                                                 c["D"], c["B"])
    ones = [1 if T else 0 for T in c["lens"]]
    dec = o.decode(q0, kp, vp, bt, lens, 0.3, "f32")
    pre = o.prefill(q0[[i for i, T in enumerate(c["lens"]) if T]], kp, vp, bt, lens, ones, 0.3,
                    "f32")
    assert np.array_equal(pre, dec[[i for i, T in enumerate(c["lens"]) if T]])
    # sequence 5 (40 tokens): its last 30 positions as one chunk, or as 10 + 20
    T = c["lens"][5]
    q = np.random.default_rng(7).standard_normal((30, c["Hq"], c["D"])).astype(np.float32)
    one = o.prefill(q, kp, vp, bt[5:6], [T], [30], 0.3, "f32")
    a = o.prefill(q[:10], kp, vp, bt[5:6], [T - 20], [10], 0.3, "f32")
    b = o.prefill(q[10:], kp, vp, bt[5:6], [T], [20], 0.3, "f32")
    assert np.array_equal(one, np.concatenate([a, b]))
    # a whole prompt as one chunk: its row 0 is v_0 for every head
    G = c["Hq"] // c["Hkv"]
    whole = o.prefill(q[:5], kp, vp, bt[1:2], [5], [5], 0.3, "f32")
    for h in range(c["Hq"]):
        assert np.array_equal(whole[0, h], np.asarray(cv[1][0][h // G], dtype=np.float64))
    # causality: poison every slot after position 9 of sequence 5
    kp2, vp2 = kp.copy(), vp.copy()
    for t in range(10, T):
        blk, off = bt[5, t // c["B"]], t % c["B"]
        kp2[blk, :, off, :] = np.nan
        vp2[blk, :, off, :] = np.nan
    early = o.prefill(q[:10], kp2, vp2, bt[5:6], [10], [10], 0.3, "f32")
    assert np.isfinite(early).all()
    assert np.array_equal(early, o.prefill(q[:10], kp, vp, bt[5:6], [10], [10], 0.3, "f32"))


# ---------------------------------------------------------------------------
# FP8 KV cache: OCP E4M3 codes with one float32 scale per pool
# ---------------------------------------------------------------------------
def pin_fp8_codec(o):
    """Fixed values of the OFP8 E4M3 definition; every finite code survives
    decode-encode; encoding is the nearest finite code with ties to an even
    mantissa (found by brute force over all codes, not by the encoder's own
    arithmetic), saturating at 448."""
    dec = o.fp8_e4m3_decode
    fixed = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0x77: 240.0, 0xB8: -1.0, 0xFE: -448.0}
    for code, val in fixed.items():
        assert dec(np.array([code], np.uint8))[0] == val
    assert np.signbit(dec(np.array([0x80], np.uint8))[0])
    assert np.isnan(dec(np.array([0x7F, 0xFF], np.uint8))).all()
    codes = np.arange(256, dtype=np.uint8)
    vals = dec(codes)
    fin = ~np.isnan(vals)
    assert np.array_equal(o.fp8_e4m3_encode(vals[fin].astype(np.float32)), codes[fin])
    # brute force: nearest code, ties to even mantissa, on random values and
    # on every midpoint between neighbouring codes
    pos = np.sort(vals[:0x7F])                       # 0 .. 448, increasing
    mids = (pos[1:] + pos[:-1]) / 2
    rng = np.random.default_rng(5)
    xs = np.concatenate([mids, -mids, rng.standard_normal(3000) * 40.0,
                         np.exp2(rng.uniform(-12, 9, 3000)), [500.0, -1e6, 447.9, 2.0 ** -11]])
    xs = xs.astype(np.float32)
    got = o.fp8_e4m3_encode(xs)
    for x, code in zip(xs.astype(np.float64), got):
        a = min(abs(x), 448.0)
        d = np.abs(pos - a)
        best = np.flatnonzero(d == d.min())
        k = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        want = k | (0x80 if np.signbit(x) else 0)
        assert code == want, (x, code, want)


def pin_fp8_decode(o):
    """Decode over FP8 pools equals the plain decode over the dequantized
    values (code times scale; scales of few significant bits keep that product
    exact in float32), and the dequantized write is within half a step of the
    original values."""
    c = WINDOW_CASES[0]
    q, kp, vp, bt, lens, ck, cv = _tiny_problem(c["seed"], c["lens"], c["Hq"], c["Hkv"],
                                                c["D"], c["B"])
    ks, vs = 3.0 / 64.0, 2.0 ** -5
    kc = o.quantize_fp8(np.nan_to_num(kp), "f32", ks)
    vc = o.quantize_fp8(np.nan_to_num(vp), "f32", vs)
    got = o.decode(q, kc, vc, bt, lens, 0.3, "f32", kv_dtype="fp8e4m3", k_scale=ks, v_scale=vs)
    kf = (o.fp8_e4m3_decode(kc) * np.float32(ks)).astype(np.float32)
    vf = (o.fp8_e4m3_decode(vc) * np.float32(vs)).astype(np.float32)
    assert np.array_equal(kf.astype(np.float64), o.fp8_e4m3_decode(kc) * float(np.float32(ks)))
    want = o.decode(q, kf, vf, bt, lens, 0.3, "f32")
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)
    x = np.random.default_rng(9).standard_normal(20000).astype(np.float32) * 3.0
    err = np.abs(o.fp8_e4m3_decode(o.quantize_fp8(x, "f32", ks)) * np.float32(ks) - x)
    step = np.where(np.abs(x) / ks < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.abs(x) / ks)) - 3)) * ks
    assert (err <= step / 2 * (1 + 1e-6)).all()
    # the slot write into FP8 pools stores the quantized rows at their slots
    pool = np.zeros((4, 1, 2, 3), np.uint8)
    k_new = np.array([[[1.0, -2.5, 1000.0]], [[0.1, 0.0, -0.3]]], np.float32)
    kq, vq = o.write_kv_fp8(pool, pool, k_new, -k_new, [5, 0], 2, "f32", 0.5, 2.0)
    assert np.array_equal(kq[2, 0, 1], o.quantize_fp8(k_new[0, 0], "f32", 0.5))
    assert np.array_equal(vq[0, 0, 0], o.quantize_fp8(-k_new[1, 0], "f32", 2.0))
    assert o.fp8_e4m3_decode(kq[2, 0, 1])[2] == 448.0      # 2000 saturates


ALL_PINS = [
    pin_contiguous_bruteforce,
    pin_page_sketch_torch,
    pin_placement_invariance,
    pin_prefix_sharing,
    pin_closed_forms,
    pin_hard_max,
    pin_element_decoding,
    pin_write_roundtrip,
    pin_slot_formula,
    pin_block_counts,
    pin_byte_accounting,
    pin_toy_batch_config,
    pin_poison_isolated,
    pin_window_bruteforce,
    pin_window_closed_forms,
    pin_window_blocks,
    pin_prefill_bruteforce,
    pin_prefill_special_cases,
    pin_fp8_codec,
    pin_fp8_decode,
]
