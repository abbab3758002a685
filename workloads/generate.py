"""Seeded synthetic decode workloads, shared by the tests and ``bench.py``.

This module only draws random numbers and lays blocks out the way the pages'
block manager does.  It contains no attention arithmetic.  The oracle and the
GPU library are both fed from what it returns; neither is imported here.

Layout of what it builds (one layer):

* ``k_pool``, ``v_pool``: ``[num_blocks][num_kv_heads][block_size][head_dim]``.
* ``block_tables``: int32 ``[num_seqs][max_blocks_per_seq]``; entries past a
  sequence's ``ceil(T/B)`` blocks hold ``PAD_ENTRY`` (-1) and must never be read.
* ``context_lens``: int32 ``[num_seqs]``; ``T_i`` includes the newest token.
* ``new_k``, ``new_v``: ``[num_seqs][num_kv_heads][head_dim]``; the newest token
  (position ``T_i - 1``) of every sequence, not yet in the pool.
  ``slot_mapping`` (int32 ``[num_seqs]``) says where it goes.  Before the write
  that slot holds NaN, so a decode that runs before the write is visible.

Values are float32 N(0, 1) draws rounded to the element type
(round-to-nearest-even).  bf16 elements are carried as uint16 bit patterns.
With ``poison=True`` every pool slot that holds no live token is NaN.  Table
padding is -1 in every case.

Draw order per workload: context lengths, block placement, q, pool contents,
new-token k/v.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

PAD_ENTRY = -1
DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


# ---------------------------------------------------------------------------
# element rounding
# ---------------------------------------------------------------------------
def round_to_dtype(x32: np.ndarray, dtype: str) -> np.ndarray:
    """float32 array -> element array of ``dtype`` (RNE; NaN stays NaN)."""
    if dtype == "f32":
        return x32.astype(np.float32, copy=False)
    if dtype == "f16":
        return x32.astype(np.float16)
    if dtype == "bf16":
        bits = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
        rounded = (bits + np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        out = rounded.astype(np.uint16)
        nan = np.isnan(x32)
        if nan.any():
            out[nan] = np.uint16(0x7FC0)
        return out
    raise ValueError(dtype)


def nan_element(dtype: str):
    return {"f32": np.float32(np.nan), "f16": np.float16(np.nan),
            "bf16": np.uint16(0x7FC0)}[dtype]


def numpy_dtype(dtype: str):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]


# ---------------------------------------------------------------------------
# workload container
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    q: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    block_tables: np.ndarray
    context_lens: np.ndarray
    new_k: np.ndarray
    new_v: np.ndarray
    slot_mapping: np.ndarray
    scale: float
    refcount: np.ndarray          # tables referencing each physical block
    seed: int = 0

    @property
    def num_seqs(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def elem_bytes(self) -> int:
        return DTYPE_BYTES[self.dtype]


# ---------------------------------------------------------------------------
# building blocks
# ---------------------------------------------------------------------------
_CHUNK = 1 << 22
_POOL = None


def _threads():
    global _POOL
    if _POOL is None:
        import os
        from concurrent.futures import ThreadPoolExecutor
        n = min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 8)
        _POOL = ThreadPoolExecutor(max(1, n))
    return _POOL


def _normal(rng: np.random.Generator, shape, dtype: str):
    """N(0,1) float32 draws rounded to ``dtype``.

    The array is cut into fixed 4 Mi-element chunks, each drawn by its own
    PCG64 stream spawned from one seed taken from ``rng``; the result depends
    only on ``rng``'s state, not on how many threads fill the chunks."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=numpy_dtype(dtype))
    flat = out.reshape(-1)
    n = flat.size
    seed = int(rng.integers(0, 2 ** 63))
    if n == 0:
        return out
    kids = np.random.SeedSequence(seed).spawn(-(-n // _CHUNK))

    def fill(i):
        a, b = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        g = np.random.Generator(np.random.PCG64(kids[i]))
        flat[a:b] = round_to_dtype(g.standard_normal(b - a, dtype=np.float32), dtype)

    if len(kids) == 1:
        fill(0)
    else:
        list(_threads().map(fill, range(len(kids))))
    return out


def _blocks_needed(T: int, B: int) -> int:
    return -(-int(T) // int(B))


def _place(tables_blocks, lens, B, num_blocks, max_blocks):
    """Dense int32 block table from per-sequence block lists (padding -1)."""
    bt = np.full((len(lens), max_blocks), PAD_ENTRY, dtype=np.int32)
    for i, blocks in enumerate(tables_blocks):
        bt[i, :len(blocks)] = blocks
    return bt


def _live_tokens(table_row, T: int, B: int):
    """(block, offset) of the T live tokens of one sequence, token order:
    the pages' placement, token t in block table[t // B] at offset t % B."""
    t = np.arange(T, dtype=np.int64)
    return np.asarray(table_row, dtype=np.int64)[t // B], t % B


def _finish(name, dtype, Hq, Hkv, D, B, lens, tables_blocks, num_blocks,
            max_blocks, rng, poison, seed, pool_fill=None):
    """Common tail: q, pools, new tokens, poisoning, slot mapping."""
    lens = np.asarray(lens, dtype=np.int32)
    N = len(lens)
    bt = _place(tables_blocks, lens, B, num_blocks, max_blocks)
    q = _normal(rng, (N, Hq, D), dtype)
    if pool_fill is None:
        k_pool = _normal(rng, (num_blocks, Hkv, B, D), dtype)
        v_pool = _normal(rng, (num_blocks, Hkv, B, D), dtype)
    else:
        k_pool, v_pool = pool_fill(rng)
    new_k = _normal(rng, (N, Hkv, D), dtype)
    new_v = _normal(rng, (N, Hkv, D), dtype)

    refcount = np.zeros(num_blocks, dtype=np.int32)
    for blocks in tables_blocks:
        for p in blocks:
            refcount[p] += 1

    nan = nan_element(dtype)
    if poison:
        live = np.zeros((num_blocks, B), dtype=bool)
        for i in range(N):
            p, r = _live_tokens(bt[i], int(lens[i]), B)
            live[p, r] = True
        dead_p, dead_r = np.nonzero(~live)
        k_pool[dead_p, :, dead_r, :] = nan
        v_pool[dead_p, :, dead_r, :] = nan

    slots = np.full(N, -1, dtype=np.int32)
    for i in range(N):
        T = int(lens[i])
        if T == 0:
            continue
        p, r = _live_tokens(bt[i], T, B)
        p, r = int(p[-1]), int(r[-1])
        slots[i] = p * B + r
        # the newest token is not in the pool yet
        k_pool[p, :, r, :] = nan
        v_pool[p, :, r, :] = nan
    if len(set(int(s) for s in slots if s >= 0)) != int((slots >= 0).sum()):
        raise AssertionError("two sequences write one slot; sharing must end before the newest token")

    return Workload(name=name, dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv,
                    head_dim=D, block_size=B, q=q, k_pool=k_pool, v_pool=v_pool,
                    block_tables=bt, context_lens=lens, new_k=new_k, new_v=new_v,
                    slot_mapping=slots, scale=float(np.float32(1.0 / math.sqrt(D))),
                    refcount=refcount, seed=seed)


def random_paged(name, dtype, Hq, Hkv, D, B, lens, seed, *, spare_frac=0.0,
                 max_blocks=None, poison=True, rng=None):
    """Sequences with private blocks scattered over a shuffled pool.

    ``num_blocks = ceil((1 + spare_frac) * sum ceil(T_i/B))``; sequence i takes
    the next ``ceil(T_i/B)`` blocks of a random permutation of the pool."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    lens = [int(x) for x in lens]
    need = [_blocks_needed(T, B) for T in lens]
    used = sum(need)
    num_blocks = max(1, int(math.ceil((1.0 + spare_frac) * used - 1e-9)))
    perm = rng.permutation(num_blocks)
    tables_blocks, at = [], 0
    for n in need:
        tables_blocks.append([int(x) for x in perm[at:at + n]])
        at += n
    mb = max_blocks if max_blocks is not None else max([1] + need)
    if mb < max([0] + need):
        raise ValueError("max_blocks smaller than a sequence needs")
    return _finish(name, dtype, Hq, Hkv, D, B, lens, tables_blocks, num_blocks,
                   mb, rng, poison, seed)


# ---------------------------------------------------------------------------
# the five configurations
# ---------------------------------------------------------------------------
def tiny(seed: int = 1, poison: bool = True) -> Workload:
    """fp32, 4 seqs with lens [7, 8, 9, 8] (prompt + output of the toy batch
    in "Why is batching multiple requests difficult ..."), 4 q = 4 kv heads,
    head_dim 64, block size 4, 16 physical blocks; the tables are the first 9
    entries of a seeded permutation of the pool, in sequence order."""
    rng = np.random.default_rng(seed)
    prompts, outputs = [3, 6, 2, 5], [4, 2, 7, 3]
    lens = [p + o for p, o in zip(prompts, outputs)]
    B, NB = 4, 16
    perm = rng.permutation(NB)
    tables_blocks, at = [], 0
    for T in lens:
        n = _blocks_needed(T, B)
        tables_blocks.append([int(x) for x in perm[at:at + n]])
        at += n
    return _finish("tiny-f32", "f32", 4, 4, 64, B, lens, tables_blocks, NB, 3,
                   rng, poison, seed)


def qwen2_05b(seed: int = 2, poison: bool = True, num_seqs: int = 32,
              max_len: int = 4096) -> Workload:
    """Qwen2-0.5B-shaped layer, fp16: 14 q / 2 kv heads, head_dim 64, block 16,
    context lens uniform on 1..max_len, 20% spare blocks, shuffled tables."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, max_len, size=num_seqs, endpoint=True)
    return random_paged("qwen2-0.5b-f16", "f16", 14, 2, 64, 16, lens, seed,
                        spare_frac=0.2, max_blocks=_blocks_needed(max_len, 16),
                        poison=poison, rng=rng)


LLAMA3_SIGMA = math.log(735.0 / 260.0) / 1.6448536269514722
LLAMA3_MU = math.log(400.0) - 0.5 * LLAMA3_SIGMA ** 2


def llama3_8b(seed: int = 3, poison: bool = True, num_seqs: int = 256,
              max_len: int = 4096) -> Workload:
    """Llama-3-8B-shaped layer, bf16: 32 q / 8 kv heads, head_dim 128, block 16,
    256 seqs, lognormal context lens with mean 400 (sigma from the sudo.vn
    page's median 260 / p95 735 length mix), rounded and clipped to
    1..max_len; exactly the blocks the sequences need, shuffled."""
    rng = np.random.default_rng(seed)
    x = rng.lognormal(LLAMA3_MU, LLAMA3_SIGMA, size=num_seqs)
    lens = np.clip(np.rint(x), 1, max_len).astype(np.int64)
    return random_paged("llama3-8b-bf16", "bf16", 32, 8, 128, 16, lens, seed,
                        spare_frac=0.0, max_blocks=_blocks_needed(max_len, 16),
                        poison=poison, rng=rng)


def llama2_7b(seed: int = 4, poison: bool = True, num_seqs: int = 64,
              context_len: int = 4096) -> Workload:
    """Llama-2-7B-shaped MHA layer, fp16: 32 q = 32 kv heads, head_dim 128,
    block 16, every sequence at context_len tokens, shuffled pool with no
    spare blocks."""
    rng = np.random.default_rng(seed)
    lens = [context_len] * num_seqs
    return random_paged("llama2-7b-f16", "f16", 32, 32, 128, 16, lens, seed,
                        spare_frac=0.0, max_blocks=_blocks_needed(context_len, 16),
                        poison=poison, rng=rng)


def prefix_shared(seed: int = 5, poison: bool = True, num_seqs: int = 12,
                  prefix_len: int = 1800, max_suffix: int = 512,
                  share: bool = True) -> Workload:
    """70B-style head shape, bf16: 64 q / 8 kv heads, head_dim 128, block 16.
    ``num_seqs`` sequences share a ``prefix_len``-token prefix (the twelve
    requests with an 1,800-token prefix on the bibekananda.in page), then hold
    private suffixes of U{0..max_suffix} tokens plus the new token.

    Only full prefix blocks are shared (refcount num_seqs).  The tail of the
    prefix that does not fill a block is copied into each sequence's first
    private block, which also receives its suffix; the newest token lands in
    a private block.  With ``share=False`` every sequence holds private
    copies of the same prefix content instead (same values, other blocks)."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, D, dtype = 16, 64, 8, 128, "bf16"
    suffix = rng.integers(0, max_suffix, size=num_seqs, endpoint=True)
    lens = [prefix_len + int(s) + 1 for s in suffix]
    n_shared = prefix_len // B
    tail = prefix_len - n_shared * B
    private_need = [_blocks_needed(T - n_shared * B, B) for T in lens]
    num_blocks = n_shared + sum(private_need)
    perm = [int(x) for x in rng.permutation(num_blocks)]
    shared_blocks = perm[:n_shared]
    at = n_shared
    privates = []
    for n in private_need:
        privates.append(perm[at:at + n])
        at += n
    max_blocks = _blocks_needed(prefix_len + max_suffix + 1, B)

    # token contents drawn in token order: prefix once, then each suffix
    def fill(rng_):
        prefix_k = _normal(rng_, (prefix_len, Hkv, D), dtype)
        prefix_v = _normal(rng_, (prefix_len, Hkv, D), dtype)
        k_pool = np.zeros((num_blocks, Hkv, B, D), dtype=numpy_dtype(dtype))
        v_pool = np.zeros_like(k_pool)
        for jb, p in enumerate(shared_blocks):
            k_pool[p] = prefix_k[jb * B:(jb + 1) * B].transpose(1, 0, 2)
            v_pool[p] = prefix_v[jb * B:(jb + 1) * B].transpose(1, 0, 2)
        for i, T in enumerate(lens):
            rest = T - n_shared * B           # tokens in private blocks
            sk = _normal(rng_, (rest, Hkv, D), dtype)
            sv = _normal(rng_, (rest, Hkv, D), dtype)
            sk[:tail] = prefix_k[n_shared * B:]
            sv[:tail] = prefix_v[n_shared * B:]
            for jb, p in enumerate(privates[i]):
                lo, hi = jb * B, min(rest, (jb + 1) * B)
                k_pool[p, :, :hi - lo, :] = sk[lo:hi].transpose(1, 0, 2)
                v_pool[p, :, :hi - lo, :] = sv[lo:hi].transpose(1, 0, 2)
        return k_pool, v_pool

    tables_blocks = [shared_blocks + privates[i] for i in range(num_seqs)]
    w = _finish("prefix-70b-bf16", dtype, Hq, Hkv, D, B, lens, tables_blocks,
                num_blocks, max_blocks, rng, poison, seed, pool_fill=fill)
    if not share:
        w = unshare_blocks(w)
    return w


CONFIGS = {
    1: tiny,
    2: qwen2_05b,
    3: llama3_8b,
    4: llama2_7b,
    5: prefix_shared,
}


def make(config: int, seed: int | None = None, poison: bool = True, **kw) -> Workload:
    fn = CONFIGS[int(config)]
    return fn(seed=int(config) if seed is None else int(seed), poison=poison, **kw)


# ---------------------------------------------------------------------------
# structural transforms used by the invariance checks
# ---------------------------------------------------------------------------
def relabel_blocks(w: Workload, perm: np.ndarray) -> Workload:
    """Move physical block p to perm[p] (pool and tables); the logical
    content of every sequence is unchanged."""
    perm = np.asarray(perm, dtype=np.int64)
    NB = w.num_blocks
    if sorted(perm.tolist()) != list(range(NB)):
        raise ValueError("perm must be a permutation of the pool")
    k_pool = np.empty_like(w.k_pool)
    v_pool = np.empty_like(w.v_pool)
    k_pool[perm] = w.k_pool
    v_pool[perm] = w.v_pool
    bt = w.block_tables.copy()
    m = bt >= 0
    bt[m] = perm[bt[m]].astype(np.int32)
    B = w.block_size
    slots = w.slot_mapping.copy()
    s = slots >= 0
    slots[s] = (perm[slots[s] // B] * B + slots[s] % B).astype(np.int32)
    refcount = np.empty_like(w.refcount)
    refcount[perm] = w.refcount
    return dataclasses.replace(w, k_pool=k_pool, v_pool=v_pool, block_tables=bt,
                               slot_mapping=slots, refcount=refcount)


def unshare_blocks(w: Workload) -> Workload:
    """Give every table its own copy of each block it shares with another
    table (same contents, fresh physical blocks appended to the pool)."""
    bt = w.block_tables.copy()
    extra_k, extra_v = [], []
    NB = w.num_blocks
    seen = {}
    for i in range(w.num_seqs):
        for j in range(bt.shape[1]):
            p = int(bt[i, j])
            if p < 0 or w.refcount[p] <= 1:
                continue
            if p in seen:                    # later users get copies
                bt[i, j] = NB + len(extra_k)
                extra_k.append(w.k_pool[p])
                extra_v.append(w.v_pool[p])
            else:
                seen[p] = i
    if not extra_k:
        return w
    k_pool = np.concatenate([w.k_pool, np.stack(extra_k)])
    v_pool = np.concatenate([w.v_pool, np.stack(extra_v)])
    refcount = np.zeros(k_pool.shape[0], dtype=np.int32)
    for row in bt:
        for p in row:
            if p >= 0:
                refcount[p] += 1
    return dataclasses.replace(w, k_pool=k_pool, v_pool=v_pool, block_tables=bt,
                               refcount=refcount)
