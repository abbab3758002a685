"""CPU oracle for paged decode attention and the paged KV slot write.

TEST INFRASTRUCTURE ONLY.  This module is the independent definition that the
GPU library is checked against.  Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it.  The
library never imports it, and it imports nothing from the library: the two
share no code.  Its inputs are plain NumPy arrays.

Everything is computed in float64 and written straight from the definitions on
the pages:

* "vLLM Framework and Inference Engine Design" (vineetganti.com), section
  "What is the essence of vLLM's PagedAttention?": token ``t`` sits in logical
  block ``j = floor(t / B)`` at offset ``r = t mod B``; the sequence's block
  table maps ``j`` to a physical block ``p``; its key and value are
  ``K_cache[p][r]`` and ``V_cache[p][r]`` in a pool kept per layer; ``T``
  tokens take ``ceil(T / B)`` blocks.  The page's PyTorch sketch then computes
  ``softmax(q . K^T / sqrt(d)) . V`` over the first ``T`` gathered tokens.
* Same page, section "How is vLLM's KV cache paged?": a new token's K and V
  are copied into slot ``block_table[floor(t / B)] * B + (t mod B)``; the list
  of these per-token slots is the slot mapping.
* Same page, section "How does it support prompts of arbitrary length? Does it
  have a sliding window?": in a layer trained with a sliding window of ``W``
  tokens each token attends only to the last ``W`` tokens, so only the blocks
  inside the window are needed (at most ``ceil(W / B) + 1`` of them) and older
  ones may already be released.

Readings taken where the pages leave a step open:

* Pool layout ``[num_blocks][num_kv_heads][block_size][head_dim]``.  The pages
  leave the layout to the attention backend; the oracle indexes named axes, so
  the layout is only a convention for its inputs.
* Grouped-query attention: query head ``h`` reads kv head ``floor(h / G)``
  with ``G = Hq / Hkv`` (the sudo.vn page, section "How big the KV cache is",
  only says there are fewer KV heads than query heads).
* ``scale`` is an argument (the sketch hard-codes ``1/sqrt(head_dim)``); it is
  the float32 value the GPU receives, widened to float64.
* ``T = 0`` gives an all-zero output (the sketch's softmax and sum over an
  empty set).
* The softmax subtracts the row maximum first, an exact identity.
* A negative slot in the slot mapping means "no token"; slots must be
  distinct.
* Sliding window: the token being decoded (position ``T - 1``) is one of the
  last ``W`` tokens, so the keys are positions ``max(0, T - W) .. T - 1``; table
  entries of blocks wholly before them are never read.
* FP8 KV cache (same page, the engine settings: ``kv_cache_dtype="fp8"``
  halves the KV memory; the besthub page, "Quantization: Reducing Weight & KV
  Precision": ``--kv-cache-dtype fp8`` stores the KV cache in FP8).  The
  format and scale are not on the pages (readings): OCP 8-bit floating point
  E4M3 (the published OFP8 definition: sign, 4 exponent bits with bias 7,
  3 mantissa bits, largest finite 448, no infinities, S.1111.111 is NaN) with
  one float32 scale per pool: a code is E4M3 of ``float32(x) /
  float32(scale)``, rounded to nearest even and saturated to +-448; its value
  is the decoded code times the scale.
* Chunked prefill (same page, sections on the scheduler step and on long
  prompts: a long prompt is read in chunks that run in one batch with other
  requests' decode tokens).  A sequence brings ``M`` new query rows, the last
  ``M`` of its ``T`` tokens (their K/V already written, as for a decode
  token); row ``r`` sits at position ``T - M + r`` and attends to positions
  ``0 .. T - M + r`` (causal).  A decode token is the case ``M = 1``.

Parity pins (tests/test_oracle_pins.py): contiguous brute force, a torch
float64 rendering of the page's sketch, placement invariance, shared-prefix
equality, closed forms (T = 1, q = 0, equal keys, hard maximum) and the pages'
printed byte and block arithmetic.  No function here is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

# dtype tags shared by the inputs: 'f32' and 'f16' are NumPy float arrays;
# 'bf16' arrays hold the raw 16-bit patterns as uint16 (NumPy has no bfloat16).
DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8e4m3": 1}


FP8_E4M3_MAX = 448.0


def fp8_e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Exact float64 value of E4M3 codes (uint8): normal 2^(E-7) * (1 + m/8),
    subnormal (E = 0) m * 2^-9, S.1111.111 NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(E == 0, m * 2.0 ** -9, np.ldexp(1.0 + m / 8.0, E - 7))
    out = sign * mag
    return np.where((E == 15) & (m == 7), np.nan, out)


def fp8_e4m3_encode(y) -> np.ndarray:
    """E4M3 code of float32 values: round to nearest, ties to an even
    mantissa; magnitudes of 448 and above (infinities too) saturate to 448;
    NaN gives S.1111.111."""
    y = np.asarray(y, dtype=np.float32)
    sign = (np.signbit(y).astype(np.int64) << 7)
    a = np.abs(y.astype(np.float64))
    nan = np.isnan(a)
    a = np.minimum(np.where(nan, 0.0, a), 2.0 * FP8_E4M3_MAX)   # all of these saturate
    # normal range: a = 2^e * f with f in [1, 2)
    frac, exp = np.frexp(np.where(a > 0, a, 1.0))
    e = exp - 1
    q = np.rint((frac * 2.0 - 1.0) * 8.0).astype(np.int64)        # half to even
    e = np.where(q == 8, e + 1, e)
    q = np.where(q == 8, 0, q)
    normal = ((e + 7) << 3) | q
    # subnormal range: multiples of 2^-9 (8 rounds up into the first normal)
    sub = np.rint(a * 2.0 ** 9).astype(np.int64)
    code = np.where(a < 2.0 ** -6, sub, normal)
    code = np.where(a >= FP8_E4M3_MAX, 0x7E, code)
    code = np.where(nan, 0x7F, code)
    return (code | sign).astype(np.uint8)


def quantize_fp8(x: np.ndarray, dtype: str, scale: float) -> np.ndarray:
    """Codes stored for elements x (of ``dtype``) in a pool with this scale."""
    x32 = to_float64(x, dtype).astype(np.float32)      # exact for every dtype here
    return fp8_e4m3_encode(x32 / np.float32(scale))


# ---------------------------------------------------------------------------
# element decoding
# ---------------------------------------------------------------------------
def to_float64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of every element.

    A bfloat16 number is the upper half of a float32, so its bit pattern
    shifted left by 16 is that float32; fp16 and fp32 widen exactly.
    """
    if dtype == "fp8e4m3":
        return fp8_e4m3_decode(arr)
    if dtype == "bf16":
        if arr.dtype != np.uint16:
            raise TypeError("bf16 arrays are carried as uint16 bit patterns")
        wide = arr.astype(np.uint32) << np.uint32(16)
        return wide.view(np.float32).astype(np.float64)
    if dtype == "f16":
        if arr.dtype != np.float16:
            raise TypeError("f16 arrays must be numpy.float16")
        return arr.astype(np.float64)
    if dtype == "f32":
        if arr.dtype != np.float32:
            raise TypeError("f32 arrays must be numpy.float32")
        return arr.astype(np.float64)
    raise ValueError(f"unknown dtype tag {dtype!r}")


# ---------------------------------------------------------------------------
# block arithmetic ("What is the essence of vLLM's PagedAttention?")
# ---------------------------------------------------------------------------
def blocks_for_tokens(num_tokens: int, block_size: int) -> int:
    """ceil(T / B): the number of blocks a sequence of T tokens holds."""
    return -(-int(num_tokens) // int(block_size))


def token_location(table_row, t, block_size: int):
    """Physical block and in-block offset of token t of one sequence.

    Logical block j = floor(t / B), offset r = t mod B, physical block
    p = block_table[j].  ``t`` may be an int or an integer array.
    """
    j = t // block_size
    r = t % block_size
    return np.asarray(table_row)[j], r


def slot_of_token(table_row, t: int, block_size: int) -> int:
    """The slot-mapping entry of token t: block_table[floor(t/B)] * B + (t mod B)
    ("How is vLLM's KV cache paged?", the writing step)."""
    p, r = token_location(table_row, t, block_size)
    return int(p) * block_size + int(r)


def slot_location(slot: int, block_size: int) -> tuple[int, int]:
    """Inverse of the slot formula: (physical block, offset) of a slot."""
    return slot // block_size, slot % block_size


def write_kv_fp8(k_pool: np.ndarray, v_pool: np.ndarray, k: np.ndarray, v: np.ndarray,
                 slot_mapping, block_size: int, dtype: str, k_scale: float, v_scale: float,
                 inplace: bool = False):
    """The slot write into FP8 pools (uint8 codes): the new rows, of
    ``dtype``, quantized with the pools' scales."""
    return write_kv(k_pool, v_pool, quantize_fp8(k, dtype, k_scale),
                    quantize_fp8(v, dtype, v_scale), slot_mapping, block_size, inplace=inplace)


def kv_head_for_query_head(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """Grouped-query attention: contiguous groups of G = Hq / Hkv query heads
    share one kv head (a reading; the pages only state Hkv < Hq)."""
    group = num_q_heads // num_kv_heads
    return h // group


# ---------------------------------------------------------------------------
# the slot write (reshape_and_cache)
# ---------------------------------------------------------------------------
def write_kv(k_pool: np.ndarray, v_pool: np.ndarray, k: np.ndarray,
             v: np.ndarray, slot_mapping: np.ndarray, block_size: int,
             inplace: bool = False):
    """Copy each new token's K and V into its slot; return the new pools.

    k_pool, v_pool: [num_blocks][Hkv][B][D]; k, v: [num_tokens][Hkv][D] of the
    same element type; slot_mapping: int [num_tokens].  A negative slot skips
    its token.  The copy is of raw elements, so the result is bit-exact.
    With ``inplace`` the given pools are updated and returned (no copy of a
    multi-GiB pool).
    """
    num_blocks, num_kv_heads, bs, head_dim = k_pool.shape
    if bs != block_size:
        raise ValueError("pool block size does not match block_size")
    if k.shape != (len(slot_mapping), num_kv_heads, head_dim) or v.shape != k.shape:
        raise ValueError("k/v must be [num_tokens][Hkv][D]")
    live = [int(s) for s in slot_mapping if int(s) >= 0]
    if len(set(live)) != len(live):
        raise ValueError("slot mapping repeats a slot")
    if any(s >= num_blocks * block_size for s in live):
        raise ValueError("slot outside the pool")
    k_new = k_pool if inplace else k_pool.copy()
    v_new = v_pool if inplace else v_pool.copy()
    for n, s in enumerate(slot_mapping):
        s = int(s)
        if s < 0:
            continue
        p, r = slot_location(s, block_size)
        k_new[p, :, r, :] = k[n]
        v_new[p, :, r, :] = v[n]
    return k_new, v_new


# ---------------------------------------------------------------------------
# decode attention through the block table
# ---------------------------------------------------------------------------
def gather_tokens(pool: np.ndarray, table_row, num_tokens: int,
                  block_size: int, dtype: str) -> np.ndarray:
    """float64 [T][Hkv][D]: the T cached rows of one sequence, in token order,
    each read at (p, r) = token_location(t) for t = 0 .. T-1."""
    num_blocks = pool.shape[0]
    n_blocks = blocks_for_tokens(num_tokens, block_size)
    if n_blocks > len(table_row):
        raise ValueError("context longer than the block table")
    t = np.arange(num_tokens, dtype=np.int64)
    p, r = token_location(table_row, t, block_size)
    if num_tokens and (p.min() < 0 or p.max() >= num_blocks):
        raise ValueError("block table entry outside the pool")
    # advanced indices on axes 0 and 2 -> shape [T][Hkv][D]
    return to_float64(pool[p, :, r, :], dtype)


def window_start(num_tokens: int, window) -> int:
    """First position a decoded token attends to: the last ``window`` tokens,
    the newest included (``None``: every token)."""
    if window is None:
        return 0
    return max(0, int(num_tokens) - int(window))


def gather_window(pool: np.ndarray, table_row, first: int, num_tokens: int,
                  block_size: int, dtype: str) -> np.ndarray:
    """float64 [T - first][Hkv][D]: rows of tokens first .. T-1 in token order.
    Only table entries of blocks holding those tokens are read."""
    num_blocks = pool.shape[0]
    if blocks_for_tokens(num_tokens, block_size) > len(table_row):
        raise ValueError("context longer than the block table")
    t = np.arange(first, num_tokens, dtype=np.int64)
    p, r = token_location(table_row, t, block_size)
    if t.size and (p.min() < 0 or p.max() >= num_blocks):
        raise ValueError("block table entry outside the pool")
    return to_float64(pool[p, :, r, :], dtype)


def window_blocks(num_tokens: int, window, block_size: int) -> int:
    """Blocks a sequence of T tokens needs under a sliding window: those that
    hold positions window_start(T) .. T-1."""
    if num_tokens <= 0:
        return 0
    first = window_start(num_tokens, window)
    return (num_tokens - 1) // block_size - first // block_size + 1


def attend(q_h: np.ndarray, keys: np.ndarray, values: np.ndarray,
           scale: float) -> np.ndarray:
    """softmax(scale * keys . q_h) . values for one query row, in float64.

    q_h: [D]; keys, values: [T][D].  The maximum score is subtracted before the
    exponential (an identity that keeps exp finite)."""
    scores = scale * (keys @ q_h)
    weights = np.exp(scores - scores.max())
    return (weights @ values) / weights.sum()


def decode(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
           block_tables: np.ndarray, context_lens, scale: float,
           dtype: str, seqs=None, window=None, kv_dtype=None, k_scale: float = 1.0,
           v_scale: float = 1.0) -> np.ndarray:
    """Decode-step attention for every (sequence, query head); float64 out.

    q: [N][Hq][D]; pools: [num_blocks][Hkv][B][D]; block_tables: int [N][MB];
    context_lens: int [N] (T_i counts the newest token, whose K/V is already in
    the pool).  ``seqs`` restricts the work to some sequences (their rows of the
    result are filled, the others are left NaN) for sampled checks at full size.
    ``window``: a sliding window of that many tokens (None: full attention).
    ``kv_dtype``: the pools' element type when it differs from q's (FP8 pools,
    "fp8e4m3", hold codes whose values are multiplied by k_scale / v_scale).
    """
    num_seqs, num_q_heads, head_dim = q.shape
    _, num_kv_heads, block_size, pool_dim = k_pool.shape
    if pool_dim != head_dim or v_pool.shape != k_pool.shape:
        raise ValueError("q, k_pool and v_pool disagree on shapes")
    if num_q_heads % num_kv_heads:
        raise ValueError("query heads must be a multiple of kv heads")
    sc = float(np.float32(scale))
    out = np.full((num_seqs, num_q_heads, head_dim), np.nan, dtype=np.float64)
    q64 = to_float64(q, dtype)
    todo = range(num_seqs) if seqs is None else seqs
    for i in todo:
        T = int(context_lens[i])
        if T == 0:
            out[i] = 0.0
            continue
        pool_dtype = dtype if kv_dtype is None else kv_dtype
        if window is None:
            keys = gather_tokens(k_pool, block_tables[i], T, block_size, pool_dtype)
            values = gather_tokens(v_pool, block_tables[i], T, block_size, pool_dtype)
        else:
            first = window_start(T, window)
            keys = gather_window(k_pool, block_tables[i], first, T, block_size, pool_dtype)
            values = gather_window(v_pool, block_tables[i], first, T, block_size, pool_dtype)
        if kv_dtype is not None:
            keys = keys * float(np.float32(k_scale))
            values = values * float(np.float32(v_scale))
        for h in range(num_q_heads):
            g = kv_head_for_query_head(h, num_q_heads, num_kv_heads)
            out[i, h] = attend(q64[i, h], keys[:, g, :], values[:, g, :], sc)
    return out


def query_position(num_tokens: int, num_queries: int, r: int) -> int:
    """Position of query row r of a chunk that ends the sequence's T tokens."""
    return int(num_tokens) - int(num_queries) + int(r)


def causal_keys(position: int) -> int:
    """Keys a query at this position attends to: positions 0 .. position."""
    return int(position) + 1


def prefill(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
            block_tables: np.ndarray, context_lens, query_lens, scale: float,
            dtype: str) -> np.ndarray:
    """Causal attention of each sequence's last M_i tokens (a prompt chunk, or
    one decode token) over its cached tokens; float64 out.

    q: [sum M_i][Hq][D], sequence i's rows consecutive (sequence order);
    context_lens: T_i, counting the chunk; query_lens: M_i, 0 <= M_i <= T_i.
    """
    num_rows, num_q_heads, head_dim = q.shape
    _, num_kv_heads, block_size, pool_dim = k_pool.shape
    if pool_dim != head_dim or v_pool.shape != k_pool.shape:
        raise ValueError("q, k_pool and v_pool disagree on shapes")
    if num_q_heads % num_kv_heads:
        raise ValueError("query heads must be a multiple of kv heads")
    lens = [int(x) for x in context_lens]
    mq = [int(x) for x in query_lens]
    if sum(mq) != num_rows or any(m < 0 or m > T for m, T in zip(mq, lens)):
        raise ValueError("query lengths do not match q, or exceed the context")
    sc = float(np.float32(scale))
    q64 = to_float64(q, dtype)
    out = np.zeros((num_rows, num_q_heads, head_dim), dtype=np.float64)
    row = 0
    for i, (T, M) in enumerate(zip(lens, mq)):
        if M:
            keys = gather_tokens(k_pool, block_tables[i], T, block_size, dtype)
            values = gather_tokens(v_pool, block_tables[i], T, block_size, dtype)
        for r in range(M):
            n = causal_keys(query_position(T, M, r))
            for h in range(num_q_heads):
                g = kv_head_for_query_head(h, num_q_heads, num_kv_heads)
                out[row + r, h] = attend(q64[row + r, h], keys[:n, g, :], values[:n, g, :], sc)
        row += M
    return out


# ---------------------------------------------------------------------------
# byte and block accounting
# ---------------------------------------------------------------------------
def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int,
                       dtype_bytes: int) -> int:
    """2 (key and value) x layers x kv heads x head_dim x bytes per element
    (sudo.vn page, "How big the KV cache is: a formula and a real
    measurement")."""
    return 2 * layers * kv_heads * head_dim * dtype_bytes


def block_bytes(layers: int, block_size: int, kv_heads: int, head_dim: int,
                dtype_bytes: int) -> int:
    """Bytes of one block across all layers, K and V
    ("How is vLLM's KV cache paged?", pool set-up)."""
    return 2 * layers * block_size * kv_heads * head_dim * dtype_bytes


def kv_bytes_read(context_lens, kv_heads: int, head_dim: int,
                  dtype_bytes: int) -> int:
    """KV bytes one decode step must read for one layer: every cached token's
    K and V once per kv head (the step-time model in "How does vLLM's
    scheduling achieve both minimal latency and maximum throughput?" charges
    every cached token)."""
    total_tokens = int(np.sum(np.asarray(context_lens, dtype=np.int64)))
    return 2 * kv_heads * head_dim * dtype_bytes * total_tokens


def wasted_slots_paged(context_lens, block_size: int) -> int:
    """Allocated but unused slots with paging: sum of ceil(T/B)*B - T
    ("What operations can cause memory fragmentation ...")."""
    return sum(blocks_for_tokens(T, block_size) * block_size - int(T)
               for T in context_lens)


def wasted_slots_contiguous(context_lens, max_len: int) -> int:
    """Reserved but unused slots when every request reserves max_len."""
    return sum(int(max_len) - int(T) for T in context_lens)


def static_batch_useful_fraction(prompts, outputs) -> float:
    """sum(p_i + o_i) / (n * (max p + max o)) ("Why is batching multiple
    requests difficult for traditional inference engines?")."""
    n = len(prompts)
    return (sum(prompts) + sum(outputs)) / (n * (max(prompts) + max(outputs)))
