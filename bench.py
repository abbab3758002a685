"""Paged decode-attention benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 3] [--gpus 1]

One step is the whole hot path for one decode batch.  Where the batch writes
new tokens (configurations 3 and 5) that is pa_append_decode: each sequence's
newest K/V rows go into the pools and the attention reads them, in one call
(the stream kernel plus the piece merge, which also writes the rows).  The
same step as two calls, pa_write_kv then pa_decode, is timed beside it and
reported as "two_call".  Other configurations decode only (pa_decode).
With --fp8 the pools hold FP8 (E4M3) codes and the step is
pa_append_decode_fp8 (two calls: pa_write_kv_fp8 then pa_decode_fp8).
Inputs are resident in HBM before timing starts.  To keep the timed reads
cold in the GPU caches, steps rotate over several copies of the pools
(together well above the 256 MB Infinity Cache).

Printed: one JSON line with the metric (KV bytes read per second, TB/s, over
the whole step), the roofline of the attention kernel (KV bytes over its mean
duration, timed by HIP events attached to its own dispatch), the whole decode
call's time, and the CPU oracle timed on a bounded sample as a baseline.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, vendor figure

WORKLOAD_NAMES = {
    1: "tiny-decode-f32: 4 seqs, 4q/4kv heads, d64, B4, lens [7,8,9,8]",
    2: "qwen2-0.5b-decode-f16: 32 seqs, 14q/2kv heads, d64, B16, lens U{1..4096}",
    3: "llama3-8b-decode-bf16: 256 seqs, 32q/8kv heads, d128, B16, lognormal lens mean~400 cap 4096, 256 new tokens written",
    4: "llama2-7b-decode-f16: 64 seqs, 32q/32kv heads, d128, B16, every len 4096",
    5: "prefix-shared-decode-bf16: 12 seqs, 64q/8kv heads, d128, B16, 1800-token shared prefix + U{0..512} + 1",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--partition", type=int, default=0, help="partition tokens (0 = library choice)")
    ap.add_argument("--step", choices=("both", "append", "two-call"), default="both",
                    help="where the batch writes new tokens: time the one-call step "
                         "(pa_append_decode, or pa_append_decode_fp8 with --fp8; the headline) "
                         "and the two calls (both), or only one of them")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window in tokens (pa_decode_sliding; 0 = full attention)")
    ap.add_argument("--prefill", type=int, default=0,
                    help="chunked prefill instead of decode: every sequence of the first 16 of "
                         "the Llama-3-8B batch gets a chunk of this many new tokens (pa_prefill)")
    ap.add_argument("--cow", type=int, default=0,
                    help="copy-on-write instead of decode: one pa_copy_blocks launch copying "
                         "this many shared blocks in all 64 pools of Llama-3-8B (32 layers, K "
                         "and V), plus the host block manager's cost for the same batch")
    ap.add_argument("--fp8", action="store_true",
                    help="FP8 (E4M3) pools with per-pool scales: pa_append_decode_fp8 (two calls: "
                         "pa_write_kv_fp8 + pa_decode_fp8)")
    ap.add_argument("--replicas", type=int, default=0, help="pool copies to rotate (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the streaming-read ceiling (pa_stream_read of 2 GiB) in the line")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 512 MiB buffer 10 times (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


def copy_calibration():
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    n = 512 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": 10}), flush=True)


# State the oracle workers read: set in the parent before the pool forks, so
# the children share the arrays (copy-on-write) instead of receiving copies.
_ORACLE = {}


def _oracle_rows(seqs):
    """Worker: the oracle's decode of some sequences (their output rows)."""
    import oracle.paged_attention_ref as ref
    st = _ORACLE
    w = st["w"]
    out = ref.decode(w.q, st["k"], st["v"], w.block_tables, w.context_lens, w.scale, w.dtype,
                     seqs=seqs, window=st["window"] or None,
                     kv_dtype="fp8e4m3" if st["fp8"] else None,
                     k_scale=st["fp8"][0] if st["fp8"] else 1.0,
                     v_scale=st["fp8"][1] if st["fp8"] else 1.0)
    return out[seqs]


def _oracle_prefill(i):
    """Worker: the oracle's prefill of sequence i's chunk (its flops)."""
    import oracle.paged_attention_ref as ref
    st = _ORACLE
    M, lens = st["M"], st["lens"]
    ref.prefill(st["q"][i * M:(i + 1) * M], st["k"], st["v"], st["w"].block_tables[i:i + 1],
                [lens[i]], [M], st["w"].scale, "bf16")
    return 4 * 32 * 128 * sum(lens[i] - M + r + 1 for r in range(M))


def _oracle_write(w, fp8_scales, kc=None, vc=None):
    import oracle.paged_attention_ref as ref
    if fp8_scales:
        return ref.write_kv_fp8(kc, vc, w.new_k, w.new_v, w.slot_mapping, w.block_size, w.dtype,
                                *fp8_scales)
    return ref.write_kv(w.k_pool, w.v_pool, w.new_k, w.new_v, w.slot_mapping, w.block_size)


def cpu_baseline(w, budget_s: float, kv_bytes: int, window: int = 0, fp8_scales=None):
    """The oracle as it stands (the slot write, then the decode), on the same
    host arrays.  All cores: each step's decode is spread over a pool of
    processes (one BLAS thread each), forked before the GPU is touched; steps
    repeat until half the budget is spent.  One core: the same code on one
    process, one whole sequence at a time in shuffled passes over the batch,
    for the other half.  Returns
    (TB/s all cores, cores, TB/s one core, sample description)."""
    import multiprocessing as mp

    import numpy as np

    import oracle.paged_attention_ref as ref
    from threadpoolctl import threadpool_limits
    n = w.num_seqs
    kc = vc = None
    if fp8_scales:
        kc = ref.quantize_fp8(w.k_pool, w.dtype, fp8_scales[0])
        vc = ref.quantize_fp8(w.v_pool, w.dtype, fp8_scales[1])
    with threadpool_limits(1):
        k, v = _oracle_write(w, fp8_scales, kc, vc)
    _ORACLE.update(w=w, k=k, v=v, window=window, fp8=fp8_scales)
    cores = max(1, min(16, len(os.sched_getaffinity(0)), n))
    # about equal work per task: sequences dealt out longest first
    order = np.argsort(-np.asarray(w.context_lens), kind="stable")
    tasks = [np.sort(order[i::cores * 2]) for i in range(cores * 2)]
    tasks = [t for t in tasks if len(t)]
    steps, secs = 0, 0.0
    with threadpool_limits(1):
        ctx = mp.get_context("fork")
        with ctx.Pool(cores) as pool:
            pool.map(_oracle_rows, tasks[:cores])            # workers up
            while secs < budget_s / 2:
                t0 = time.perf_counter()
                _oracle_write(w, fp8_scales, kc, vc)
                pool.map(_oracle_rows, tasks)
                secs += time.perf_counter() - t0
                steps += 1
        all_tbps = kv_bytes * steps / secs / 1e12
        # one core: whole sequences until the other half of the budget is spent
        done_bytes, one_secs, done = 0, 0.0, 0
        lens = np.asarray(w.context_lens, dtype=np.int64)
        attended = np.minimum(lens, window) if window > 0 else lens
        per_token = kv_bytes / max(1, int(attended.sum()))
        rng = np.random.default_rng(0)
        while one_secs < budget_s / 2:
            for i in rng.permutation(n):
                t0 = time.perf_counter()
                _oracle_rows(np.array([i]))
                one_secs += time.perf_counter() - t0
                done_bytes += per_token * int(attended[i])
                done += 1
                if one_secs >= budget_s / 2:
                    break
    one_tbps = done_bytes / one_secs / 1e12
    sample = (f"all cores: {steps} full steps (write + decode of all {n} sequences) in "
              f"{secs:.1f} s over {cores} processes; one core: {done} single-sequence decodes "
              f"(the {n} sequences in shuffled passes) in {one_secs:.1f} s")
    return all_tbps, cores, one_tbps, sample


PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "decode_stream_llama3-8b-bf16.json")
COPY_PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "copy_blocks_llama3-8b-cow256-bf16.json")
PREFILL_PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "prefill_llama3-8b-chunk512-bf16.json")


def summary_traffic(path, sources):
    """HBM bytes per launch of a kernel from a committed rocprofv3 counter
    summary, or None when the summary does not describe the kernel as built
    now (it records the sha256 of the kernel's source files, concatenated in
    the order given)."""
    import hashlib
    if not os.path.exists(path):
        return None, None
    with open(path) as f:
        prof = json.load(f)
    h = hashlib.sha256()
    for source in sources:
        with open(os.path.join(ROOT, "paged_kv_cache_75_amd", "csrc", source), "rb") as f:
            h.update(f.read())
    sha = h.hexdigest()
    if sha != prof.get("kernel_source_sha256"):
        return None, None
    return prof["traffic_bytes_per_launch"], prof


DECODE_SOURCES = ("pa_device.h", "pa_kernels.hip")
WINDOW_PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "decode_sliding_llama3-8b-w256-bf16.json")
FP8_PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "decode_fp8_llama3-8b-e4m3.json")
C4_PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "decode_stream_llama2-7b-f16.json")
C5_PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "decode_stream_prefix-shared-bf16.json")


def profiled_summary(cfg, fused, window, fp8, partition):
    """The committed counter summary of the attention kernel a bench line
    measures, for the workloads that were profiled (configuration 3: the
    appending step, the 256-token window, FP8 pools; configuration 4;
    configuration 5's appending step), else None."""
    if partition:
        return None
    if cfg == 4 and not (window or fp8):
        return C4_PROFILE_SUMMARY
    if cfg == 5 and fused and not (window or fp8):
        return C5_PROFILE_SUMMARY
    if cfg != 3:
        return None
    if fp8:
        return FP8_PROFILE_SUMMARY
    if window:
        return WINDOW_PROFILE_SUMMARY if window == 256 else None
    return PROFILE_SUMMARY if fused else None


def kv_bytes_per_step(w, window: int = 0) -> int:
    """Algorithmic KV bytes of one decode step: every attended token's K and V
    row, once per kv head (with a sliding window, the last `window` tokens of
    each sequence)."""
    import numpy as np
    lens = w.context_lens.astype("int64")
    if window:
        lens = np.minimum(lens, window)
    return 2 * w.num_kv_heads * w.head_dim * w.elem_bytes * int(lens.sum())


def unique_kv_bytes(w, window: int = 0) -> int:
    """KV bytes of the distinct pool rows a step attends over: a row that
    several sequences reach through shared blocks counts once."""
    import numpy as np
    rows = set()
    B = w.block_size
    for i, T in enumerate(w.context_lens.astype(int)):
        first = max(0, T - window) if window else 0
        t = np.arange(first, T)
        rows.update((w.block_tables[i, t // B].astype(np.int64) * B + t % B).tolist())
    return 2 * w.num_kv_heads * w.head_dim * w.elem_bytes * len(rows)


def prefill_main(args):
    """Chunked prefill: each of 16 Llama-3-8B-shaped sequences (the first 16
    lengths of the decode batch, seed 3) gets a chunk of args.prefill new
    tokens.  Step = pa_write_kv of every chunk token + pa_prefill.  Work unit:
    one (query row, attended key) pair per query head, 4 * D flops (QK^T and
    P.V); bound by the matrix cores."""
    import numpy as np
    import torch

    import workloads
    from workloads.generate import round_to_dtype
    from paged_kv_cache_75_amd import (pa_prefill, pa_profile_start, pa_profile_stop,
                                       pa_write_kv)
    M = args.prefill
    base = workloads.make(3, seed=3, poison=False).context_lens[:16]
    lens = [int(T) + M for T in base]
    w = workloads.random_paged("llama3-8b-prefill", "bf16", 32, 8, 128, 16, lens, seed=args.seed or 3,
                               poison=False)
    rng = np.random.default_rng(11)
    n = len(lens)
    q = round_to_dtype(rng.standard_normal((n * M, 32, 128)).astype(np.float32), "bf16")
    ck = round_to_dtype(rng.standard_normal((n * M, 8, 128)).astype(np.float32), "bf16")
    cv = round_to_dtype(rng.standard_normal((n * M, 8, 128)).astype(np.float32), "bf16")
    slots = np.array([int(w.block_tables[i, t // 16]) * 16 + t % 16
                      for i, T in enumerate(lens) for t in range(T - M, T)], dtype=np.int32)

    # the oracle first, on all host cores (a pool forked before the GPU is
    # touched: chunks dealt out whole, one BLAS thread each), then on one core
    cpu = None
    if not args.no_cpu_baseline:
        import multiprocessing as mp

        import oracle.paged_attention_ref as ref
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1):
            k, v = ref.write_kv(w.k_pool, w.v_pool, ck, cv, slots, 16)
            _ORACLE.update(w=w, k=k, v=v, q=q, M=M, lens=lens)
            cores = max(1, min(16, len(os.sched_getaffinity(0)), n))
            order = sorted(range(n), key=lambda i: -lens[i])       # longest first
            done, secs, passes = 0, 0.0, 0
            with mp.get_context("fork").Pool(cores) as pool:
                while secs < args.cpu_seconds / 2:
                    t = time.perf_counter()
                    done += sum(pool.map(_oracle_prefill, order, chunksize=1))
                    secs += time.perf_counter() - t
                    passes += 1
            one_done, one_secs, one_n = 0, 0.0, 0
            while one_secs < args.cpu_seconds / 2:
                for i in range(n):
                    t = time.perf_counter()
                    one_done += _oracle_prefill(i)
                    one_secs += time.perf_counter() - t
                    one_n += 1
                    if one_secs >= args.cpu_seconds / 2:
                        break
        cpu = {"value": round(done / secs / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
               "kind": "oracle", "one_core_value": round(one_done / one_secs / 1e12, 6),
               "sample": f"all cores: {passes} passes over the {n} chunks in {secs:.1f} s over "
                         f"{cores} processes; one core: {one_n} chunks in {one_secs:.1f} s"}
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(a, bf16):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if bf16 else torch.from_numpy(a)
        return t.to(dev)

    dq, dck, dcv, dslots = up(q, True), up(ck, True), up(cv, True), up(slots, False)
    kp, vp = up(w.k_pool, True), up(w.v_pool, True)
    bt, cl = up(w.block_tables.astype(np.int32), False), up(np.array(lens, np.int32), False)
    qs = up(np.arange(0, (n + 1) * M, M, dtype=np.int32), False)
    out = torch.empty_like(dq)
    maxlen = max(lens)

    def step():
        pa_write_kv(dck, dcv, dslots, kp, vp)
        pa_prefill(dq, kp, vp, bt, cl, qs, w.scale, out=out, max_context_len=maxlen,
                   max_query_len=M)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    pa_profile_start()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    launches, kernel_us = pa_profile_stop()
    pairs = sum(T - M + r + 1 for T in lens for r in range(M))       # (query, key) pairs
    flops = 4 * 32 * 128 * pairs
    kv_bytes = 2 * 8 * 128 * 2 * sum(lens)
    achieved = flops / (kernel_us * 1e-6) / 1e12
    traffic_bytes, _ = (summary_traffic(PREFILL_PROFILE_SUMMARY, ("pa_device.h", "pa_prefill.hip"))
                        if M == 512 else (None, None))
    result = {
        "metric": "chunked prefill attention: TFLOP/s (bf16 matrix cores), us/step",
        "value": round(flops / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "us_per_step": round(ms * 1e3, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"llama3-8b-prefill-bf16: 16 seqs, 32q/8kv heads, d128, B16, "
                               f"a {M}-token chunk after each of the first 16 decode-batch contexts",
                   "query_rows": n * M, "attended_pairs_per_head": pairs,
                   "flops_per_step": flops, "kv_bytes_per_step": kv_bytes,
                   "step_calls": "pa_write_kv (chunk tokens) + pa_prefill"},
        "roofline": {"bound": "mfma", "kernel": "prefill_kernel (attention kernel of pa_prefill)",
                     "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None if traffic_bytes is None else round(traffic_bytes),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                     "copy-calibrated)",
                     "traffic_source": (os.path.relpath(PREFILL_PROFILE_SUMMARY, ROOT)
                                        if traffic_bytes is not None else None),
                     "kernel_us_mean": round(kernel_us, 2),
                     "kernel_launches_timed": launches},
    }
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


def cow_main(args):
    """Copy-on-write: N sequences each write into a block they share, so N
    (source, destination) block pairs are copied in every pool of the model:
    32 layers x (K, V) = 64 pools of [2048][8][16][128] bf16 (32 KiB per
    block).  Step = one pa_copy_blocks launch; unit: bytes moved (each block
    read once and written once).  Steps rotate over several pair sets so
    the reads stay cold in the caches.  The native block manager's host time
    for the batch that produces the pairs is reported beside it."""
    import numpy as np
    import torch

    import oracle.block_manager_ref as bm_ref
    from paged_kv_cache_75_amd import (BlockManager, PoolSet, pa_copy_blocks, pa_profile_start,
                                       pa_profile_stop)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    N = args.cow
    layers, nb, hkv, bs, hd = 32, 2048, 8, 16, 128
    if 2 * N > nb:
        sys.exit(f"--cow {N}: at most {nb // 2} pairs")
    block_bytes = hkv * bs * hd * 2
    pools = [torch.empty((nb, hkv, bs, hd), dtype=torch.bfloat16, device=dev)
             for _ in range(2 * layers)]
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed or 7)
    for p in pools:
        p.normal_(generator=g)
    moved = 2 * N * len(pools) * block_bytes                  # read + write per launch
    sets = max(1, min(16, -(-(2 << 30) // moved)))
    rng = np.random.default_rng(args.seed or 7)
    maps = []
    for _ in range(sets):
        perm = rng.permutation(nb)
        maps.append(torch.from_numpy(np.stack([perm[N:2 * N], perm[:N]], 1).astype(np.int32))
                    .to(dev))

    pool_set = PoolSet(pools)

    def step(k):
        pa_copy_blocks(pool_set, maps[k % sets])

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    pa_profile_start()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    launches, kernel_us = pa_profile_stop()
    assert launches == args.steps, (launches, args.steps)
    # a torch device copy of the same byte count, timed the same way, as the
    # practical ceiling of a copy on this GPU
    src = torch.empty(moved // 2, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(3)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    torch_copy_us = e0.elapsed_time(e1) * 1e3 / 10
    del src, dst
    # the last launch copied maps[(steps - 1) % sets]: destinations equal sources
    last = maps[(args.steps - 1) % sets].long()
    for p in (pools[0], pools[-1]):
        assert torch.equal(p[last[:, 1]], p[last[:, 0]]), "copied blocks differ from sources"

    # the host side of the same batch: N sequence pairs (a prompt of ~400
    # tokens and a fork of it); one member of each pair appends a token into
    # the shared partial block (N copy-on-write pairs), then 15 plain batches
    prompt_rng = np.random.default_rng(5)
    prompts = [prompt_rng.integers(0, 32000, 400 + i % 7 + 1) for i in range(N)]
    seqs = np.arange(0, 2 * N, 2)
    cow_s, plain_s, plain_n = 0.0, 0.0, 0
    for _ in range(10):
        m = BlockManager(2 * N * 32 + 64, bs)
        for i in range(N):
            m.allocate(2 * i, prompts[i])
            m.fork(2 * i, 2 * i + 1)
        t = time.perf_counter()
        _, pairs = m.append(seqs, np.full(N, 11))
        cow_s += time.perf_counter() - t
        assert len(pairs) == N
        for _ in range(15):
            t = time.perf_counter()
            m.append(seqs, np.full(N, 12))
            plain_s += time.perf_counter() - t
            plain_n += 1
    sys_prompt = prompt_rng.integers(0, 32000, 1800)
    m2 = BlockManager(8192, bs)
    m2.allocate(0, np.concatenate([sys_prompt, [1]]))
    t = time.perf_counter()
    for i in range(1, 101):
        assert m2.allocate(i, np.concatenate([sys_prompt, [i + 1]])) == 112 * bs
    alloc_us = (time.perf_counter() - t) * 1e6 / 100

    achieved = moved / (kernel_us * 1e-6) / 1e9
    traffic_bytes, _ = summary_traffic(COPY_PROFILE_SUMMARY, ("pa_copy.hip",)) if N == 256 else (None, None)
    result = {
        "metric": "copy-on-write block copy: bytes moved/s (TB/s, read + write), us/step",
        "value": round(moved / (ms * 1e-3) / 1e12, 4),
        "unit": "TB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "us_per_step": round(ms * 1e3, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"llama3-8b-cow-bf16: {N} block pairs x 64 pools (32 layers x K/V) "
                               f"of [2048][8][16][128], 32 KiB per block",
                   "pairs": N, "pools": len(pools), "block_bytes": block_bytes,
                   "bytes_moved_per_step": moved, "pair_sets_rotated": sets,
                   "step_calls": "pa_copy_blocks"},
        "roofline": {"bound": "hbm", "kernel": "copy_blocks_kernel (pa_copy_blocks)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic_bytes is None else round(traffic_bytes),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                     "copy-calibrated)",
                     "traffic_source": (os.path.relpath(COPY_PROFILE_SUMMARY, ROOT)
                                        if traffic_bytes is not None else None),
                     "kernel_us_mean": round(kernel_us, 2), "kernel_launches_timed": launches,
                     "torch_copy_same_bytes_us": round(torch_copy_us, 2),
                     "torch_copy_GBps": round(moved / (torch_copy_us * 1e-6) / 1e9, 1)},
        "host_block_manager": {
            "append_batch_cow_us": round(cow_s * 1e6 / 10, 2),
            "append_batch_us": round(plain_s * 1e6 / plain_n, 2),
            "append_batch": f"{N} sequences, one token each; the copy-on-write batch has every "
                            f"sequence write into a block it shares with a fork ({N} pairs)",
            "allocate_prefix_hit_us": round(alloc_us, 2),
            "allocate": "1801-token prompt, 112 of 113 blocks hit (1800-token shared prefix)",
        },
    }
    if not args.no_cpu_baseline:
        # the oracle's block copy on host pools of the same block shape (64
        # pools of 4 * N blocks), N pairs per call, one thread
        host = [np.zeros((2 * N + 2, hkv, bs, hd), np.uint16) for _ in range(2 * layers)]
        pairs = [(i, N + i) for i in range(N)]
        done, secs, calls = 0, 0.0, 0
        while secs < min(args.cpu_seconds, 10.0):
            t = time.perf_counter()
            bm_ref.copy_blocks(host, pairs, inplace=True)
            secs += time.perf_counter() - t
            done += moved
            calls += 1
        result["cpu_baseline"] = {"value": round(done / secs / 1e12, 6), "unit": "TB/s",
                                  "cores": 1, "kind": "oracle",
                                  "sample": f"{calls} calls of the oracle's copy_blocks, {N} pairs "
                                            f"x 64 host pools, {secs:.1f} s"}
    print(json.dumps(result), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads
    from paged_kv_cache_75_amd import (fp8_pool_desc, pa_append_decode, pa_append_decode_fp8,
                                       pa_decode, pa_decode_fp8, pa_decode_partitioned,
                                       pa_decode_partitioned_workspace_bytes, pa_decode_sliding,
                                       pa_profile_start, pa_profile_stop, pa_stream_read,
                                       pa_write_kv, pa_write_kv_fp8, pool_desc)

    # torch.cuda.device_count() does not start the GPU runtime: the oracle's
    # worker processes below are forked before anything touches the GPU
    if torch.cuda.device_count() < 1:
        sys.exit("bench.py needs a GPU")
    if args.prefill:
        prefill_main(args)
        return
    if args.cow:
        cow_main(args)
        return
    cfg = args.config
    seed = cfg if args.seed is None else args.seed
    w = workloads.make(cfg, seed=seed, poison=False)
    ks = vs = 4.0 / 448.0              # FP8 pools: about +-4 maps to the top of E4M3
    kv_bytes = kv_bytes_per_step(w, args.window) // (w.elem_bytes if args.fp8 else 1)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds, kv_bytes, args.window,
                           (ks, vs) if args.fp8 else None)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(a, dt):
        a = np.ascontiguousarray(a)
        if dt == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    q = up(w.q, w.dtype)
    bt = up(w.block_tables.astype(np.int32), None)
    cl = up(w.context_lens.astype(np.int32), None)
    slots = up(w.slot_mapping.astype(np.int32), None)
    nk, nv = up(w.new_k, w.dtype), up(w.new_v, w.dtype)
    k0, v0 = up(w.k_pool, w.dtype), up(w.v_pool, w.dtype)
    if args.fp8:
        # every slot of the pools quantized on the GPU by the slot write
        nb, hkv, bsz, hd = (int(x) for x in k0.shape)
        allslots = torch.arange(nb * bsz, dtype=torch.int32, device=dev)
        kq = torch.empty(k0.shape, dtype=torch.uint8, device=dev)
        vq = torch.empty_like(kq)
        pa_write_kv_fp8(k0.permute(0, 2, 1, 3).reshape(-1, hkv, hd).contiguous(),
                        v0.permute(0, 2, 1, 3).reshape(-1, hkv, hd).contiguous(), allslots,
                        kq, vq, ks, vs)
        torch.cuda.synchronize()
        k0, v0 = kq, vq
    pool_bytes = 2 * k0.numel() * k0.element_size()
    reps = args.replicas or max(1, min(8, -(-(1 << 30) // pool_bytes) + 1))
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(reps - 1)]
    out = torch.empty_like(q)
    desc = fp8_pool_desc(k0, q) if args.fp8 else pool_desc(k0)
    ws_bytes = pa_decode_partitioned_workspace_bytes(w.num_seqs, w.num_q_heads, desc,
                                                     w.max_context_len, args.partition)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    writes = cfg in (3, 5)

    def decode(kp, vp):
        if args.fp8:
            pa_decode_fp8(q, kp, vp, bt, cl, w.scale, ks, vs, out=out,
                          max_context_len=w.max_context_len, workspace=ws)
        elif args.window:
            pa_decode_sliding(q, kp, vp, bt, cl, w.scale, args.window, out=out,
                              max_context_len=w.max_context_len, workspace=ws,
                              partition_tokens=args.partition)
        elif args.partition:
            pa_decode_partitioned(q, kp, vp, bt, cl, w.scale, args.partition, out=out,
                                  max_context_len=w.max_context_len, workspace=ws)
        else:
            pa_decode(q, kp, vp, bt, cl, w.scale, out=out, max_context_len=w.max_context_len,
                      workspace=ws)

    def append_decode(kp, vp):
        if args.fp8:
            pa_append_decode_fp8(q, nk, nv, kp, vp, bt, cl, w.scale, ks, vs, out=out,
                                 max_context_len=w.max_context_len, workspace=ws)
        else:
            pa_append_decode(q, nk, nv, kp, vp, bt, cl, w.scale, out=out,
                             max_context_len=w.max_context_len, workspace=ws,
                             partition_tokens=args.partition)

    def timed(pre, call):
        """Step time: K steps between device synchronisations, nothing else
        on the stream.  Call time: K more steps with HIP events on the stream
        around `call` (the decode call) in each; an event record costs the
        stream a few microseconds, so the loops are kept apart.  Kernel time:
        K more steps with the library's kernel timing on (start and stop
        events attached to the attention kernel's own dispatch)."""
        for k in range(args.warmup):
            kp, vp = pools[k % reps]
            pre(kp, vp)
            call(kp, vp)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            kp, vp = pools[k % reps]
            pre(kp, vp)
            call(kp, vp)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        stream = torch.cuda.current_stream()
        for k in range(args.steps):
            kp, vp = pools[k % reps]
            pre(kp, vp)
            ev[k][0].record(stream)
            call(kp, vp)
            ev[k][1].record(stream)
        torch.cuda.synchronize()
        pa_profile_start()
        for k in range(args.steps):
            kp, vp = pools[k % reps]
            pre(kp, vp)
            call(kp, vp)
        torch.cuda.synchronize()
        launches, kernel_us = pa_profile_stop()
        assert launches == args.steps, (launches, args.steps)
        # warm: the same steps on one copy of the pools, back to back (what the
        # 256 MB Infinity Cache holds of them is then read from it)
        kp, vp = pools[0]
        for _ in range(3):
            pre(kp, vp)
            call(kp, vp)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for _ in range(args.steps):
            pre(kp, vp)
            call(kp, vp)
        torch.cuda.synchronize()
        warm_ms = (time.perf_counter() - t2) * 1e3 / args.steps
        return ((t1 - t0) * 1e3 / args.steps, [a.elapsed_time(b) for a, b in ev], kernel_us,
                warm_ms)

    def write(kp, vp):
        if args.fp8:
            pa_write_kv_fp8(nk, nv, slots, kp, vp, ks, vs)
        else:
            pa_write_kv(nk, nv, slots, kp, vp)

    def nothing(kp, vp):
        pass

    K = args.steps
    fused = writes and args.step != "two-call" and not args.window
    two_call = writes and args.step != "append"
    if two_call:
        two_ms, two_decode_ms, two_kernel_us, two_warm_ms = timed(write, decode)
    if fused:
        ms_per_step, decode_ms, kernel_us, warm_ms = timed(nothing, append_decode)
    elif writes:
        ms_per_step, decode_ms, kernel_us, warm_ms = two_ms, two_decode_ms, two_kernel_us, two_warm_ms
    else:
        ms_per_step, decode_ms, kernel_us, warm_ms = timed(nothing, decode)

    # the measured read ceiling: one streaming read of 2 GiB, timed like the
    # attention kernel (events attached to its dispatch), best of 10
    ceiling = None
    if not args.no_read_ceiling:
        buf = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
        buf.fill_(7)
        sink = torch.zeros(4, dtype=torch.int32, device=dev)
        for _ in range(3):
            pa_stream_read(buf, sink)
        runs = []
        for _ in range(10):
            pa_profile_start()
            pa_stream_read(buf, sink)
            torch.cuda.synchronize()
            runs.append(pa_profile_stop()[1])
        del buf
        ceiling = {"TBps": round((2 << 30) / (min(runs) * 1e-6) / 1e12, 4),
                   "TBps_median": round((2 << 30) / (float(np.median(runs)) * 1e-6) / 1e12, 4),
                   "bytes": 2 << 30,
                   "kernel": "stream_read_kernel (pa_stream_read: every byte read once, "
                             "16-byte non-temporal loads, four in flight per thread)"}

    balanced = args.partition == 0 and w.dtype != "f32" and w.block_size >= 16 and w.num_seqs <= 1024
    attention_kernel = "decode_stream_kernel" if balanced else "decode_partition_kernel"
    decode_ms_mean = sum(decode_ms) / len(decode_ms)
    call_us = np.array(decode_ms) * 1e3
    # bytes the HBM must supply: a block shared by several sequences (a
    # common prefix) is one block of memory, read once per kv head however
    # many sequences attend over it; the metric's KV bytes count it once per
    # sequence (the "effective" rate)
    unique_bytes = unique_kv_bytes(w, args.window) // (w.elem_bytes if args.fp8 else 1)
    roof_bytes = unique_bytes if unique_bytes < kv_bytes else kv_bytes
    achieved = roof_bytes / (kernel_us * 1e-6) / 1e9
    value = kv_bytes / (ms_per_step * 1e-3) / 1e12

    summary = profiled_summary(cfg, fused, args.window, args.fp8, args.partition)
    traffic_bytes, prof = summary_traffic(summary, DECODE_SOURCES) if summary else (None, None)
    traffic = None if traffic_bytes is None else round(traffic_bytes)
    result = {
        "metric": "paged decode attention: KV bytes read/s (TB/s), % HBM peak, us/step",
        "value": round(value, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "pct_hbm_peak": round(100 * value * 1e3 / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_NAMES[cfg] + (f", sliding window {args.window}" if args.window else "")
                        + (", FP8 (E4M3) pools" if args.fp8 else ""),
            "seed": seed,
            "num_seqs": w.num_seqs,
            "sum_context_tokens": int(w.context_lens.sum()),
            "max_context_len": w.max_context_len,
            "kv_bytes_per_step": kv_bytes,
            "kv_bytes_unique_per_step": unique_bytes,
            "new_tokens_written": int((w.slot_mapping >= 0).sum()) if writes else 0,
            "pool_copies_rotated": reps,
            "partition_tokens": args.partition or "auto",
            "step_calls": (("pa_append_decode_fp8" if args.fp8 else "pa_append_decode") if fused else
                           ("pa_write_kv_fp8 + pa_decode_fp8" if args.fp8 else
                            ("pa_write_kv + " if writes else "") +
                            ("pa_decode_sliding" if args.window else "pa_decode"))),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": (attention_kernel + " (attention kernel of " +
                       (("pa_append_decode_fp8" if args.fp8 else "pa_append_decode") if fused
                        else "pa_decode_fp8" if args.fp8 else
                        "pa_decode_sliding" if args.window else "pa_decode") + ")"),
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "bytes": "unique KV bytes (each shared block once)" if roof_bytes < kv_bytes
                     else "KV bytes",
            "frac_of_read_ceiling": (round(achieved / (ceiling["TBps"] * 1e3), 4)
                                     if ceiling else None),
            "traffic": traffic,
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "traffic_source": os.path.relpath(summary, ROOT) if traffic is not None else None,
            "kernel_us_mean": round(kernel_us, 2),
            "kernel_timing": "HIP start/stop events attached to the kernel's dispatch "
                             "(pa_profile_start / pa_profile_stop), mean over the steps",
            "call_us_mean": round(decode_ms_mean * 1e3, 2),
            "call_us_median": round(float(np.median(call_us)), 2),
            "call_us_p10": round(float(np.percentile(call_us, 10)), 2),
            "call_us_p90": round(float(np.percentile(call_us, 90)), 2),
            "call_TBps": round(kv_bytes / (decode_ms_mean * 1e-3) / 1e12, 4),
        },
        "warm": {"us_per_step": round(warm_ms * 1e3, 2),
                 "value": round(kv_bytes / (warm_ms * 1e-3) / 1e12, 4),
                 "note": "one copy of the pools, steps back to back (the timed steps above "
                         f"rotate over {reps} copies, cold in the 256 MB Infinity Cache)"},
        "read_ceiling": ceiling,
    }
    if roof_bytes < kv_bytes:
        result["value_is"] = ("effective: KV bytes counted once per sequence that attends over "
                              "them; shared prefix blocks are read from memory once per kv head")
        result["unique_TBps"] = round(unique_bytes / (ms_per_step * 1e-3) / 1e12, 4)
    if two_call and fused:
        result["two_call"] = {
            "calls": "pa_write_kv_fp8 + pa_decode_fp8" if args.fp8 else "pa_write_kv + pa_decode",
            "us_per_step": round(two_ms * 1e3, 2),
            "value": round(kv_bytes / (two_ms * 1e-3) / 1e12, 4),
            "decode_call_us_mean": round(sum(two_decode_ms) / len(two_decode_ms) * 1e3, 2),
            "kernel_us_mean": round(two_kernel_us, 2),
        }
    if cpu is not None:
        all_tbps, cores, one_tbps, sample = cpu
        result["cpu_baseline"] = {"value": round(all_tbps, 6), "unit": "TB/s", "cores": cores,
                                  "kind": "oracle", "sample": sample,
                                  "one_core_value": round(one_tbps, 6)}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
