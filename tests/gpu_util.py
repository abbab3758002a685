"""Helpers for the GPU parity tests: move a generated workload to the device,
run the library's step (write, then decode) and compare with the oracle."""

from __future__ import annotations

import dataclasses
import sys

import numpy as np

import oracle.paged_attention_ref as ref

# max-abs and mean-abs bars: fp16/bf16 from the stated parity target; fp32 is
# a reading (float32 accumulation of a float64-exact definition).
TOL = {"f32": (1e-5, 1e-6), "f16": (1e-2, 1e-3), "bf16": (1e-2, 1e-3)}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def to_device(arr: np.ndarray, dtype: str | None, dev):
    import torch
    arr = np.ascontiguousarray(arr)
    if dtype == "bf16":
        t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(arr)
    return t.to(dev)


def to_host(t, dtype: str) -> np.ndarray:
    """Device tensor -> the generator's host representation."""
    import torch
    t = t.detach().cpu()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def to_f64(t) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


@dataclasses.dataclass
class DeviceWorkload:
    q: object
    k_pool: object
    v_pool: object
    block_tables: object
    context_lens: object
    new_k: object
    new_v: object
    slot_mapping: object
    scale: float
    max_context_len: int


def upload(w, dev="cuda") -> DeviceWorkload:
    return DeviceWorkload(
        q=to_device(w.q, w.dtype, dev),
        k_pool=to_device(w.k_pool, w.dtype, dev),
        v_pool=to_device(w.v_pool, w.dtype, dev),
        block_tables=to_device(w.block_tables.astype(np.int32), None, dev),
        context_lens=to_device(w.context_lens.astype(np.int32), None, dev),
        new_k=to_device(w.new_k, w.dtype, dev),
        new_v=to_device(w.new_v, w.dtype, dev),
        slot_mapping=to_device(w.slot_mapping.astype(np.int32), None, dev),
        scale=w.scale,
        max_context_len=w.max_context_len,
    )


def gpu_step(dw: DeviceWorkload, partition_tokens: int = 0, write: bool = True, out=None):
    from paged_kv_cache_75_amd import pa_decode, pa_write_kv
    if write:
        pa_write_kv(dw.new_k, dw.new_v, dw.slot_mapping, dw.k_pool, dw.v_pool)
    return pa_decode(dw.q, dw.k_pool, dw.v_pool, dw.block_tables, dw.context_lens, dw.scale,
                     out=out, max_context_len=dw.max_context_len,
                     partition_tokens=partition_tokens)


def oracle_step(w, seqs=None, inplace=False):
    k, v = ref.write_kv(w.k_pool, w.v_pool, w.new_k, w.new_v, w.slot_mapping, w.block_size,
                        inplace=inplace)
    return ref.decode(w.q, k, v, w.block_tables, w.context_lens, w.scale, w.dtype, seqs=seqs), k, v


def compare(got: np.ndarray, want: np.ndarray, dtype: str, seqs=None, label: str = ""):
    """max-abs / mean-abs check on the rows the oracle computed."""
    if seqs is not None:
        got, want = got[list(seqs)], want[list(seqs)]
    assert np.isfinite(want).all(), "oracle produced non-finite values"
    assert np.isfinite(got).all(), f"{label}: GPU output has non-finite values"
    err = np.abs(got - want)
    max_tol, mean_tol = TOL[dtype]
    # one output ulp is the floor for elements whose magnitude alone puts the
    # final rounding above the bar (|o| >= 4 in bf16); reported, not hidden
    ulp = {"f32": 2.0 ** -23, "f16": 2.0 ** -10, "bf16": 2.0 ** -7}[dtype]
    bound = np.maximum(max_tol, ulp * np.exp2(np.floor(np.log2(np.maximum(np.abs(want), 1e-30)))))
    worst = float(err.max()) if err.size else 0.0
    mean = float(err.mean()) if err.size else 0.0
    say(f"  {label}: max_abs={worst:.3e} mean_abs={mean:.3e} (bars {max_tol:g}/{mean_tol:g})")
    assert (err <= bound).all(), f"{label}: max abs error {worst:.3e} > {max_tol}"
    assert mean <= mean_tol, f"{label}: mean abs error {mean:.3e} > {mean_tol}"
    return worst, mean
