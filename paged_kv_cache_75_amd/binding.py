"""Thin ctypes binding of libpa.so, with the C entry points' names.

Only argument marshalling happens here: shapes and dtypes of the torch tensors
are checked and turned into pointers and sizes, then the C function is called
on the current torch stream.  Every step of the computation runs in the HIP
kernels.  If the library has not been built, the first call raises
RuntimeError; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
import re

# PA_LIBRARY selects another build of the same library (A/B measurements)
LIB_PATH = os.environ.get("PA_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "_lib", "libpa.so")
INCLUDE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")

PA_OK = 0
PA_ERR_INVALID_ARGUMENT = 1
PA_ERR_UNSUPPORTED = 2
PA_ERR_WORKSPACE_TOO_SMALL = 3
PA_ERR_HIP = 4
PA_ERR_OUT_OF_BLOCKS = 5
PA_ERR_HOST_MEMORY = 6

PA_F32, PA_F16, PA_BF16 = 0, 1, 2

PA_CHECK_SLOT_RANGE, PA_CHECK_SLOT_DUP, PA_CHECK_LENGTH, PA_CHECK_TABLE = 1, 2, 3, 4


class PaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {pa_status_string(status)} ({status})")
        self.status = status


class pa_pool_desc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


_lib = None


def declared_functions(include_dir: str = INCLUDE_DIR) -> list[str]:
    """Names of the functions the headers under include/ declare."""
    names = set()
    for h in sorted(os.listdir(include_dir)):
        if h.endswith(".h"):
            text = open(os.path.join(include_dir, h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names.update(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def lib():
    """The loaded library (raises RuntimeError when it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libpa.so is not built ({LIB_PATH}); run __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    desc = ctypes.POINTER(pa_pool_desc)
    c_int = ctypes.c_int
    signatures = {
        "pa_write_kv": ([vp, vp, vp, i32, vp, vp, desc, vp], c_int),
        "pa_decode_workspace_bytes": ([i32, i32, desc, i32], sz),
        "pa_decode_partitioned_workspace_bytes": ([i32, i32, desc, i32, i32], sz),
        "pa_decode": ([vp, vp, vp, desc, vp, i32, vp, i32, i32, i32, ctypes.c_float,
                       vp, vp, sz, vp], c_int),
        "pa_decode_partitioned": ([vp, vp, vp, desc, vp, i32, vp, i32, i32, i32, ctypes.c_float,
                                   vp, vp, sz, i32, vp], c_int),
        "pa_decode_noalloc": ([vp, vp, vp, desc, vp, i32, vp, i32, i32, i32, ctypes.c_float,
                               vp, vp], c_int),
        "pa_decode_sliding": ([vp, vp, vp, desc, vp, i32, vp, i32, i32, i32, ctypes.c_float,
                               i32, vp, vp, sz, i32, vp], c_int),
        "pa_append_decode": ([vp, vp, vp, vp, vp, desc, vp, i32, vp, i32, i32, i32,
                              ctypes.c_float, vp, vp, sz, i32, vp], c_int),
        "pa_prefill": ([vp, vp, vp, desc, vp, i32, vp, vp, i32, i32, i32, i32, ctypes.c_float,
                        vp, vp], c_int),
        "pa_write_kv_fp8": ([vp, vp, vp, i32, vp, vp, desc, ctypes.c_float, ctypes.c_float, vp],
                            c_int),
        "pa_decode_fp8": ([vp, vp, vp, desc, vp, i32, vp, i32, i32, i32, ctypes.c_float,
                           ctypes.c_float, ctypes.c_float, vp, vp, sz, vp], c_int),
        "pa_append_decode_fp8": ([vp, vp, vp, vp, vp, desc, vp, i32, vp, i32, i32, i32,
                                  ctypes.c_float, ctypes.c_float, ctypes.c_float, vp, vp, sz, vp],
                                 c_int),
        "pa_stream_read": ([vp, sz, vp, vp], c_int),
        "pa_profile_start": ([], c_int),
        "pa_profile_stop": ([ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double)],
                            c_int),
        "pa_status_string": ([c_int], ctypes.c_char_p),
        "pa_check_scratch_bytes": ([desc], sz),
        "pa_check_inputs": ([vp, i32, vp, i32, vp, i32, i32, desc, vp, vp, vp], c_int),
        "pa_copy_blocks": ([ctypes.POINTER(vp), i32, i32, ctypes.c_int64, vp, i32, vp], c_int),
        "pa_bm_create": ([i32, i32, i32, ctypes.POINTER(vp)], c_int),
        "pa_bm_destroy": ([vp], None),
        "pa_bm_allocate": ([vp, ctypes.c_int64, vp, i32, vp, i32, vp], c_int),
        "pa_bm_append": ([vp, vp, vp, i32, vp, vp, vp], c_int),
        "pa_bm_fork": ([vp, ctypes.c_int64, ctypes.c_int64], c_int),
        "pa_bm_free": ([vp, ctypes.c_int64], c_int),
        "pa_bm_tables": ([vp, vp, i32, i32, vp, vp], c_int),
        "pa_bm_num_free": ([vp], i32),
        "pa_bm_block_info": ([vp, i32, vp, vp, vp, vp], c_int),
        "pa_bm_free_queue": ([vp, vp, i32, vp], c_int),
        "pa_sha256": ([vp, sz, vp], c_int),
    }
    # a symbol the library lacks stays undeclared: calling it raises
    # AttributeError (tests/test_abi.py checks that every one is exported)
    for name, (args, res) in signatures.items():
        if hasattr(L, name):
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
    _lib = L
    return L


def pa_status_string(status: int) -> str:
    return lib().pa_status_string(int(status)).decode()


def pa_stream_read(buf, sink, stream=None) -> None:
    """Read every byte of the device tensor ``buf`` once (the read-ceiling
    measurement); ``sink`` is a device int32/uint32 tensor of at least one
    element."""
    _check(buf, "buf")
    _check(sink, "sink", device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    st = lib().pa_stream_read(buf.data_ptr(), nbytes - nbytes % 16, sink.data_ptr(),
                              _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_stream_read")


def pa_profile_start() -> None:
    """Time the attention kernel of every decode call until pa_profile_stop."""
    st = lib().pa_profile_start()
    if st != PA_OK:
        raise PaError(st, "pa_profile_start")


def pa_profile_stop() -> tuple[int, float]:
    """Stop timing; (launches timed, their mean duration in microseconds)."""
    n, mean = ctypes.c_int32(0), ctypes.c_double(0.0)
    st = lib().pa_profile_stop(ctypes.byref(n), ctypes.byref(mean))
    if st != PA_OK:
        raise PaError(st, "pa_profile_stop")
    return int(n.value), float(mean.value)


# ---------------------------------------------------------------------------
# torch-facing marshalling
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    codes = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}
    if t.dtype not in codes:
        raise ValueError(f"unsupported element type {t.dtype}")
    return codes[t.dtype]


def pool_desc(k_pool) -> pa_pool_desc:
    if k_pool.dim() != 4:
        raise ValueError("pools are [num_blocks][num_kv_heads][block_size][head_dim]")
    nb, hkv, bs, d = (int(x) for x in k_pool.shape)
    return pa_pool_desc(nb, bs, hkv, d, dtype_code(k_pool))


def fp8_pool_desc(k_pool, element) -> pa_pool_desc:
    """Descriptor of an FP8 pool (uint8 codes, [NB][Hkv][B][D]) whose rows are
    written from, and read into, tensors of ``element``'s dtype."""
    torch = _torch()
    if k_pool.dim() != 4 or k_pool.dtype != torch.uint8:
        raise ValueError("FP8 pools are uint8 [num_blocks][num_kv_heads][block_size][head_dim]")
    nb, hkv, bs, d = (int(x) for x in k_pool.shape)
    return pa_pool_desc(nb, bs, hkv, d, dtype_code(element))


def _stream(stream):
    if stream is not None:
        return int(stream) if not hasattr(stream, "cuda_stream") else int(stream.cuda_stream)
    return int(_torch().cuda.current_stream().cuda_stream)


def _check(t, name, dtype=None, dim=None, device=None):
    # the kernels dereference every pointer on the GPU: a host tensor would
    # hand them host addresses
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor, got one on {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dimensions")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _on_current_device(t, name):
    """Work is enqueued on the current device's stream: the tensors must be
    there."""
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor, got one on {t.device}")
    cur = _torch().cuda.current_device()
    if t.device.index is not None and t.device.index != cur:
        raise ValueError(f"{name} is on {t.device} but the current device is cuda:{cur}")


def pa_write_kv(k, v, slot_mapping, k_pool, v_pool, stream=None) -> None:
    """Copy k[n], v[n] ([num_tokens][Hkv][D]) into slot slot_mapping[n] of the
    pools; negative slots are skipped."""
    torch = _torch()
    _on_current_device(k_pool, "k_pool")
    desc = pool_desc(k_pool)
    dev = k_pool.device
    for t, n in ((k_pool, "k_pool"), (v_pool, "v_pool"), (k, "k"), (v, "v")):
        _check(t, n, dtype=k_pool.dtype, device=dev)
    if v_pool.shape != k_pool.shape:
        raise ValueError("k_pool and v_pool differ in shape")
    _check(slot_mapping, "slot_mapping", dtype=torch.int32, dim=1, device=dev)
    n_tok = int(slot_mapping.shape[0])
    want = (n_tok, desc.num_kv_heads, desc.head_dim)
    if tuple(k.shape) != want or tuple(v.shape) != want:
        raise ValueError(f"k and v must be {want}")
    st = lib().pa_write_kv(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), n_tok,
                           k_pool.data_ptr(), v_pool.data_ptr(), ctypes.byref(desc),
                           _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_write_kv")


def pa_write_kv_fp8(k, v, slot_mapping, k_pool, v_pool, k_scale, v_scale, stream=None) -> None:
    """pa_write_kv into FP8 (E4M3) pools: each row of k, v is stored as
    codes of x / scale."""
    torch = _torch()
    _on_current_device(k_pool, "k_pool")
    desc = fp8_pool_desc(k_pool, k)
    dev = k_pool.device
    for t, n in ((k_pool, "k_pool"), (v_pool, "v_pool")):
        _check(t, n, dtype=torch.uint8, device=dev)
    for t, n in ((k, "k"), (v, "v")):
        _check(t, n, dtype=k.dtype, device=dev)
    if v_pool.shape != k_pool.shape:
        raise ValueError("k_pool and v_pool differ in shape")
    _check(slot_mapping, "slot_mapping", dtype=torch.int32, dim=1, device=dev)
    n_tok = int(slot_mapping.shape[0])
    want = (n_tok, desc.num_kv_heads, desc.head_dim)
    if tuple(k.shape) != want or tuple(v.shape) != want:
        raise ValueError(f"k and v must be {want}")
    st = lib().pa_write_kv_fp8(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), n_tok,
                               k_pool.data_ptr(), v_pool.data_ptr(), ctypes.byref(desc),
                               float(k_scale), float(v_scale), _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_write_kv_fp8")


def pa_decode_fp8(q, k_pool, v_pool, block_tables, context_lens, scale, k_scale, v_scale,
                  out=None, *, max_context_len, workspace=None, stream=None):
    """pa_decode over FP8 (E4M3) pools with per-pool scales."""
    torch = _torch()
    _on_current_device(k_pool, "k_pool")
    desc = fp8_pool_desc(k_pool, q)
    dev = k_pool.device
    _check(k_pool, "k_pool", dtype=torch.uint8, device=dev)
    _check(v_pool, "v_pool", dtype=torch.uint8, device=dev)
    if v_pool.shape != k_pool.shape:
        raise ValueError("k_pool and v_pool differ in shape")
    _check(q, "q", dim=3, device=dev)
    _check(block_tables, "block_tables", dtype=torch.int32, dim=2, device=dev)
    _check(context_lens, "context_lens", dtype=torch.int32, dim=1, device=dev)
    n, hq, d = (int(x) for x in q.shape)
    if d != desc.head_dim:
        raise ValueError("q head_dim differs from the pool's")
    if int(block_tables.shape[0]) != n or int(context_lens.shape[0]) != n:
        raise ValueError("block_tables / context_lens rows must equal num_seqs")
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", dtype=q.dtype, device=dev)
    need = pa_decode_workspace_bytes(n, hq, desc, max_context_len)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(workspace, "workspace", device=dev)
    st = lib().pa_decode_fp8(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                             ctypes.byref(desc), block_tables.data_ptr(),
                             int(block_tables.shape[1]), context_lens.data_ptr(), n,
                             int(max_context_len), hq, float(scale), float(k_scale),
                             float(v_scale), out.data_ptr(), workspace.data_ptr(),
                             workspace.numel() * workspace.element_size(), _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_decode_fp8")
    return out


def pa_append_decode_fp8(q, new_k, new_v, k_pool, v_pool, block_tables, context_lens, scale,
                         k_scale, v_scale, out=None, *, max_context_len, workspace=None,
                         stream=None):
    """Quantize token T_i - 1 of every sequence (rows of new_k / new_v,
    [N][Hkv][D], q's dtype) into the FP8 pools and decode, in one call; same
    result as pa_write_kv_fp8 followed by pa_decode_fp8."""
    torch = _torch()
    _on_current_device(k_pool, "k_pool")
    desc = fp8_pool_desc(k_pool, q)
    dev = k_pool.device
    _check(k_pool, "k_pool", dtype=torch.uint8, device=dev)
    _check(v_pool, "v_pool", dtype=torch.uint8, device=dev)
    if v_pool.shape != k_pool.shape:
        raise ValueError("k_pool and v_pool differ in shape")
    _check(q, "q", dim=3, device=dev)
    _check(block_tables, "block_tables", dtype=torch.int32, dim=2, device=dev)
    _check(context_lens, "context_lens", dtype=torch.int32, dim=1, device=dev)
    n, hq, d = (int(x) for x in q.shape)
    if d != desc.head_dim:
        raise ValueError("q head_dim differs from the pool's")
    if int(block_tables.shape[0]) != n or int(context_lens.shape[0]) != n:
        raise ValueError("block_tables / context_lens rows must equal num_seqs")
    want = (n, desc.num_kv_heads, desc.head_dim)
    for t, name in ((new_k, "new_k"), (new_v, "new_v")):
        _check(t, name, dtype=q.dtype, device=dev)
        if tuple(t.shape) != want:
            raise ValueError(f"{name} must be {want}")
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", dtype=q.dtype, device=dev)
    need = pa_decode_workspace_bytes(n, hq, desc, max_context_len)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(workspace, "workspace", device=dev)
    st = lib().pa_append_decode_fp8(q.data_ptr(), new_k.data_ptr(), new_v.data_ptr(),
                                    k_pool.data_ptr(), v_pool.data_ptr(), ctypes.byref(desc),
                                    block_tables.data_ptr(), int(block_tables.shape[1]),
                                    context_lens.data_ptr(), n, int(max_context_len), hq,
                                    float(scale), float(k_scale), float(v_scale), out.data_ptr(),
                                    workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(), _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_append_decode_fp8")
    return out


def pa_decode_workspace_bytes(num_seqs: int, num_q_heads: int, desc: pa_pool_desc,
                              max_context_len: int) -> int:
    return int(lib().pa_decode_workspace_bytes(int(num_seqs), int(num_q_heads),
                                               ctypes.byref(desc), int(max_context_len)))


def pa_decode_partitioned_workspace_bytes(num_seqs: int, num_q_heads: int, desc: pa_pool_desc,
                                          max_context_len: int, partition_tokens: int) -> int:
    return int(lib().pa_decode_partitioned_workspace_bytes(
        int(num_seqs), int(num_q_heads), ctypes.byref(desc), int(max_context_len),
        int(partition_tokens)))


def pa_decode(q, k_pool, v_pool, block_tables, context_lens, scale, out=None, *,
              max_context_len, workspace=None, stream=None):
    """Paged decode attention; returns ``out`` ([N][Hq][D], pool dtype).

    ``max_context_len`` is the host bound on context_lens (the library never
    reads device arrays on the host, so it is not derived here).
    ``workspace`` is a uint8 or float32 device tensor of at least
    pa_decode_workspace_bytes(...) bytes; when omitted a fresh one is taken
    from torch's caching allocator."""
    return _decode(q, None, None, k_pool, v_pool, block_tables, context_lens, scale, out,
                   max_context_len, workspace, 0, stream)


def pa_decode_noalloc(q, k_pool, v_pool, block_tables, context_lens, scale, out, *,
                      max_context_len, stream=None):
    """pa_decode on the library's own per-GPU workspace: the call allocates
    nothing (``out`` must be given).  Calls that may overlap on one GPU race."""
    torch = _torch()
    _on_current_device(k_pool, "k_pool")
    desc = pool_desc(k_pool)
    dev = k_pool.device
    _check(k_pool, "k_pool")
    _check(v_pool, "v_pool", dtype=k_pool.dtype, device=dev)
    if v_pool.shape != k_pool.shape:
        raise ValueError("k_pool and v_pool differ in shape")
    _check(q, "q", dtype=k_pool.dtype, dim=3, device=dev)
    _check(block_tables, "block_tables", dtype=torch.int32, dim=2, device=dev)
    _check(context_lens, "context_lens", dtype=torch.int32, dim=1, device=dev)
    _check(out, "out", dtype=q.dtype, device=dev)
    n, hq, d = (int(x) for x in q.shape)
    if d != desc.head_dim or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q / out shapes disagree with the pool")
    if int(block_tables.shape[0]) != n or int(context_lens.shape[0]) != n:
        raise ValueError("block_tables / context_lens rows must equal num_seqs")
    st = lib().pa_decode_noalloc(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                 ctypes.byref(desc), block_tables.data_ptr(),
                                 int(block_tables.shape[1]), context_lens.data_ptr(), n,
                                 int(max_context_len), hq, float(scale), out.data_ptr(),
                                 _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_decode_noalloc")
    return out


def pa_decode_partitioned(q, k_pool, v_pool, block_tables, context_lens, scale,
                          partition_tokens: int, out=None, *, max_context_len, workspace=None,
                          stream=None):
    """pa_decode with fixed context partitions of ``partition_tokens`` tokens
    (a multiple of 16) merged by the log-sum-exp reduce kernel."""
    if int(partition_tokens) <= 0:
        raise ValueError("partition_tokens must be positive (pa_decode is the library's split)")
    return _decode(q, None, None, k_pool, v_pool, block_tables, context_lens, scale, out,
                   max_context_len, workspace, int(partition_tokens), stream)


def pa_decode_sliding(q, k_pool, v_pool, block_tables, context_lens, scale, window: int,
                      out=None, *, max_context_len, workspace=None, partition_tokens: int = 0,
                      stream=None):
    """pa_decode over each sequence's last ``window`` tokens only (a layer
    trained with sliding-window attention)."""
    return _decode(q, None, None, k_pool, v_pool, block_tables, context_lens, scale, out,
                   max_context_len, workspace, partition_tokens, stream, window=int(window))


def pa_prefill(q, k_pool, v_pool, block_tables, context_lens, query_start, scale, out=None, *,
               max_context_len, max_query_len, stream=None):
    """Causal attention of each sequence's last M_i tokens (a prompt chunk or
    a decode token): q and out are [query_start[-1]][Hq][D]; rows
    query_start[i] .. query_start[i+1]-1 belong to sequence i.
    ``max_context_len`` and ``max_query_len`` are host bounds on T_i and M_i."""
    torch = _torch()
    _on_current_device(k_pool, "k_pool")
    desc = pool_desc(k_pool)
    dev = k_pool.device
    _check(k_pool, "k_pool")
    _check(v_pool, "v_pool", dtype=k_pool.dtype, device=dev)
    if v_pool.shape != k_pool.shape:
        raise ValueError("k_pool and v_pool differ in shape")
    _check(q, "q", dtype=k_pool.dtype, dim=3, device=dev)
    _check(block_tables, "block_tables", dtype=torch.int32, dim=2, device=dev)
    _check(context_lens, "context_lens", dtype=torch.int32, dim=1, device=dev)
    _check(query_start, "query_start", dtype=torch.int32, dim=1, device=dev)
    n = int(context_lens.shape[0])
    rows, hq, d = (int(x) for x in q.shape)
    if d != desc.head_dim:
        raise ValueError("q head_dim differs from the pool's")
    if int(block_tables.shape[0]) != n or int(query_start.shape[0]) != n + 1:
        raise ValueError("block_tables rows must equal num_seqs, query_start num_seqs + 1")
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", dtype=q.dtype, device=dev)
    if tuple(out.shape) != (rows, hq, d):
        raise ValueError("out must have q's shape")
    st = lib().pa_prefill(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), ctypes.byref(desc),
                          block_tables.data_ptr(), int(block_tables.shape[1]),
                          context_lens.data_ptr(), query_start.data_ptr(), n,
                          int(max_context_len), int(max_query_len), hq, float(scale),
                          out.data_ptr(), _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_prefill")
    return out


def pa_append_decode(q, new_k, new_v, k_pool, v_pool, block_tables, context_lens, scale,
                     out=None, *, max_context_len, workspace=None,
                     partition_tokens: int = 0, stream=None):
    """Write token T_i - 1 of every sequence (rows of new_k / new_v,
    [N][Hkv][D]) into the pools through the block tables and decode, in one
    call; same result as pa_write_kv followed by pa_decode."""
    return _decode(q, new_k, new_v, k_pool, v_pool, block_tables, context_lens, scale, out,
                   max_context_len, workspace, partition_tokens, stream)


def _decode(q, new_k, new_v, k_pool, v_pool, block_tables, context_lens, scale, out,
            max_context_len, workspace, partition_tokens, stream, window=None):
    torch = _torch()
    _on_current_device(k_pool, "k_pool")
    desc = pool_desc(k_pool)
    dev = k_pool.device
    _check(k_pool, "k_pool")
    _check(v_pool, "v_pool", dtype=k_pool.dtype, device=dev)
    if v_pool.shape != k_pool.shape:
        raise ValueError("k_pool and v_pool differ in shape")
    _check(q, "q", dtype=k_pool.dtype, dim=3, device=dev)
    _check(block_tables, "block_tables", dtype=torch.int32, dim=2, device=dev)
    _check(context_lens, "context_lens", dtype=torch.int32, dim=1, device=dev)
    n, hq, d = (int(x) for x in q.shape)
    if d != desc.head_dim:
        raise ValueError("q head_dim differs from the pool's")
    if int(block_tables.shape[0]) != n or int(context_lens.shape[0]) != n:
        raise ValueError("block_tables / context_lens rows must equal num_seqs")
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", dtype=q.dtype, device=dev)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    if new_k is not None:
        want = (n, desc.num_kv_heads, desc.head_dim)
        for t, name in ((new_k, "new_k"), (new_v, "new_v")):
            _check(t, name, dtype=k_pool.dtype, device=dev)
            if tuple(t.shape) != want:
                raise ValueError(f"{name} must be {want}")
    need = pa_decode_partitioned_workspace_bytes(n, hq, desc, max_context_len, partition_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(workspace, "workspace", device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    tail = (ctypes.byref(desc), block_tables.data_ptr(), int(block_tables.shape[1]),
            context_lens.data_ptr(), n, int(max_context_len), hq, float(scale),
            out.data_ptr(), workspace.data_ptr(), ws_bytes, int(partition_tokens),
            _stream(stream))
    if window is not None:
        st = lib().pa_decode_sliding(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                     *tail[:8], int(window), *tail[8:])
        where = "pa_decode_sliding"
    elif new_k is None and partition_tokens == 0:
        st = lib().pa_decode(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                             *tail[:11], tail[12])
        where = "pa_decode"
    elif new_k is None:
        st = lib().pa_decode_partitioned(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                         *tail)
        where = "pa_decode_partitioned"
    else:
        st = lib().pa_append_decode(q.data_ptr(), new_k.data_ptr(), new_v.data_ptr(),
                                    k_pool.data_ptr(), v_pool.data_ptr(), *tail)
        where = "pa_append_decode"
    if st != PA_OK:
        raise PaError(st, where)
    return out


# ---------------------------------------------------------------------------
# block copy (copy-on-write) and the host block manager
# ---------------------------------------------------------------------------
class PoolSet:
    """Pools for pa_copy_blocks, checked once: GPU tensors of one shape and
    dtype on one device, axis 0 the block.  Keeps the C array of their
    pointers, so a step that copies blocks in every layer's pools pays no
    per-pool work.  The pointers are taken here: the tensors' storage must
    not be resized or replaced while the set is in use."""

    def __init__(self, pools):
        pools = list(pools)
        if not pools:
            raise ValueError("no pools")
        ref = pools[0]
        if ref.dim() < 1:
            raise ValueError("pools need a block axis")
        for i, t in enumerate(pools):
            _check(t, f"pools[{i}]", dtype=ref.dtype, device=ref.device)
            if t.shape != ref.shape:
                raise ValueError("pools differ in shape")
        self.pools = pools                   # keeps the tensors alive
        self.device = ref.device
        self.num_blocks = int(ref.shape[0])
        self.block_bytes = ((ref.numel() // self.num_blocks) * ref.element_size()
                            if self.num_blocks else 16)
        self.ptrs = (ctypes.c_void_p * len(pools))(*[t.data_ptr() for t in pools])

    def __len__(self):
        return len(self.pools)


def pa_copy_blocks(pools, block_mapping, stream=None) -> None:
    """For every (source, destination) row of ``block_mapping`` (int32 [n][2]
    on the pools' device), copy block source to block destination in every
    pool (a PoolSet, or a list of tensors of one shape and dtype)."""
    torch = _torch()
    ps = pools if isinstance(pools, PoolSet) else PoolSet(pools)
    _on_current_device(ps.pools[0], "pools")
    _check(block_mapping, "block_mapping", dtype=torch.int32, device=ps.device)
    if block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [num_pairs][2]")
    st = lib().pa_copy_blocks(ps.ptrs, len(ps), ps.num_blocks, ps.block_bytes,
                              block_mapping.data_ptr(), int(block_mapping.shape[0]),
                              _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_copy_blocks")


def pa_sha256(data: bytes) -> bytes:
    out = (ctypes.c_uint8 * 32)()
    buf = ctypes.create_string_buffer(bytes(data), len(data)) if data else None
    st = lib().pa_sha256(buf, len(data), out)
    if st != PA_OK:
        raise PaError(st, "pa_sha256")
    return bytes(out)


class OutOfBlocks(PaError):
    """Not enough free blocks (the manager is unchanged)."""


class BlockManager:
    """The library's host block manager (free queue, reference counts,
    chained prefix hashes, copy-on-write).  Host-side NumPy in and out."""

    def __init__(self, num_blocks: int, block_size: int, prefix_caching: bool = True):
        h = ctypes.c_void_p()
        st = lib().pa_bm_create(int(num_blocks), int(block_size), int(bool(prefix_caching)),
                                ctypes.byref(h))
        if st != PA_OK:
            raise PaError(st, "pa_bm_create")
        self._h = h
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self) -> None:
        if self._h:
            lib().pa_bm_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _raise(self, st, where):
        if st == PA_ERR_OUT_OF_BLOCKS:
            raise OutOfBlocks(st, where)
        if st != PA_OK:
            raise PaError(st, where)

    def allocate(self, seq: int, prompt, salt: bytes = b"") -> int:
        """Admit ``seq``; returns the number of prompt tokens already cached."""
        import numpy as np
        toks = np.ascontiguousarray(np.asarray(prompt, dtype=np.int32).reshape(-1))
        cached = ctypes.c_int32(0)
        salt = bytes(salt)
        sbuf = ctypes.create_string_buffer(salt, len(salt)) if salt else None
        st = lib().pa_bm_allocate(self._h, int(seq), toks.ctypes.data if toks.size else None,
                                  int(toks.size), sbuf, len(salt), ctypes.byref(cached))
        self._raise(st, "pa_bm_allocate")
        return int(cached.value)

    def append(self, seqs, tokens):
        """Append tokens[i] to seqs[i] (in order); returns (slots int32 [n],
        copy-on-write pairs int32 [k][2])."""
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64).reshape(-1))
        toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))
        if ids.size != toks.size:
            raise ValueError("seqs and tokens differ in length")
        n = int(ids.size)
        slots = np.zeros(max(n, 1), np.int32)
        pairs = np.zeros((max(n, 1), 2), np.int32)
        k = ctypes.c_int32(0)
        st = lib().pa_bm_append(self._h, ids.ctypes.data, toks.ctypes.data, n, slots.ctypes.data,
                                pairs.ctypes.data, ctypes.byref(k))
        self._raise(st, "pa_bm_append")
        return slots[:n].copy(), pairs[:k.value].copy()

    def append_one(self, seq: int, token: int):
        """One token; returns (slot, (source, destination) or None)."""
        slots, pairs = self.append([seq], [token])
        return int(slots[0]), (tuple(int(x) for x in pairs[0]) if len(pairs) else None)

    def fork(self, parent: int, child: int) -> None:
        self._raise(lib().pa_bm_fork(self._h, int(parent), int(child)), "pa_bm_fork")

    def free_seq(self, seq: int) -> None:
        self._raise(lib().pa_bm_free(self._h, int(seq)), "pa_bm_free")

    def tables(self, seqs, max_blocks: int):
        """(block tables int32 [n][max_blocks] padded with -1, context lengths)."""
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64).reshape(-1))
        tab = np.zeros((ids.size, max_blocks), np.int32)
        lens = np.zeros(ids.size, np.int32)
        st = lib().pa_bm_tables(self._h, ids.ctypes.data, int(ids.size), int(max_blocks),
                                tab.ctypes.data, lens.ctypes.data)
        self._raise(st, "pa_bm_tables")
        return tab, lens

    def block_table(self, seq: int) -> list[int]:
        tab, _ = self.tables([seq], self.num_blocks)
        row = tab[0]
        return [int(b) for b in row[row >= 0]]

    def num_tokens(self, seq: int) -> int:
        return int(self.tables([seq], self.num_blocks)[1][0])

    def num_free(self) -> int:
        return int(lib().pa_bm_num_free(self._h))

    def block_info(self, block: int):
        """(reference count, digest bytes or None, registered)."""
        ref, has, reg = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
        d = (ctypes.c_uint8 * 32)()
        st = lib().pa_bm_block_info(self._h, int(block), ctypes.byref(ref), ctypes.byref(has), d,
                                    ctypes.byref(reg))
        self._raise(st, "pa_bm_block_info")
        return int(ref.value), (bytes(d) if has.value else None), bool(reg.value)

    def free_queue(self) -> list[int]:
        import numpy as np
        out = np.zeros(max(self.num_blocks, 1), np.int32)
        n = ctypes.c_int32(0)
        st = lib().pa_bm_free_queue(self._h, out.ctypes.data, self.num_blocks, ctypes.byref(n))
        self._raise(st, "pa_bm_free_queue")
        return [int(b) for b in out[:n.value]]


# ---------------------------------------------------------------------------
# contract check of the device arrays
# ---------------------------------------------------------------------------
def pa_check_inputs(k_pool, slot_mapping=None, block_tables=None, context_lens=None,
                    max_context_len=None, duplicates: bool = True, stream=None):
    """Check the arrays a write or decode call would read against the pool
    k_pool ([num_blocks][Hkv][B][D], any element type).  Returns (count,
    kind, index, value) of the violations, kind/index/value those of the
    first (0s when there is none).  Synchronizes the stream to read them."""
    torch = _torch()
    _on_current_device(k_pool, "k_pool")
    if k_pool.dim() != 4:
        raise ValueError("pools are [num_blocks][num_kv_heads][block_size][head_dim]")
    nb, hkv, bs, d = (int(x) for x in k_pool.shape)
    desc = pa_pool_desc(nb, bs, hkv, d, PA_BF16)     # the element type plays no part here
    dev = k_pool.device
    n_tok, n_seq, mb = 0, 0, 0
    if slot_mapping is not None:
        _check(slot_mapping, "slot_mapping", dtype=torch.int32, dim=1, device=dev)
        n_tok = int(slot_mapping.shape[0])
    if block_tables is not None or context_lens is not None:
        if block_tables is None or context_lens is None:
            raise ValueError("block_tables and context_lens go together")
        _check(block_tables, "block_tables", dtype=torch.int32, dim=2, device=dev)
        _check(context_lens, "context_lens", dtype=torch.int32, dim=1, device=dev)
        n_seq, mb = int(block_tables.shape[0]), int(block_tables.shape[1])
        if int(context_lens.shape[0]) != n_seq:
            raise ValueError("context_lens rows must equal block_tables rows")
        if max_context_len is None:
            max_context_len = mb * bs
    report = torch.zeros(4, dtype=torch.int32, device=dev)
    scratch = None
    if duplicates and n_tok:
        scratch = torch.empty(max(int(lib().pa_check_scratch_bytes(ctypes.byref(desc))), 4),
                              dtype=torch.uint8, device=dev)
    st = lib().pa_check_inputs(slot_mapping.data_ptr() if n_tok else None, n_tok,
                               block_tables.data_ptr() if n_seq else None, mb,
                               context_lens.data_ptr() if n_seq else None, n_seq,
                               int(max_context_len or 0), ctypes.byref(desc), report.data_ptr(),
                               scratch.data_ptr() if scratch is not None else None,
                               _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_check_inputs")
    return tuple(int(x) for x in report.cpu().tolist())
