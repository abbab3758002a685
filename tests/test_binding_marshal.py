"""The Python binding's marshalling, on the CPU: every wrapper calls its C
entry point with exactly the arguments the library declares (ctypes would
otherwise fail only on a GPU machine, at the first call).

The wrappers run on host tensors here with the device checks switched off and
the library replaced by a stand-in whose functions check the argument count
against the argtypes the binding gives the real libpa.so; nothing is
computed."""
import ctypes
import os

import pytest
import torch

from paged_kv_cache_75_amd import binding as B

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="libpa.so not built")


class _Lib:
    """Stands in for libpa.so: records calls, checks their arity."""

    def __init__(self, real):
        self.real = real
        self.calls = []

    def __getattr__(self, name):
        fn = getattr(self.real, name)

        def call(*args):
            assert fn.argtypes is not None, f"{name} has no declared argtypes"
            assert len(args) == len(fn.argtypes), (
                f"{name}: {len(args)} arguments, the library takes {len(fn.argtypes)}")
            self.calls.append(name)
            if fn.restype is ctypes.c_size_t:
                return 1 << 20
            return B.PA_OK
        return call


@pytest.fixture
def fake(monkeypatch):
    lib = _Lib(B.lib())
    monkeypatch.setattr(B, "lib", lambda: lib)
    monkeypatch.setattr(B, "_check", lambda *a, **k: None)
    monkeypatch.setattr(B, "_on_current_device", lambda *a, **k: None)
    monkeypatch.setattr(B, "_stream", lambda s: 0)
    return lib


def test_every_decode_wrapper_passes_the_declared_arguments(fake):
    n, hkv, hq, d, bs, nb = 3, 2, 8, 128, 16, 12
    pool = torch.zeros((nb, hkv, bs, d), dtype=torch.bfloat16)
    fp8 = torch.zeros((nb, hkv, bs, d), dtype=torch.uint8)
    q = torch.zeros((n, hq, d), dtype=torch.bfloat16)
    new = torch.zeros((n, hkv, d), dtype=torch.bfloat16)
    bt = torch.zeros((n, 4), dtype=torch.int32)
    cl = torch.ones(n, dtype=torch.int32)
    qs = torch.arange(n + 1, dtype=torch.int32)
    B.pa_write_kv(new, new, cl, pool, pool)
    B.pa_decode(q, pool, pool, bt, cl, 0.1, max_context_len=64)
    B.pa_decode_partitioned(q, pool, pool, bt, cl, 0.1, 32, max_context_len=64)
    B.pa_decode_sliding(q, pool, pool, bt, cl, 0.1, 8, max_context_len=64)
    B.pa_append_decode(q, new, new, pool, pool, bt, cl, 0.1, max_context_len=64)
    B.pa_append_decode(q, new, new, pool, pool, bt, cl, 0.1, max_context_len=64,
                       partition_tokens=32)
    B.pa_prefill(q, pool, pool, bt, cl, qs, 0.1, max_context_len=64, max_query_len=1)
    B.pa_write_kv_fp8(new, new, cl, fp8, fp8, 1.0, 1.0)
    B.pa_decode_fp8(q, fp8, fp8, bt, cl, 0.1, 1.0, 1.0, max_context_len=64)
    B.pa_append_decode_fp8(q, new, new, fp8, fp8, bt, cl, 0.1, 1.0, 1.0, max_context_len=64)
    called = set(fake.calls)
    assert {"pa_write_kv", "pa_decode", "pa_decode_partitioned", "pa_decode_sliding",
            "pa_append_decode", "pa_prefill", "pa_write_kv_fp8", "pa_decode_fp8",
            "pa_append_decode_fp8"} <= called


def test_max_context_len_is_required():
    q = torch.zeros((1, 2, 64))
    with pytest.raises(TypeError):
        B.pa_decode(q, q, q, q, q, 0.1)
    with pytest.raises(TypeError):
        B.pa_prefill(q, q, q, q, q, q, 0.1)
