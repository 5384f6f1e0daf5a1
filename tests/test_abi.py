"""CPU-side checks of the C ABI: the library loads, exports every entry point
``include/pa.h`` declares, and rejects bad arguments before any HIP call.
No kernel is launched here (every call below fails validation or has
nothing to do)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import paged_kv_cache_pa_amd as pa
from paged_kv_cache_pa_amd import CacheParams, DecodeParams

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP, WS = 0, -1, -2, -3, -4, -5, -6


def declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^[A-Za-z_][\w \*]*?\b(pa_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    return pa.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert {"pa_decode", "pa_decode_dense", "pa_cache_write", "pa_copy_blocks",
            "pa_decode_workspace_size", "pa_status_string", "pa_build_info",
            "pa_bm_create", "pa_bm_destroy", "pa_bm_reserve", "pa_bm_tables", "pa_bm_fork",
            "pa_bm_free", "pa_bm_swap_out", "pa_bm_swap_in"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/ but not exported"


def test_status_strings(L):
    for code, name in pa.STATUS.items():
        assert L.pa_status_string(code).decode().startswith(name)
    assert L.pa_status_string(12345)
    assert b"gfx950" in L.pa_build_info()


def params(**kw):
    base = dict(num_seqs=4, num_q_heads=8, num_kv_heads=8, head_dim=64, block_size=16,
                max_blocks_per_seq=7, num_blocks=64, max_context_len=112, partition_size=0,
                dtype=0, layout=0)
    base.update(kw)
    return DecodeParams(*[base[f] for f, _ in DecodeParams._fields_])


class Buf:
    """Aligned host memory standing in for device pointers (never dereferenced:
    every call using it fails validation first)."""

    def __init__(self, n=4096):
        self.raw = ctypes.create_string_buffer(n + 64)
        base = ctypes.addressof(self.raw)
        self.p = ctypes.c_void_p((base + 15) & ~15)
        self.odd = ctypes.c_void_p(((base + 15) & ~15) + 2)


def decode(L, p, q=None, k=None, v=None, t=None, c=None, out=None, ws=None, nbytes=0):
    b = Buf()
    args = [b.p if x is None else x for x in (q, k, v, t, c)]
    return L.pa_decode(*args, ctypes.c_float(0.125), b.p if out is None else out,
                       ctypes.byref(p), ws, nbytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), DTYPE), (dict(dtype=-1), DTYPE),
    (dict(num_seqs=-1), SHAPE), (dict(num_q_heads=0), SHAPE), (dict(num_kv_heads=0), SHAPE),
    (dict(num_q_heads=12, num_kv_heads=5), SHAPE), (dict(block_size=12), SHAPE),
    (dict(block_size=512), SHAPE), (dict(block_size=0), SHAPE),
    (dict(max_blocks_per_seq=0), SHAPE), (dict(num_blocks=0), SHAPE),
    (dict(max_context_len=-1), SHAPE), (dict(max_context_len=7 * 16 + 1), SHAPE),
    (dict(partition_size=8), SHAPE), (dict(partition_size=-16), SHAPE),
    (dict(layout=2), SHAPE), (dict(layout=-1), SHAPE),
    (dict(head_dim=96), UNSUP), (dict(head_dim=256), UNSUP),
    (dict(num_kv_heads=1 << 20, num_q_heads=1 << 20), UNSUP),
    (dict(num_q_heads=18, num_kv_heads=2), UNSUP),            # fp32: at most 8 per kv head
    (dict(num_q_heads=34, num_kv_heads=2, dtype=1), UNSUP),   # fp16: at most 16
    (dict(num_q_heads=34, num_kv_heads=2, dtype=2), UNSUP),   # bf16: at most 16
])
def test_decode_rejects_bad_shapes(L, kw, code):
    assert decode(L, params(**kw)) == code


def test_decode_rejects_null_and_misaligned(L):
    b = Buf()
    p = params()
    for i in range(6):
        args = [b.p] * 6
        args[i] = None
        assert L.pa_decode(*args[:5], ctypes.c_float(1.0), args[5], ctypes.byref(p), None, 0,
                           None) == NULL
    for i in (0, 1, 2, 5):  # q, k, v, out must be 16-byte aligned
        args = [b.p] * 6
        args[i] = b.odd
        assert L.pa_decode(*args[:5], ctypes.c_float(1.0), args[5], ctypes.byref(p), None, 0,
                           None) == ALIGN
    assert L.pa_decode(b.p, b.p, b.p, b.p, b.p, ctypes.c_float(1.0), b.p, None, None, 0,
                       None) == NULL


def test_decode_split_needs_workspace(L):
    p = params(partition_size=32)
    need = pa.pa_decode_workspace_size(p)
    assert need == 4 * 8 * 4 * (64 + 2) * 4  # ceil(112 / 32) = 4 partitions
    b = Buf(need + 64)
    assert decode(L, p) == WS
    assert decode(L, p, ws=b.p, nbytes=need - 4) == WS


def test_workspace_size_formula():
    assert pa.pa_decode_workspace_size(params()) == 0
    assert pa.pa_decode_workspace_size(params(partition_size=112)) == 0   # one partition
    assert pa.pa_decode_workspace_size(params(partition_size=16)) == 4 * 8 * 7 * 66 * 4
    big = params(num_seqs=8, num_q_heads=12, num_kv_heads=2, head_dim=128, max_blocks_per_seq=1024,
                 max_context_len=16384, partition_size=512, dtype=2)
    assert pa.pa_decode_workspace_size(big) == 8 * 12 * 32 * 130 * 4
    with pytest.raises(pa.PaError):
        pa.pa_decode_workspace_size(params(dtype=9))


def test_decode_append_checks(L):
    b = Buf()
    p = params()
    f = ctypes.c_float(1.0)
    args = [b.p, b.p, b.p, b.p, b.p, b.p, b.p]
    assert L.pa_decode_append(*args, f, b.p, ctypes.byref(params(dtype=9)), None, 0,
                              None) == DTYPE
    for i in (1, 2):
        a = list(args)
        a[i] = None
        assert L.pa_decode_append(*a, f, b.p, ctypes.byref(p), None, 0, None) == NULL
        a[i] = b.odd
        assert L.pa_decode_append(*a, f, b.p, ctypes.byref(p), None, 0, None) == ALIGN
    a = list(args)
    a[3] = None   # k_cache
    assert L.pa_decode_append(*a, f, b.p, ctypes.byref(p), None, 0, None) == NULL
    assert L.pa_decode_append(*args, f, b.p, ctypes.byref(params(partition_size=32)), None, 0,
                              None) == WS
    assert L.pa_decode_append(None, None, None, None, None, None, None, f, None,
                              ctypes.byref(params(num_seqs=0)), None, 0, None) == OK


def test_zero_sequences_is_a_no_op(L):
    p = params(num_seqs=0)
    assert L.pa_decode(None, None, None, None, None, ctypes.c_float(1.0), None, ctypes.byref(p),
                       None, 0, None) == OK


def test_dense_checks(L):
    b = Buf()
    p = params(max_context_len=100)
    assert L.pa_decode_dense(b.p, b.p, b.p, b.p, ctypes.c_float(1.0), b.p, ctypes.byref(p), 0,
                             None, 0, None) == SHAPE               # max_seq_len < 1
    assert L.pa_decode_dense(b.p, b.p, b.p, b.p, ctypes.c_float(1.0), b.p, ctypes.byref(p), 64,
                             None, 0, None) == SHAPE               # max_context_len > max_seq_len
    p = params(max_context_len=100, partition_size=24)
    assert L.pa_decode_dense(b.p, b.p, b.p, b.p, ctypes.c_float(1.0), b.p, ctypes.byref(p), 128,
                             None, 0, None) == SHAPE               # partition not a multiple of 16
    p = params(max_context_len=100, partition_size=32)
    assert L.pa_decode_dense(b.p, b.p, b.p, b.p, ctypes.c_float(1.0), b.p, ctypes.byref(p), 128,
                             None, 0, None) == WS
    p = params(num_seqs=0, max_context_len=1)
    assert L.pa_decode_dense(None, None, None, None, ctypes.c_float(1.0), None, ctypes.byref(p), 1,
                             None, 0, None) == OK


def cparams(**kw):
    base = dict(num_blocks=64, block_size=16, num_kv_heads=8, head_dim=64, dtype=0, layout=0)
    base.update(kw)
    return CacheParams(*[base[f] for f, _ in CacheParams._fields_])


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), DTYPE), (dict(num_blocks=0), SHAPE), (dict(block_size=3), SHAPE),
    (dict(num_kv_heads=0), SHAPE), (dict(head_dim=0), SHAPE),
    (dict(head_dim=6, dtype=1), SHAPE),   # 12-byte rows cannot be moved as 16-byte vectors
    (dict(layout=7), SHAPE),
])
def test_cache_write_and_copy_reject_bad_params(L, kw, code):
    b = Buf()
    p = cparams(**kw)
    assert L.pa_cache_write(b.p, b.p, b.p, b.p, b.p, 4, ctypes.byref(p), None) == code
    assert L.pa_copy_blocks(b.p, b.p, b.p, 4, ctypes.byref(p), None) == code


def test_cache_write_and_copy_pointer_checks(L):
    b = Buf()
    p = cparams()
    assert L.pa_cache_write(b.p, b.p, b.p, b.p, b.p, -1, ctypes.byref(p), None) == SHAPE
    assert L.pa_cache_write(None, None, None, None, None, 0, ctypes.byref(p), None) == OK
    for i in range(5):
        args = [b.p] * 5
        args[i] = None
        assert L.pa_cache_write(*args, 3, ctypes.byref(p), None) == NULL
    for i in range(4):
        args = [b.p] * 5
        args[i] = b.odd
        assert L.pa_cache_write(*args, 3, ctypes.byref(p), None) == ALIGN
    assert L.pa_copy_blocks(b.p, b.p, b.p, -2, ctypes.byref(p), None) == SHAPE
    assert L.pa_copy_blocks(None, None, None, 0, ctypes.byref(p), None) == OK
    assert L.pa_copy_blocks(b.p, None, b.p, 2, ctypes.byref(p), None) == NULL
    assert L.pa_copy_blocks(b.odd, b.p, b.p, 2, ctypes.byref(p), None) == ALIGN
    assert L.pa_cache_write(b.p, b.p, b.p, b.p, b.p, 3, None, None) == NULL


def test_multi_layer_copy_and_swap_checks(L):
    """Per-layer pointer arrays are checked entry by entry before any launch."""
    b = Buf()
    p = cparams()
    P = ctypes.c_void_p

    def arr(*xs):
        return (P * len(xs))(*xs)

    good = arr(b.p, b.p, b.p)
    assert L.pa_copy_blocks_layers(good, good, 3, b.p, 0, ctypes.byref(p), None) == OK
    assert L.pa_copy_blocks_layers(good, good, 0, b.p, 2, ctypes.byref(p), None) == SHAPE
    assert L.pa_copy_blocks_layers(good, good, 3, b.p, -1, ctypes.byref(p), None) == SHAPE
    assert L.pa_copy_blocks_layers(None, good, 3, b.p, 2, ctypes.byref(p), None) == NULL
    assert L.pa_copy_blocks_layers(arr(b.p, None, b.p), good, 3, b.p, 2, ctypes.byref(p),
                                   None) == NULL
    assert L.pa_copy_blocks_layers(good, arr(b.p, b.p, b.odd), 3, b.p, 2, ctypes.byref(p),
                                   None) == ALIGN
    assert L.pa_copy_blocks_layers(good, good, 3, None, 2, ctypes.byref(p), None) == NULL
    assert L.pa_copy_blocks_layers(good, good, 3, b.p, 2, ctypes.byref(cparams(dtype=9)),
                                   None) == DTYPE
    # too many (pair, layer, K|V) workgroups for one grid dimension
    assert L.pa_copy_blocks_layers(good, good, 3, b.p, 1 << 30, ctypes.byref(p), None) == UNSUP
    cw = L.pa_cache_write_layers
    assert cw(good, good, good, good, 3, b.p, 0, ctypes.byref(p), None) == OK
    assert cw(good, good, good, good, 0, b.p, 2, ctypes.byref(p), None) == SHAPE
    assert cw(good, good, good, good, 3, b.p, -1, ctypes.byref(p), None) == SHAPE
    assert cw(good, None, good, good, 3, b.p, 2, ctypes.byref(p), None) == NULL
    assert cw(good, good, arr(b.p, b.p, None), good, 3, b.p, 2, ctypes.byref(p), None) == NULL
    assert cw(arr(b.p, b.odd, b.p), good, good, good, 3, b.p, 2, ctypes.byref(p), None) == ALIGN
    assert cw(good, good, good, good, 3, None, 2, ctypes.byref(p), None) == NULL
    assert cw(good, good, good, good, 3, P(b.p.value + 2), 2, ctypes.byref(p), None) == ALIGN
    assert cw(good, good, good, good, 3, b.p, 2, ctypes.byref(cparams(dtype=9)), None) == DTYPE
    sw = L.pa_swap_blocks
    assert sw(good, good, 8, good, good, 64, 3, b.p, 0, ctypes.byref(p), None) == OK
    assert sw(good, good, 0, good, good, 64, 3, b.p, 2, ctypes.byref(p), None) == SHAPE
    assert sw(good, good, 8, good, good, 0, 3, b.p, 2, ctypes.byref(p), None) == SHAPE
    assert sw(good, None, 8, good, good, 64, 3, b.p, 2, ctypes.byref(p), None) == NULL
    assert sw(good, good, 8, arr(b.odd, b.p, b.p), good, 64, 3, b.p, 2, ctypes.byref(p),
              None) == ALIGN
    assert sw(good, good, 8, good, good, 64, 3, P(b.p.value + 2), 2, ctypes.byref(p), None) == ALIGN


def pparams(**kw):
    base = dict(num_seqs=2, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                max_blocks_per_seq=8, num_blocks=32, total_query_rows=40, max_query_len=32,
                max_context_len=128, dtype=1, layout=1)
    base.update(kw)
    return pa.PrefillParams(*[base[f] for f, _ in pa.PrefillParams._fields_])


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), DTYPE), (dict(dtype=0), UNSUP), (dict(head_dim=96), UNSUP),
    (dict(num_q_heads=6, num_kv_heads=4), SHAPE), (dict(layout=3), SHAPE),
    (dict(block_size=12), SHAPE), (dict(max_context_len=129), SHAPE),
    (dict(max_query_len=200), SHAPE), (dict(num_seqs=-1), SHAPE),
    (dict(total_query_rows=-1), SHAPE), (dict(max_blocks_per_seq=0), SHAPE),
])
def test_prefill_rejects_bad_params(L, kw, code):
    b = Buf()
    p = pparams(**kw)
    assert L.pa_prefill(b.p, b.p, b.p, b.p, b.p, b.p, ctypes.c_float(1.0), b.p,
                        ctypes.byref(p), None) == code


def test_prefill_pointer_checks(L):
    b = Buf()
    p = pparams()
    f = ctypes.c_float(1.0)
    for i in range(7):
        args = [b.p] * 7
        args[i] = None
        assert L.pa_prefill(*args[:6], f, args[6], ctypes.byref(p), None) == NULL
    for i in (0, 1, 2, 6):
        args = [b.p] * 7
        args[i] = b.odd
        assert L.pa_prefill(*args[:6], f, args[6], ctypes.byref(p), None) == ALIGN
    odd4 = ctypes.c_void_p(b.p.value + 2)
    for i in (3, 4, 5):
        args = [b.p] * 7
        args[i] = odd4
        assert L.pa_prefill(*args[:6], f, args[6], ctypes.byref(p), None) == ALIGN
    for kw in (dict(num_seqs=0), dict(total_query_rows=0), dict(max_query_len=0)):
        assert L.pa_prefill(None, None, None, None, None, None, f, None,
                            ctypes.byref(pparams(**kw)), None) == OK
    assert L.pa_prefill(b.p, b.p, b.p, b.p, b.p, b.p, f, b.p, None, None) == NULL


def test_binding_refuses_cpu_tensors():
    import torch

    q = torch.zeros(1, 1, 64)
    with pytest.raises(ValueError):
        pa.pa_decode(q, q, q, q, q, 1.0, q)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import importlib

    monkeypatch.setattr(pa, "_lib", None)
    monkeypatch.setattr(pa, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        pa.lib()
    importlib.reload(pa)


def test_one_hip_runtime_per_process():
    """Loading the library before anything imports torch must still leave the
    process with one HIP runtime (torch's), not torch's and the system's."""
    import subprocess
    import sys

    code = ("import paged_kv_cache_pa_amd as pa; pa.lib(); import torch; "
            "m = open('/proc/self/maps').read().splitlines(); "
            "print(len({l.split()[-1] for l in m if 'libamdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "1"


def test_decode_no_alloc_checks(L):
    """pa_decode_no_alloc validates like pa_decode and refuses a split whose
    partials exceed its fixed scratch array, all before any HIP call."""
    SCRATCH = -10
    assert pa.STATUS[SCRATCH] == "PA_ERR_SCRATCH"
    assert pa.NO_ALLOC_SCRATCH_BYTES == 16 << 20
    b = Buf()

    def call(p, *ptrs):
        args = list(ptrs) if ptrs else [b.p] * 6
        return L.pa_decode_no_alloc(*args[:5], ctypes.c_float(0.125), args[5],
                                    None if p is None else ctypes.byref(p), None)

    assert call(None) == NULL
    assert call(params(dtype=7)) == DTYPE
    assert call(params(partition_size=24)) == SHAPE       # not a multiple of the block size
    assert call(params(head_dim=96)) == UNSUP
    assert call(params(num_seqs=0)) == OK                 # nothing to do, nothing launched
    for i in range(6):
        args = [b.p] * 6
        args[i] = None
        assert call(params(), *args) == NULL
    for i in (0, 1, 2, 5):
        args = [b.p] * 6
        args[i] = b.odd
        assert call(params(), *args) == ALIGN
    # 64 sequences x 40 query heads x (D 128 + 2) x 4 bytes per partition:
    # 12 partitions fit in 16 MiB, 13 do not
    fits = params(num_seqs=64, num_q_heads=40, num_kv_heads=40, head_dim=128, block_size=16,
                  max_blocks_per_seq=128, num_blocks=2048, max_context_len=12 * 128,
                  partition_size=128, dtype=1)
    assert pa.pa_decode_workspace_size(fits) == 64 * 40 * 12 * 130 * 4 <= pa.NO_ALLOC_SCRATCH_BYTES
    over = params(num_seqs=64, num_q_heads=40, num_kv_heads=40, head_dim=128, block_size=16,
                  max_blocks_per_seq=128, num_blocks=2048, max_context_len=13 * 128,
                  partition_size=128, dtype=1)
    assert pa.pa_decode_workspace_size(over) > pa.NO_ALLOC_SCRATCH_BYTES
    assert call(over) == SCRATCH
    assert b"scratch" in L.pa_status_string(SCRATCH)


def test_grid_thread_count_fits_32_bits(L):
    """One workgroup of up to 512 threads per (sequence, kv head, partition):
    a launch whose thread count would pass 2^32 is refused."""
    p = params(num_seqs=65536, num_q_heads=128, num_kv_heads=128, head_dim=128,
               max_blocks_per_seq=1, block_size=16, max_context_len=16, num_blocks=64)
    assert decode(L, p) == UNSUP                       # 2^23 workgroups x 512 threads = 2^32
    p = params(num_seqs=65535, num_q_heads=128, num_kv_heads=128, head_dim=128,
               max_blocks_per_seq=1, block_size=16, max_context_len=16, num_blocks=64)
    assert L.pa_decode_workspace_size(ctypes.byref(p), ctypes.byref(ctypes.c_size_t())) == OK


def test_decode_shared_checks(L):
    """pa_decode_shared validates its extra arguments (16-bit types only, a
    split, a group count within the batch, a shared-block bound within the
    table row, the group arrays) before any HIP call, and its workspace is
    pa_decode's rounded up to 16 bytes plus one int32 per sequence."""
    b = Buf()

    def call(p, gs=b.p, gsh=b.p, ng=2, msb=4, ws=None, nbytes=0):
        return L.pa_decode_shared(b.p, b.p, b.p, b.p, b.p, gs, gsh, ng, msb,
                                  ctypes.c_float(0.125), b.p,
                                  None if p is None else ctypes.byref(p), ws, nbytes, None)

    half = dict(dtype=1, partition_size=32)
    assert call(None) == NULL
    assert call(params(dtype=0, partition_size=32)) == UNSUP      # fp32: no matrix-core tile
    assert call(params(dtype=1)) == SHAPE                         # no split
    assert call(params(**half), ng=-1) == SHAPE
    assert call(params(**half), ng=5) == SHAPE                    # more groups than sequences
    assert call(params(**half), msb=-1) == SHAPE
    assert call(params(**half), msb=8) == SHAPE                   # past max_blocks_per_seq (7)
    assert call(params(num_seqs=0, **half), ng=0) == OK           # nothing to do
    assert call(params(**half), gs=None) == NULL
    assert call(params(**half), gsh=None) == NULL
    assert call(params(**half), gs=b.odd) == ALIGN
    assert call(params(**half), gsh=b.odd) == ALIGN
    # the workspace: 4 x 8 x ceil(112 / 32) x 66 x 4 bytes of partials, then 4 x 4
    p = params(**half)
    assert pa.pa_decode_shared_workspace_size(p) == 4 * 8 * 4 * 66 * 4 + 16
    assert call(p, ws=b.p, nbytes=4 * 8 * 4 * 66 * 4) == WS       # room for the partials only
    # max_context_len within one partition: no partials, the per-sequence counts only
    p1 = params(dtype=1, partition_size=128)
    assert pa.pa_decode_shared_workspace_size(p1) == 16
    assert call(p1, ws=None, nbytes=0) == WS
