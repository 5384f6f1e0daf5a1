"""fp64 CPU oracle for paged decode attention, cache_write and copy_blocks.

TEST INFRASTRUCTURE ONLY: tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are the only callers.  The library path
(``paged_kv_cache_pa_amd``) never imports this package, and this package
imports nothing from it.

``oracle.c`` (built to ``liboracle.so`` with gcc) holds the arithmetic;
``brute.py`` holds a pure-Python scalar version for hand-sized inputs.  Each
function cites the passage of the pages it follows.  Every function here is
pinned by ``tests/test_oracle.py``; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_DT = {"f32": 0, "f16": 1, "bf16": 2}
_LAYOUT = {"NHD": 0, "HND": 1}  # token-major [.., tokens, Hkv, D] / head-major [.., Hkv, tokens, D]


def _dims(a, layout):
    """(outer, tokens, kv heads, head_dim) of a pool or dense tensor."""
    x, y, z, d = a.shape
    return (x, y, z, d) if _LAYOUT[layout] == 0 else (x, z, y, d)
_lib = None


def build(verbose=False, src=None, out=None) -> str:
    """Compile oracle.c with gcc (fp64, OpenMP, no fast-math)."""
    src = src or os.path.join(_HERE, "oracle.c")
    out = out or LIB_PATH
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           "-fno-fast-math", "-ffp-contract=off", src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def load(path):
    """Load a built oracle library and declare its signatures."""
    L = ctypes.CDLL(path)
    P, I, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
    L.oracle_decode.argtypes = [P, P, P, P, P, D, I, I, I, I, I, I, I, I, I, P, I, P, P, I, I]
    L.oracle_decode_dense.argtypes = [P, P, P, P, D, I, I, I, I, I, I, I, P, I, P, I]
    L.oracle_decode_split.argtypes = [P, P, P, P, P, D, I, I, I, I, I, I, I, I, I, I, P, I]
    L.oracle_cache_write.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I]
    L.oracle_copy_blocks.argtypes = [P, P, P, I, I, I, I, I, I]
    L.oracle_prefill.argtypes = [P, P, P, P, P, P, D, I, I, I, I, I, I, I, I, I, I, P, I]
    L.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    L.oracle_half_to_double.restype = D
    L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    L.oracle_bf16_to_double.restype = D
    for f in ("oracle_decode", "oracle_decode_dense", "oracle_decode_split",
              "oracle_cache_write", "oracle_copy_blocks", "oracle_prefill"):
        getattr(L, f).restype = I
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = load(LIB_PATH)
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype=None):
    return np.ascontiguousarray(a, dtype=dtype)


def _threads(n):
    if n is not None:
        return int(n)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


class OracleError(RuntimeError):
    pass


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what} returned {rc}")


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, dtype,
           units=None, want_weights=False, nthreads=None, layout="NHD"):
    """Paged decode in fp64.  Returns out [S, Hq, D] (float64); with
    ``want_weights`` also the softmax weights [S, Hq, MBS*B] (zeros past n).

    ``units``: optional int array [(s, h), ...]; only those rows are computed
    (the rest of ``out`` is zero)."""
    q, k_cache, v_cache = _c(q), _c(k_cache), _c(v_cache)
    bt, cl = _c(block_tables, np.int32), _c(context_lens, np.int32)
    S, Hq, D = q.shape
    NB, B, Hkv, _ = _dims(k_cache, layout)
    MBS = bt.shape[1]
    out = np.zeros((S, Hq, D), dtype=np.float64)
    w = np.zeros((S, Hq, MBS * B), dtype=np.float64) if want_weights else None
    u = None if units is None else _c(units, np.int32).reshape(-1, 2)
    rc = lib().oracle_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt), _ptr(cl),
                             float(scale), S, Hq, Hkv, D, B, MBS, NB, _DT[dtype],
                             _LAYOUT[layout], _ptr(u), 0 if u is None else u.shape[0], _ptr(out), _ptr(w),
                             MBS * B, _threads(nthreads))
    _check(rc, "oracle_decode")
    return (out, w) if want_weights else out


def decode_dense(q, k, v, context_lens, scale, dtype, units=None, nthreads=None, layout="NHD"):
    """Contiguous-layout decode in fp64; k, v are [S, Smax, Hkv, D] ("NHD")
    or [S, Hkv, Smax, D] ("HND")."""
    q, k, v = _c(q), _c(k), _c(v)
    cl = _c(context_lens, np.int32)
    S, Hq, D = q.shape
    _, Smax, Hkv, _ = _dims(k, layout)
    out = np.zeros((S, Hq, D), dtype=np.float64)
    u = None if units is None else _c(units, np.int32).reshape(-1, 2)
    rc = lib().oracle_decode_dense(_ptr(q), _ptr(k), _ptr(v), _ptr(cl), float(scale),
                                   S, Hq, Hkv, D, Smax, _DT[dtype], _LAYOUT[layout], _ptr(u),
                                   0 if u is None else u.shape[0], _ptr(out),
                                   _threads(nthreads))
    _check(rc, "oracle_decode_dense")
    return out


def decode_split(q, k_cache, v_cache, block_tables, context_lens, scale, dtype,
                 partition_size, nthreads=None, layout="NHD"):
    """Paged decode with the context cut into partitions and merged (fp64)."""
    q, k_cache, v_cache = _c(q), _c(k_cache), _c(v_cache)
    bt, cl = _c(block_tables, np.int32), _c(context_lens, np.int32)
    S, Hq, D = q.shape
    NB, B, Hkv, _ = _dims(k_cache, layout)
    out = np.zeros((S, Hq, D), dtype=np.float64)
    rc = lib().oracle_decode_split(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt), _ptr(cl),
                                   float(scale), S, Hq, Hkv, D, B, bt.shape[1], NB, _DT[dtype],
                                   _LAYOUT[layout], int(partition_size), _ptr(out), _threads(nthreads))
    _check(rc, "oracle_decode_split")
    return out


def prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, dtype,
            nthreads=None, layout="NHD"):
    """Multi-token queries in fp64: q [rows, Hq, D]; sequence s owns rows
    query_start[s] .. query_start[s+1]-1, the last of its context_lens[s]
    cached tokens, and row r of its chunk attends causally to tokens
    0 .. n - T + r.  Returns out [rows, Hq, D] (float64)."""
    q, k_cache, v_cache = _c(q), _c(k_cache), _c(v_cache)
    bt, cl = _c(block_tables, np.int32), _c(context_lens, np.int32)
    qs = _c(query_start, np.int32)
    T, Hq, D = q.shape
    S = cl.shape[0]
    NB, B, Hkv, _ = _dims(k_cache, layout)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    rc = lib().oracle_prefill(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt), _ptr(cl), _ptr(qs),
                              float(scale), S, Hq, Hkv, D, B, bt.shape[1], NB, T, _DT[dtype],
                              _LAYOUT[layout], _ptr(out), _threads(nthreads))
    _check(rc, "oracle_prefill")
    return out


def cache_write(k_new, v_new, k_cache, v_cache, slot_mapping, dtype, layout="NHD"):
    """Returns new (k_cache, v_cache) copies with the tokens written."""
    k_new, v_new = _c(k_new), _c(v_new)
    kc, vc = np.array(k_cache, copy=True, order="C"), np.array(v_cache, copy=True, order="C")
    sm = _c(slot_mapping, np.int32)
    NB, B, Hkv, D = _dims(kc, layout)
    rc = lib().oracle_cache_write(_ptr(k_new), _ptr(v_new), _ptr(kc), _ptr(vc), _ptr(sm),
                                  sm.shape[0], NB, B, Hkv, D, _DT[dtype], _LAYOUT[layout])
    _check(rc, "oracle_cache_write")
    return kc, vc


def copy_blocks(k_cache, v_cache, block_pairs, dtype, layout="NHD"):
    """Returns new (k_cache, v_cache) copies with every (src, dst) block copied
    (a block is one contiguous range in either layout)."""
    kc, vc = np.array(k_cache, copy=True, order="C"), np.array(v_cache, copy=True, order="C")
    bp = _c(block_pairs, np.int32).reshape(-1, 2)
    NB, B, Hkv, D = _dims(kc, layout)
    rc = lib().oracle_copy_blocks(_ptr(kc), _ptr(vc), _ptr(bp), bp.shape[0], NB, B, Hkv, D,
                                  _DT[dtype])
    _check(rc, "oracle_copy_blocks")
    return kc, vc


def copy_blocks_layers(k_caches, v_caches, block_pairs, dtype, layout="NHD"):
    """copy_blocks applied to every layer's pool ([Kwon] §3.4 "Kernel-Level
    Optimizations", item 3: the same pairs for all layers).  Returns new
    lists of pools."""
    out = [copy_blocks(k, v, block_pairs, dtype, layout) for k, v in zip(k_caches, v_caches)]
    return [k for k, _ in out], [v for _, v in out]


def cache_write_layers(k_news, v_news, k_caches, v_caches, slot_mapping, dtype, layout="NHD"):
    """cache_write applied to every layer: layer l's rows into layer l's
    pools at the one slot mapping ([Res] "A paged KV cache, in code": a
    block id names the same position in every layer's pool).  Returns new
    lists of pools."""
    out = [cache_write(kn, vn, k, v, slot_mapping, dtype, layout)
           for kn, vn, k, v in zip(k_news, v_news, k_caches, v_caches)]
    return [k for k, _ in out], [v for _, v in out]


def swap_blocks(dst_k, dst_v, src_k, src_v, block_pairs):
    """Whole blocks from one pool into another, every layer ([Kwon] §3.4
    "Scheduling and Preemption": swapping copies a group's blocks to the CPU
    block pool and back).  For each (src, dst) pair in order and each layer:
    dst[dst_id] = src[src_id], byte for byte; pairs naming a block outside
    either pool are skipped.  Returns new lists of destination pools."""
    bp = np.asarray(block_pairs, dtype=np.int64).reshape(-1, 2)
    ok, ov = [np.array(x, copy=True, order="C") for x in dst_k], [np.array(x, copy=True, order="C") for x in dst_v]
    for layer in range(len(src_k)):
        nsrc, ndst = src_k[layer].shape[0], ok[layer].shape[0]
        for s, d in bp:
            if 0 <= s < nsrc and 0 <= d < ndst:
                ok[layer][d] = src_k[layer][s]
                ov[layer][d] = src_v[layer][s]
    return ok, ov


def half_to_double(bits: int) -> float:
    return lib().oracle_half_to_double(int(bits))


def bf16_to_double(bits: int) -> float:
    return lib().oracle_bf16_to_double(int(bits))
