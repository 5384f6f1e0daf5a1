"""Paged KV-cache decode attention for AMD MI355X (gfx950).

A thin ctypes binding over ``libpa.so`` (C ABI in ``include/pa.h``).  It only
marshals arguments: shapes are read from the tensors, pointers and the
current HIP stream are passed through, and every step of the computation
runs in the library's HIP kernels.  There is no CPU fallback: if the library
is not built, every call raises.

Entry points (same names as the C ABI):
  pa_decode, pa_decode_no_alloc, pa_decode_append, pa_decode_dense, pa_decode_workspace_size,
  pa_decode_shared, pa_decode_shared_workspace_size, pa_cache_write, pa_copy_blocks, pa_copy_blocks_layers, pa_swap_blocks, pa_prefill
and the host block manager (``include/pa_block_manager.h``) as the class
``BlockManager`` in ``paged_kv_cache_pa_amd.block_manager``.
"""
from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

__all__ = ["pa_decode", "pa_decode_no_alloc", "pa_decode_append", "pa_decode_dense", "pa_decode_workspace_size",
           "pa_decode_shared", "pa_decode_shared_workspace_size", "pa_cache_write",
           "pa_copy_blocks", "pa_copy_blocks_layers", "pa_cache_write_layers", "pa_swap_blocks",
           "pa_prefill", "PaError",
           "lib",
           "LIB_PATH", "STATUS"]

STATUS = {0: "PA_OK", -1: "PA_ERR_NULL", -2: "PA_ERR_SHAPE", -3: "PA_ERR_DTYPE",
          -4: "PA_ERR_ALIGN", -5: "PA_ERR_UNSUPPORTED", -6: "PA_ERR_WORKSPACE",
          -7: "PA_ERR_HIP", -8: "PA_ERR_NO_BLOCKS", -9: "PA_ERR_STATE", -10: "PA_ERR_SCRATCH"}

# Bytes of the fixed device array pa_decode_no_alloc uses as its workspace
# (PA_NO_ALLOC_SCRATCH_BYTES in include/pa.h).
NO_ALLOC_SCRATCH_BYTES = 16 << 20


class PaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        msg = lib().pa_status_string(status).decode()
        if status == -7:
            msg += f" ({lib().pa_last_hip_error().decode()})"
        super().__init__(f"{what}: {msg}")


class DecodeParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "num_q_heads", "num_kv_heads", "head_dim", "block_size",
        "max_blocks_per_seq", "num_blocks", "max_context_len", "partition_size", "dtype",
        "layout")]


class PrefillParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "num_q_heads", "num_kv_heads", "head_dim", "block_size",
        "max_blocks_per_seq", "num_blocks", "total_query_rows", "max_query_len",
        "max_context_len", "dtype", "layout")]


class CacheParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_blocks", "block_size", "num_kv_heads", "head_dim", "dtype", "layout")]

LAYOUTS = {"NHD": 0, "HND": 1}  # token-major [.., tokens, Hkv, D] / head-major [.., Hkv, tokens, D]


def _layout(layout) -> int:
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {list(LAYOUTS)}, got {layout!r}")
    return LAYOUTS[layout]


def pool_dims(k_cache, layout="NHD"):
    """(num_blocks, block_size, num_kv_heads, head_dim) of a pool tensor."""
    NB, a, b, D = k_cache.shape
    return (NB, a, b, D) if _layout(layout) == 0 else (NB, b, a, D)


_lib = None


def lib():
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        # torch brings its own HIP runtime (soname libamdhip64.so.7).  Load it
        # before libpa.so so that the loader binds libpa's dependency to that
        # same copy: tensors, streams and these kernels must share one
        # runtime.  Loaded the other way round, the process would hold two
        # HIP runtimes and this library's launches would not see the device.
        import torch  # noqa: F401

        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"HIP library {LIB_PATH} is not built; run `python -m paged_kv_cache_pa_amd.build` "
                "(or __graft_entry__.build()) first. There is no CPU fallback.")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        DP, CP = ctypes.POINTER(DecodeParams), ctypes.POINTER(CacheParams)
        L.pa_decode_workspace_size.argtypes = [DP, ctypes.POINTER(SZ)]
        L.pa_decode.argtypes = [P, P, P, P, P, ctypes.c_float, P, DP, P, SZ, P]
        L.pa_decode_no_alloc.argtypes = [P, P, P, P, P, ctypes.c_float, P, DP, P]
        L.pa_decode_shared_workspace_size.argtypes = [DP, ctypes.POINTER(SZ)]
        L.pa_decode_shared.argtypes = [P, P, P, P, P, P, P, I32, I32, ctypes.c_float, P, DP, P, SZ, P]
        L.pa_decode_append.argtypes = [P, P, P, P, P, P, P, ctypes.c_float, P, DP, P, SZ, P]
        L.pa_decode_dense.argtypes = [P, P, P, P, ctypes.c_float, P, DP, I32, P, SZ, P]
        L.pa_cache_write.argtypes = [P, P, P, P, P, I32, CP, P]
        L.pa_copy_blocks.argtypes = [P, P, P, I32, CP, P]
        L.pa_copy_blocks_layers.argtypes = [P, P, I32, P, I32, CP, P]
        L.pa_cache_write_layers.argtypes = [P, P, P, P, I32, P, I32, CP, P]
        L.pa_prefill.argtypes = [P, P, P, P, P, P, ctypes.c_float, P,
                                 ctypes.POINTER(PrefillParams), P]
        L.pa_swap_blocks.argtypes = [P, P, I32, P, P, I32, I32, P, I32, CP, P]
        for f in ("pa_decode_workspace_size", "pa_decode", "pa_decode_no_alloc",
                  "pa_decode_shared_workspace_size", "pa_decode_shared",
                  "pa_decode_append", "pa_decode_dense",
                  "pa_cache_write",
                  "pa_copy_blocks", "pa_copy_blocks_layers", "pa_cache_write_layers",
                  "pa_swap_blocks", "pa_prefill"):
            getattr(L, f).restype = ctypes.c_int
        L.pa_status_string.argtypes = [ctypes.c_int]
        L.pa_status_string.restype = ctypes.c_char_p
        L.pa_build_info.argtypes = []
        L.pa_build_info.restype = ctypes.c_char_p
        L.pa_last_hip_error.argtypes = []
        L.pa_last_hip_error.restype = ctypes.c_char_p
        from .block_manager import declare as _declare_bm

        _declare_bm(L)
        _lib = L
    return _lib


def _dtype_code(t) -> int:
    import torch

    codes = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch

        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:  # the current stream's handle without a Stream object (~0.1 us)
            return ctypes.c_void_p(raw(torch._C._cuda_getDevice()))
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dim=None, dtype=None):
    import torch

    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _check(rc, what):
    if rc != 0:
        raise PaError(rc, what)


def _same_head_dim(q, pool, name):
    """The kernels index q, out and the pool with one head dim: a pool whose
    rows differ from q's would be read out of bounds, so refuse it here."""
    if pool.shape[-1] != q.shape[-1]:
        raise ValueError(f"head dim of {name} ({pool.shape[-1]}) differs from q's ({q.shape[-1]})")


def _params_paged(q, k_cache, block_tables, max_context_len, partition_size, layout):
    S, Hq, D = q.shape
    _same_head_dim(q, k_cache, "k_cache")
    NB, B, Hkv, _ = pool_dims(k_cache, layout)
    MBS = block_tables.shape[1]
    return DecodeParams(S, Hq, Hkv, D, B, MBS, NB,
                        MBS * B if max_context_len is None else int(max_context_len),
                        int(partition_size), _dtype_code(q), _layout(layout))


def pa_decode_workspace_size(params: DecodeParams) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().pa_decode_workspace_size(ctypes.byref(params), ctypes.byref(n)),
           "pa_decode_workspace_size")
    return int(n.value)


def _workspace(params, workspace, device):
    import torch

    # no split: no workspace (the size query is skipped, it would return 0)
    need = pa_decode_workspace_size(params) if params.partition_size else 0
    if need and workspace is None:
        workspace = torch.empty((need + 3) // 4, dtype=torch.float32, device=device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return workspace, nbytes


def pa_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out, *,
              max_context_len=None, partition_size=0, workspace=None, stream=None,
              layout="NHD"):
    """Paged decode attention; writes ``out`` [S, Hq, D] and returns it.

    q [S, Hq, D]; k_cache, v_cache [NB, B, Hkv, D] (layout "NHD") or
    [NB, Hkv, B, D] ("HND"); block_tables [S, MBS] int32; context_lens [S]
    int32.  ``max_context_len`` (host-known bound on
    every context length, default MBS * B) sizes the split-K grid when
    ``partition_size`` > 0.  A workspace tensor is allocated by torch if one
    is needed and none is given."""
    import torch

    _need(q, "q", 3)
    _need(k_cache, "k_cache", 4, q.dtype)
    _need(v_cache, "v_cache", 4, q.dtype)
    _need(block_tables, "block_tables", 2, torch.int32)
    _need(context_lens, "context_lens", 1, torch.int32)
    _need(out, "out", 3, q.dtype)
    if v_cache.shape != k_cache.shape or out.shape != q.shape:
        raise ValueError("shape mismatch between k_cache/v_cache or q/out")
    if block_tables.shape[0] != q.shape[0] or context_lens.shape[0] != q.shape[0]:
        raise ValueError("block_tables / context_lens must have one row per sequence")
    p = _params_paged(q, k_cache, block_tables, max_context_len, partition_size, layout)
    ws, nbytes = _workspace(p, workspace, q.device)
    _check(lib().pa_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                           _ptr(context_lens), float(scale), _ptr(out), ctypes.byref(p),
                           _ptr(ws), nbytes, _stream(stream)), "pa_decode")
    return out


def pa_decode_shared_workspace_size(params: DecodeParams) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().pa_decode_shared_workspace_size(ctypes.byref(params), ctypes.byref(n)),
           "pa_decode_shared_workspace_size")
    return int(n.value)


def pa_decode_shared(q, k_cache, v_cache, block_tables, context_lens, group_start, group_shared,
                     scale, out, *, max_shared_blocks=None, max_context_len=None,
                     partition_size=512, workspace=None, stream=None, layout="NHD"):
    """pa_decode for batches whose sequences share leading blocks (parallel
    samples, beams, a common prefix): group i is sequences group_start[i] ..
    group_start[i+1] - 1 (int32 [G + 1], covering the batch in order), whose
    first group_shared[i] table entries (int32 [G]) name the same blocks.
    Blocks in a group's shared prefix are read once per group.
    ``max_shared_blocks`` (host bound on group_shared, default MBS) sizes the
    grouped grid; ``partition_size`` (> 0) is the split-K partition, and only
    whole partitions inside a shared prefix are shared.  16-bit types."""
    import torch

    _need(q, "q", 3)
    _need(k_cache, "k_cache", 4, q.dtype)
    _need(v_cache, "v_cache", 4, q.dtype)
    _need(block_tables, "block_tables", 2, torch.int32)
    _need(context_lens, "context_lens", 1, torch.int32)
    _need(group_start, "group_start", 1, torch.int32)
    _need(group_shared, "group_shared", 1, torch.int32)
    _need(out, "out", 3, q.dtype)
    if v_cache.shape != k_cache.shape or out.shape != q.shape:
        raise ValueError("shape mismatch between k_cache/v_cache or q/out")
    if block_tables.shape[0] != q.shape[0] or context_lens.shape[0] != q.shape[0]:
        raise ValueError("block_tables / context_lens must have one row per sequence")
    n_groups = group_shared.shape[0]
    if group_start.shape[0] != n_groups + 1:
        raise ValueError("group_start must have one entry more than group_shared")
    p = _params_paged(q, k_cache, block_tables, max_context_len, partition_size, layout)
    if max_shared_blocks is None:
        max_shared_blocks = p.max_blocks_per_seq
    need = pa_decode_shared_workspace_size(p)
    if workspace is None:
        workspace = torch.empty((need + 3) // 4, dtype=torch.float32, device=q.device)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().pa_decode_shared(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                  _ptr(context_lens), _ptr(group_start), _ptr(group_shared),
                                  int(n_groups), int(max_shared_blocks), float(scale), _ptr(out),
                                  ctypes.byref(p), _ptr(workspace), nbytes, _stream(stream)),
           "pa_decode_shared")
    return out


def pa_decode_no_alloc(q, k_cache, v_cache, block_tables, context_lens, scale, out, *,
                       max_context_len=None, partition_size=0, stream=None, layout="NHD"):
    """pa_decode with no workspace: the split-K partials go to the library's
    fixed 16 MiB device array (NO_ALLOC_SCRATCH_BYTES), so neither this call
    nor the library allocates anything.  Calls overlapping on one device
    share that array (order them on one stream)."""
    import torch

    _need(q, "q", 3)
    _need(k_cache, "k_cache", 4, q.dtype)
    _need(v_cache, "v_cache", 4, q.dtype)
    _need(block_tables, "block_tables", 2, torch.int32)
    _need(context_lens, "context_lens", 1, torch.int32)
    _need(out, "out", 3, q.dtype)
    if v_cache.shape != k_cache.shape or out.shape != q.shape:
        raise ValueError("shape mismatch between k_cache/v_cache or q/out")
    if block_tables.shape[0] != q.shape[0] or context_lens.shape[0] != q.shape[0]:
        raise ValueError("block_tables / context_lens must have one row per sequence")
    p = _params_paged(q, k_cache, block_tables, max_context_len, partition_size, layout)
    _check(lib().pa_decode_no_alloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                    _ptr(context_lens), float(scale), _ptr(out), ctypes.byref(p),
                                    _stream(stream)), "pa_decode_no_alloc")
    return out


def pa_decode_append(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, out,
                     *, max_context_len=None, partition_size=0, workspace=None, stream=None,
                     layout="NHD"):
    """Write each sequence's newest token (k_new, v_new [S, Hkv, D], position
    context_lens[s] - 1) into its slot and attend, in one launch; the same
    result and pool contents as pa_cache_write followed by pa_decode."""
    import torch

    _need(q, "q", 3)
    _need(k_new, "k_new", 3, q.dtype)
    _need(v_new, "v_new", 3, q.dtype)
    _need(k_cache, "k_cache", 4, q.dtype)
    _need(v_cache, "v_cache", 4, q.dtype)
    _need(block_tables, "block_tables", 2, torch.int32)
    _need(context_lens, "context_lens", 1, torch.int32)
    _need(out, "out", 3, q.dtype)
    if v_cache.shape != k_cache.shape or out.shape != q.shape or v_new.shape != k_new.shape:
        raise ValueError("shape mismatch between k_cache/v_cache, q/out or k_new/v_new")
    if block_tables.shape[0] != q.shape[0] or context_lens.shape[0] != q.shape[0]:
        raise ValueError("block_tables / context_lens must have one row per sequence")
    p = _params_paged(q, k_cache, block_tables, max_context_len, partition_size, layout)
    if tuple(k_new.shape) != (q.shape[0], p.num_kv_heads, p.head_dim):
        raise ValueError("k_new / v_new must be [S, Hkv, D]")
    ws, nbytes = _workspace(p, workspace, q.device)
    _check(lib().pa_decode_append(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                  _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
                                  float(scale), _ptr(out), ctypes.byref(p), _ptr(ws), nbytes,
                                  _stream(stream)), "pa_decode_append")
    return out


def pa_decode_dense(q, k, v, context_lens, scale, out, *, max_context_len=None,
                    partition_size=0, workspace=None, stream=None, layout="NHD"):
    """Contiguous-layout twin: k, v [S, max_seq_len, Hkv, D] ("NHD") or
    [S, Hkv, max_seq_len, D] ("HND")."""
    import torch

    _need(q, "q", 3)
    _need(k, "k", 4, q.dtype)
    _need(v, "v", 4, q.dtype)
    _need(context_lens, "context_lens", 1, torch.int32)
    _need(out, "out", 3, q.dtype)
    if v.shape != k.shape or out.shape != q.shape or k.shape[0] != q.shape[0]:
        raise ValueError("shape mismatch")
    S, Hq, D = q.shape
    _same_head_dim(q, k, "k")
    _, Smax, Hkv, _ = pool_dims(k, layout)
    p = DecodeParams(S, Hq, Hkv, D, 16, 1, 1,
                     Smax if max_context_len is None else int(max_context_len),
                     int(partition_size), _dtype_code(q), _layout(layout))
    workspace, nbytes = _workspace(p, workspace, q.device)
    _check(lib().pa_decode_dense(_ptr(q), _ptr(k), _ptr(v), _ptr(context_lens), float(scale),
                                 _ptr(out), ctypes.byref(p), int(Smax), _ptr(workspace), nbytes,
                                 _stream(stream)), "pa_decode_dense")
    return out


def _cache_params(k_cache, layout):
    NB, B, Hkv, D = pool_dims(k_cache, layout)
    return CacheParams(NB, B, Hkv, D, _dtype_code(k_cache), _layout(layout))


def pa_cache_write(k_new, v_new, k_cache, v_cache, slot_mapping, *, stream=None, layout="NHD"):
    """Scatter new tokens' K/V rows ([N, Hkv, D]) into their slots."""
    import torch

    _need(k_cache, "k_cache", 4)
    _need(v_cache, "v_cache", 4, k_cache.dtype)
    _need(k_new, "k_new", 3, k_cache.dtype)
    _need(v_new, "v_new", 3, k_cache.dtype)
    _need(slot_mapping, "slot_mapping", 1, torch.int32)
    p = _cache_params(k_cache, layout)
    if k_new.shape != v_new.shape or tuple(k_new.shape[1:]) != (p.num_kv_heads, p.head_dim) or \
            slot_mapping.shape[0] != k_new.shape[0] or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    _check(lib().pa_cache_write(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                _ptr(slot_mapping), int(k_new.shape[0]), ctypes.byref(p),
                                _stream(stream)), "pa_cache_write")


def pa_copy_blocks(k_cache, v_cache, block_pairs, *, stream=None, layout="NHD"):
    """Copy whole K and V blocks for every (src, dst) row of block_pairs [n, 2]."""
    import torch

    _need(k_cache, "k_cache", 4)
    _need(v_cache, "v_cache", 4, k_cache.dtype)
    _need(block_pairs, "block_pairs", 2, torch.int32)
    if block_pairs.shape[1] != 2 or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    p = _cache_params(k_cache, layout)
    _check(lib().pa_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(block_pairs),
                                int(block_pairs.shape[0]), ctypes.byref(p), _stream(stream)),
           "pa_copy_blocks")


def _ptr_array(tensors):
    arr = (ctypes.c_void_p * len(tensors))(*[t.data_ptr() for t in tensors])
    return arr


def _pools(ks, vs, name, allow_host=False):
    """Per-layer pools: same shape and dtype, device tensors (or pinned host
    tensors where ``allow_host``)."""
    if len(ks) == 0 or len(ks) != len(vs):
        raise ValueError(f"{name}: one K and one V pool per layer, at least one layer")
    for t in list(ks) + list(vs):
        if t.shape != ks[0].shape or t.dtype != ks[0].dtype or t.dim() != 4:
            raise ValueError(f"{name}: every pool must match the first one's shape and dtype")
        if not t.is_contiguous():
            raise ValueError(f"{name}: pools must be contiguous")
        if not (t.is_cuda or (allow_host and t.is_pinned())):
            raise ValueError(f"{name}: pools must be GPU tensors" +
                             (" or pinned host tensors" if allow_host else ""))


def pa_copy_blocks_layers(k_caches, v_caches, block_pairs, *, stream=None, layout="NHD"):
    """pa_copy_blocks over every layer's pool (lists of [NB, ...] tensors) in
    one launch per 64 layers."""
    import torch

    _pools(k_caches, v_caches, "pa_copy_blocks_layers")
    _need(block_pairs, "block_pairs", 2, torch.int32)
    if block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be [n, 2]")
    p = _cache_params(k_caches[0], layout)
    _check(lib().pa_copy_blocks_layers(_ptr_array(k_caches), _ptr_array(v_caches),
                                       len(k_caches), _ptr(block_pairs),
                                       int(block_pairs.shape[0]), ctypes.byref(p),
                                       _stream(stream)), "pa_copy_blocks_layers")


def pa_cache_write_layers(k_news, v_news, k_caches, v_caches, slot_mapping, *, stream=None,
                          layout="NHD"):
    """pa_cache_write for every layer (lists of [N, Hkv, D] rows and of
    [NB, ...] pools, one slot mapping) in one launch per 64 layers."""
    import torch

    _pools(k_caches, v_caches, "pa_cache_write_layers")
    if len(k_news) != len(k_caches) or len(v_news) != len(k_caches):
        raise ValueError("pa_cache_write_layers: one K and one V row tensor per layer")
    _need(slot_mapping, "slot_mapping", 1, torch.int32)
    p = _cache_params(k_caches[0], layout)
    for t in list(k_news) + list(v_news):
        _need(t, "k_new / v_new", 3, k_caches[0].dtype)
        if tuple(t.shape) != (slot_mapping.shape[0], p.num_kv_heads, p.head_dim):
            raise ValueError("pa_cache_write_layers: rows must be [N, Hkv, D], N = len(slot_mapping)")
    _check(lib().pa_cache_write_layers(_ptr_array(k_news), _ptr_array(v_news),
                                       _ptr_array(k_caches), _ptr_array(v_caches), len(k_caches),
                                       _ptr(slot_mapping), int(slot_mapping.shape[0]),
                                       ctypes.byref(p), _stream(stream)), "pa_cache_write_layers")


def pa_swap_blocks(dst_k, dst_v, src_k, src_v, block_pairs, *, stream=None, layout="NHD"):
    """Move blocks between two pools (lists per layer, GPU or pinned host
    tensors) for every (src, dst) row of block_pairs [n, 2] (a GPU tensor)."""
    import torch

    _pools(dst_k, dst_v, "pa_swap_blocks dst", allow_host=True)
    _pools(src_k, src_v, "pa_swap_blocks src", allow_host=True)
    if len(dst_k) != len(src_k):
        raise ValueError("pa_swap_blocks: same number of layers on both sides")
    _need(block_pairs, "block_pairs", 2, torch.int32)
    if block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be [n, 2]")
    ps, pd = _cache_params(src_k[0], layout), _cache_params(dst_k[0], layout)
    if (ps.block_size, ps.num_kv_heads, ps.head_dim, ps.dtype) != \
            (pd.block_size, pd.num_kv_heads, pd.head_dim, pd.dtype):
        raise ValueError("pa_swap_blocks: both pools need the same block geometry and dtype")
    _check(lib().pa_swap_blocks(_ptr_array(dst_k), _ptr_array(dst_v), pd.num_blocks,
                                _ptr_array(src_k), _ptr_array(src_v), ps.num_blocks,
                                len(src_k), _ptr(block_pairs), int(block_pairs.shape[0]),
                                ctypes.byref(ps), _stream(stream)), "pa_swap_blocks")


def pa_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, out, *,
               max_query_len=None, max_context_len=None, stream=None, layout="NHD"):
    """Multi-token (prompt / chunked-prefill) attention over the paged cache;
    writes ``out`` [rows, Hq, D] and returns it.  Sequence s owns q rows
    query_start[s] .. query_start[s+1]-1, the last of its context_lens[s]
    cached tokens; row r of its chunk attends causally.  ``max_query_len``
    and ``max_context_len`` are host-known bounds (default: all rows / the
    table capacity)."""
    import torch

    _need(q, "q", 3)
    _need(k_cache, "k_cache", 4, q.dtype)
    _need(v_cache, "v_cache", 4, q.dtype)
    _need(block_tables, "block_tables", 2, torch.int32)
    _need(context_lens, "context_lens", 1, torch.int32)
    _need(query_start, "query_start", 1, torch.int32)
    _need(out, "out", 3, q.dtype)
    if v_cache.shape != k_cache.shape or out.shape != q.shape:
        raise ValueError("shape mismatch between k_cache/v_cache or q/out")
    S = context_lens.shape[0]
    if block_tables.shape[0] != S or query_start.shape[0] != S + 1:
        raise ValueError("block_tables [S, MBS], context_lens [S], query_start [S + 1]")
    _same_head_dim(q, k_cache, "k_cache")
    NB, B, Hkv, D = pool_dims(k_cache, layout)
    MBS = block_tables.shape[1]
    rows = q.shape[0]
    p = PrefillParams(S, q.shape[1], Hkv, D, B, MBS, NB, rows,
                      rows if max_query_len is None else int(max_query_len),
                      MBS * B if max_context_len is None else int(max_context_len),
                      _dtype_code(q), _layout(layout))
    _check(lib().pa_prefill(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                            _ptr(context_lens), _ptr(query_start), float(scale), _ptr(out),
                            ctypes.byref(p), _stream(stream)), "pa_prefill")
    return out
