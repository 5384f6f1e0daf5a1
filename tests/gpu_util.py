"""Host <-> device marshalling for the GPU tests (numpy storage arrays, bf16
as uint16 bit patterns, to torch tensors on cuda:0 and back)."""
from __future__ import annotations

import numpy as np

import workloads as W


def dev():
    import torch

    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dtype: str | None = None):
    import torch

    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev())
    return torch.from_numpy(a).to(dev())


def to_host(t, dtype: str) -> np.ndarray:
    """Device tensor -> numpy storage array (same layout as the generators')."""
    import torch

    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def torch_dtype(dtype: str):
    import torch

    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def empty_out(p: W.Paged):
    import torch

    return torch.full(p.q.shape, float("nan"), dtype=torch_dtype(p.dtype), device=dev())


def head_major(a: np.ndarray) -> np.ndarray:
    """[X, tokens, Hkv, D] -> [X, Hkv, tokens, D]."""
    return np.ascontiguousarray(np.swapaxes(a, 1, 2))


def in_layout(a: np.ndarray, layout: str) -> np.ndarray:
    return a if layout == "NHD" else head_major(a)


def upload(p: W.Paged, layout="NHD"):
    """q, k_cache, v_cache, block_tables, context_lens on the device; the pool
    in the requested layout (the generators build token-major pools)."""
    return (to_dev(p.q, p.dtype), to_dev(in_layout(p.k_cache, layout), p.dtype),
            to_dev(in_layout(p.v_cache, layout), p.dtype), to_dev(p.block_tables),
            to_dev(p.context_lens))


def run_decode(p: W.Paged, partition_size=None, max_context_len=None, tensors=None,
               layout="NHD"):
    import torch

    import paged_kv_cache_pa_amd as pa

    q, k, v, bt, cl = tensors or upload(p, layout)
    out = empty_out(p)
    mcl = int(p.context_lens.max(initial=0)) if max_context_len is None else max_context_len
    ps = p.partition_size if partition_size is None else partition_size
    pa.pa_decode(q, k, v, bt, cl, p.scale, out, max_context_len=mcl, partition_size=ps,
                 layout=layout)
    torch.cuda.synchronize()
    return to_host(out, p.dtype)


def f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return W.to_f64(a, dtype)
