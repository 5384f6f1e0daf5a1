"""Test-side helpers: an independent numpy/scipy route to the same attention
(library primitives only: fancy indexing for the gather, scipy's softmax),
tolerance checks, and small pool builders.  Nothing here is used by the
library or by the oracle."""
from __future__ import annotations

import numpy as np
import scipy.special

import workloads as W


def np_reference(p: W.Paged, units=None):
    """out [S, Hq, D] in fp64 by numpy gather + scipy softmax."""
    S, Hq, D = p.q.shape
    B = p.block_size
    G = Hq // p.num_kv_heads
    out = np.zeros((S, Hq, D))
    todo = units if units is not None else [(s, h) for s in range(S) for h in range(Hq)]
    qf = W.to_f64(p.q, p.dtype)
    for s, h in todo:
        n = int(p.context_lens[s])
        if n == 0:
            continue
        t = np.arange(n)
        blk = p.block_tables[s, t // B]
        off = t % B
        g = h // G
        K = W.to_f64(p.k_cache[blk, off, g], p.dtype)
        V = W.to_f64(p.v_cache[blk, off, g], p.dtype)
        a = scipy.special.softmax(p.scale * (K @ qf[s, h]))
        out[s, h] = a @ V
    return out


def bits(a: np.ndarray) -> np.ndarray:
    """Raw bit patterns, so NaN payloads compare too."""
    a = np.ascontiguousarray(a)
    return a.view({1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[a.dtype.itemsize])


def same_bits(a, b) -> bool:
    a, b = np.asarray(a), np.asarray(b)
    return a.shape == b.shape and a.dtype.itemsize == b.dtype.itemsize and np.array_equal(bits(a), bits(b))


def assert_fp_close(got, ref, dtype, what=""):
    """The attention tolerance: fp16/bf16 elementwise |err| <= 2e-3 + 1e-2 |ref|;
    fp32 row-normwise max|err| / max|ref| <= 1e-5 per (s, h) row."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    if dtype in ("f16", "bf16"):
        bound = 2e-3 + 1e-2 * np.abs(ref)
        bad = err > bound
        assert not bad.any(), (f"{what}: {int(bad.sum())} elements out of tolerance, "
                               f"max err {err.max():.3e}, worst ratio {(err / bound).max():.3f}")
    else:
        num = err.max(axis=-1)
        den = np.abs(ref).max(axis=-1)
        rel = np.where(den > 0, num / np.where(den > 0, den, 1), num)
        assert (rel <= 1e-5).all(), f"{what}: row-normwise rel err {rel.max():.3e} > 1e-5"


def empty_pool(nb, b, hkv, d, dtype):
    return W.nan_fill((nb, b, hkv, d), dtype), W.nan_fill((nb, b, hkv, d), dtype)
