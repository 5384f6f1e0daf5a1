"""Seeded random sweep over the whole parameter space, against the fp64
oracle: data type, head dim, query / kv heads (every group size the
matrix-core kernel takes, up to 16, and the VALU one), block size, pool layout,
split-K partition size, lengths (including 0, 1 and block edges), for
pa_decode, pa_decode_append and pa_prefill.  Each case is small enough for
the oracle; the case's parameters are printed before it runs."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import empty_out, f64, in_layout, to_dev, to_host, torch_dtype
from helpers import assert_fp_close, same_bits

pytestmark = pytest.mark.gpu

N_CASES = 48


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def draw(seed):
    r = np.random.default_rng(1000 + seed)
    dtype = ["f32", "f16", "bf16"][seed % 3]
    D = int(r.choice([64, 128]))
    G = int(r.integers(1, 9 if dtype == "f32" else 17))   # up to 16 on the matrix cores
    hkv = int(r.integers(1, 4))
    B = int(2 ** r.integers(0, 9))
    S = int(r.integers(1, 7))
    edges = [0, 1, B - 1, B, B + 1, 15, 16, 17, 255, 256, 257]
    lens = [int(r.choice(edges)) if r.random() < 0.4 else int(r.integers(0, 900)) for _ in range(S)]
    lens = [max(0, n) for n in lens]
    ps = int(r.choice([0, 0, max(B, 16), 64, 256]))
    if ps % B:
        ps = 0
    layout = str(r.choice(["NHD", "HND"]))
    return dict(dtype=dtype, D=D, G=G, hkv=hkv, B=B, lens=lens, ps=ps, layout=layout)


def fp_check(got, ref, dtype, what):
    if dtype == "f32":
        g = f64(got, dtype)
        den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
        rel = np.abs(g - ref).max(axis=-1) / den
        assert np.isfinite(g).all() and rel.max() <= 1e-5, (what, rel.max())
    else:
        assert_fp_close(f64(got, dtype), ref, dtype, what)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_case(seed):
    import torch

    import paged_kv_cache_pa_amd as pa

    c = draw(seed)
    print("case", seed, c, flush=True)
    dt, D, G, hkv, B, lens, ps, lay = (c["dtype"], c["D"], c["G"], c["hkv"], c["B"], c["lens"],
                                       c["ps"], c["layout"])
    hq = G * hkv
    p = W.random_paged(2000 + seed, dt, lens, hq, hkv, D, block_size=B, extra_blocks=4)
    mcl = max(1, int(p.context_lens.max()))
    k, v = to_dev(in_layout(p.k_cache, lay), dt), to_dev(in_layout(p.v_cache, lay), dt)
    q, bt, cl = to_dev(p.q, dt), to_dev(p.block_tables), to_dev(p.context_lens)

    # decode
    out = empty_out(p)
    pa.pa_decode(q, k, v, bt, cl, p.scale, out, max_context_len=mcl, partition_size=ps,
                 layout=lay)
    torch.cuda.synchronize()
    ref = oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, dt)
    fp_check(to_host(out, dt), ref, dt, f"decode {c}")

    # decode_append: the newest row of every sequence comes in k_new / v_new
    # (its pool slot poisoned first); pools must end as the oracle's write
    rng = np.random.default_rng(3000 + seed)
    S = len(lens)
    kn, vn = W.randn(rng, (S, hkv, D), dt), W.randn(rng, (S, hkv, D), dt)
    slots = np.array([p.block_tables[s, (n - 1) // B] * B + (n - 1) % B if n else -1
                      for s, n in enumerate(lens)], np.int32)
    k0 = p.k_cache.copy()
    v0 = p.v_cache.copy()
    nanrow = W.nan_fill((hkv, D), dt)
    for s, n in enumerate(lens):
        if n:
            b, o = p.block_tables[s, (n - 1) // B], (n - 1) % B
            k0[b, o], v0[b, o] = nanrow, nanrow
    k2, v2 = to_dev(in_layout(k0, lay), dt), to_dev(in_layout(v0, lay), dt)
    out2 = empty_out(p)
    pa.pa_decode_append(q, to_dev(kn, dt), to_dev(vn, dt), k2, v2, bt, cl, p.scale, out2,
                        max_context_len=mcl, partition_size=ps, layout=lay)
    torch.cuda.synchronize()
    kw, vw = oracle.cache_write(kn, vn, k0, v0, slots, dt)
    assert same_bits(to_host(k2, dt), in_layout(kw, lay)), f"append pool {c}"
    assert same_bits(to_host(v2, dt), in_layout(vw, lay)), f"append pool {c}"
    ref2 = oracle.decode(p.q, kw, vw, p.block_tables, p.context_lens, p.scale, dt)
    fp_check(to_host(out2, dt), ref2, dt, f"decode_append {c}")

    # prefill (16-bit types): the last min(n, 40) tokens of each sequence
    if dt != "f32":
        chunks = np.minimum(np.array(lens), 40).astype(np.int32)
        qs = np.zeros(S + 1, np.int32)
        qs[1:] = np.cumsum(chunks)
        qp = W.randn(rng, (max(1, int(qs[-1])), hq, D), dt)
        outp = torch.full(qp.shape, float("nan"), dtype=torch_dtype(dt), device=k.device)
        pa.pa_prefill(to_dev(qp, dt), k, v, bt, cl, to_dev(qs), p.scale, outp, layout=lay)
        torch.cuda.synchronize()
        if int(qs[-1]):
            refp = oracle.prefill(qp[: int(qs[-1])], p.k_cache, p.v_cache, p.block_tables,
                                  p.context_lens, qs, p.scale, dt)
            fp_check(to_host(outp, dt)[: int(qs[-1])], refp, dt, f"prefill {c}")
