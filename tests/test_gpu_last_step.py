"""The partly filled last step of a sequence rides in the decode kernel's
one-step-ahead load pipeline, as the last step of the wave whose turn it is.
Where it falls depends on the number of full steps modulo the waves per
workgroup, so the lengths here are 16 k + t for every k up to 2 * waves + 1
and t in {0, 1, 15}, under both wave counts the launcher picks: 4 (a grid
past 1024 workgroups, longest-first ranked) and 8 (a small grid).  Plain
decode and decode_append (newest row from k_new / v_new, its slot poisoned
first) against the fp64 oracle; the pools after append bit-exact."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import empty_out, f64, in_layout, to_dev, to_host
from helpers import assert_fp_close, same_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _lengths(waves, count):
    base = [16 * k + t for k in range(2 * waves + 2) for t in (0, 1, 15)]
    rng = np.random.default_rng(77 + waves)
    extra = rng.integers(1, 16 * (2 * waves + 2), size=max(0, count - len(base))).tolist()
    return (base + extra)[:count]


# (waves the launcher picks, sequences, kv heads): 36 x 32 = 1152 workgroups
# do not fit at once (4 waves, ranked); 54 x 8 = 432 do (8 waves)
@pytest.mark.parametrize("waves,S,hkv", [(4, 36, 32), (8, 54, 8)])
@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_last_step_positions(waves, S, hkv, layout):
    import torch

    import paged_kv_cache_pa_amd as pa

    dt, D, B = "f16", 64, 16
    lens = _lengths(waves, S)
    print("case", waves, S, hkv, layout, flush=True)
    p = W.random_paged(5150 + waves, dt, lens, hkv, hkv, D, block_size=B, extra_blocks=2)
    mcl = max(1, int(p.context_lens.max()))
    k, v = to_dev(in_layout(p.k_cache, layout), dt), to_dev(in_layout(p.v_cache, layout), dt)
    q, bt, cl = to_dev(p.q, dt), to_dev(p.block_tables), to_dev(p.context_lens)

    out = empty_out(p)
    pa.pa_decode(q, k, v, bt, cl, p.scale, out, max_context_len=mcl, layout=layout)
    torch.cuda.synchronize()
    ref = oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, dt)
    assert_fp_close(f64(to_host(out, dt), dt), ref, dt, f"decode waves {waves} {layout}")

    # append: position n - 1 comes from k_new / v_new; its slot is poisoned
    rng = np.random.default_rng(5160 + waves)
    kn, vn = W.randn(rng, (S, hkv, D), dt), W.randn(rng, (S, hkv, D), dt)
    slots = np.array([p.block_tables[s, (n - 1) // B] * B + (n - 1) % B if n else -1
                      for s, n in enumerate(lens)], np.int32)
    k0, v0 = p.k_cache.copy(), p.v_cache.copy()
    nanrow = W.nan_fill((hkv, D), dt)
    for s, n in enumerate(lens):
        if n:
            b, o = p.block_tables[s, (n - 1) // B], (n - 1) % B
            k0[b, o], v0[b, o] = nanrow, nanrow
    k2, v2 = to_dev(in_layout(k0, layout), dt), to_dev(in_layout(v0, layout), dt)
    out2 = empty_out(p)
    pa.pa_decode_append(q, to_dev(kn, dt), to_dev(vn, dt), k2, v2, bt, cl, p.scale, out2,
                        max_context_len=mcl, layout=layout)
    torch.cuda.synchronize()
    kw, vw = oracle.cache_write(kn, vn, k0, v0, slots, dt)
    assert same_bits(to_host(k2, dt), in_layout(kw, layout)), "append K pool"
    assert same_bits(to_host(v2, dt), in_layout(vw, layout)), "append V pool"
    ref2 = oracle.decode(p.q, kw, vw, p.block_tables, p.context_lens, p.scale, dt)
    assert_fp_close(f64(to_host(out2, dt), dt), ref2, dt, f"decode_append waves {waves} {layout}")
