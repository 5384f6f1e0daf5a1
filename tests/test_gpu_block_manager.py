"""The host block manager driving the device entry points, step by step.

Each decode iteration: the C++ manager reserves slots for every running
sequence (forks, copy-on-write and frees happen in between), then
pa_copy_blocks applies its pairs, pa_cache_write stores the new tokens at
its slots and pa_decode attends through its tables.  The same pairs, slots
and tables are replayed on host arrays with the fp64 oracle: the pools must
match bit for bit after every step and the attention within tolerance."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import f64, in_layout, to_dev, to_host
from helpers import assert_fp_close, same_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("dtype,layout,B", [("f16", "HND", 16), ("bf16", "NHD", 16),
                                            ("f16", "NHD", 4), ("bf16", "HND", 32)])
def test_manager_driven_decode_iterations(dtype, layout, B):
    import torch

    import paged_kv_cache_pa_amd as pa
    from paged_kv_cache_pa_amd.block_manager import BlockManager

    rng = np.random.default_rng(41)
    NB, Hq, Hkv, D, MBS = 96, 8, 4, 128, 64
    scale = 1 / np.sqrt(D)
    bm = BlockManager(NB, 0, B)
    # host pools in the requested layout, every slot NaN until written
    kh = in_layout(W.nan_fill((NB, B, Hkv, D), dtype), layout)
    vh = in_layout(W.nan_fill((NB, B, Hkv, D), dtype), layout)
    kd, vd = to_dev(kh, dtype), to_dev(vh, dtype)

    def step(seqs, ks, check_decode=True):
        nonlocal kh, vh
        slots, pairs = bm.reserve(seqs, ks)
        n = int(sum(ks))
        kn, vn = W.randn(rng, (n, Hkv, D), dtype), W.randn(rng, (n, Hkv, D), dtype)
        if len(pairs):
            pa.pa_copy_blocks(kd, vd, to_dev(np.ascontiguousarray(pairs)), layout=layout)
            kh, vh = oracle.copy_blocks(kh, vh, pairs, dtype, layout=layout)
        pa.pa_cache_write(to_dev(kn, dtype), to_dev(vn, dtype), kd, vd, to_dev(slots),
                          layout=layout)
        kh, vh = oracle.cache_write(kn, vn, kh, vh, slots, dtype, layout=layout)
        torch.cuda.synchronize()
        assert same_bits(to_host(kd, dtype), kh) and same_bits(to_host(vd, dtype), vh)
        if not check_decode:
            return pairs
        bt, cl = bm.tables(seqs, MBS)
        q = W.randn(rng, (len(seqs), Hq, D), dtype)
        out = torch.empty((len(seqs), Hq, D), dtype=kd.dtype, device=kd.device)
        pa.pa_decode(to_dev(q, dtype), kd, vd, to_dev(bt), to_dev(cl), scale, out,
                     max_context_len=int(cl.max()), layout=layout)
        torch.cuda.synchronize()
        ref = oracle.decode(q, kh, vh, bt, cl, scale, dtype, layout=layout)
        assert_fp_close(f64(to_host(out, dtype), dtype), ref, dtype)
        return pairs

    root = bm.new_seq()
    step([root], [37], check_decode=True)            # prompt (prefill slots)
    beams = [root] + [bm.fork(root) for _ in range(4)]
    copies = 0
    for it in range(24):
        copies += len(step(beams, [1] * len(beams)))
        if it % 6 == 5:                              # prune two beams, fork two from the best
            bm.free(beams[-2:])
            beams = beams[:-2] + [bm.fork(beams[0]), bm.fork(beams[1])]
    assert copies > 0
    other = bm.new_seq()                             # a request with a multi-token chunk
    step(beams + [other], [2] * len(beams) + [3 * B + 1])
    g_free, _ = bm.num_free()
    assert g_free >= 0
