"""Parity behind the block-size sweep: the grouped-query batch of the
sweep (12 query / 2 kv heads, head dim 128, fp16, head-major pools) at a
reduced size, paged with blocks in order and scattered at every block size
from 1 to 256, against the contiguous twin and the fp64 oracle.  The three
layouts hold identical values, and the kernel visits tokens in the same
order whatever the block size, so the outputs must agree bit for bit."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import f64, to_dev, to_host
from helpers import assert_fp_close, same_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def batch():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rng = np.random.default_rng(61)
    S, ctx, Hq, Hkv, D = 4, 512, 12, 2, 128
    k = W.randn(rng, (S, Hkv, ctx, D), "f16")
    v = W.randn(rng, (S, Hkv, ctx, D), "f16")
    q = W.randn(rng, (S, Hq, D), "f16")
    lens = np.array([512, 497, 256, 1], np.int32)  # ragged, one single-token sequence
    return dict(S=S, ctx=ctx, Hq=Hq, Hkv=Hkv, D=D, k=k, v=v, q=q, lens=lens,
                scale=1 / np.sqrt(D))


def _decode_dense(b, partition):
    import torch

    import paged_kv_cache_pa_amd as pa

    out = torch.empty(b["q"].shape, dtype=torch.float16, device="cuda")
    pa.pa_decode_dense(to_dev(b["q"]), to_dev(b["k"]), to_dev(b["v"]), to_dev(b["lens"]),
                       b["scale"], out, max_context_len=b["ctx"], partition_size=partition,
                       layout="HND")
    torch.cuda.synchronize()
    return to_host(out, "f16")


def _paged(b, B, scattered):
    """Pools [NB, Hkv, B, D] holding the dense values, and the tables."""
    S, ctx, Hkv, D = b["S"], b["ctx"], b["Hkv"], b["D"]
    nbs = ctx // B
    nb = S * nbs
    ids = np.random.default_rng(B).permutation(nb) if scattered else np.arange(nb)
    table = ids.reshape(S, nbs).astype(np.int32)
    pools = []
    for x in (b["k"], b["v"]):
        logical = x.reshape(S, Hkv, nbs, B, D).transpose(0, 2, 1, 3, 4).reshape(nb, Hkv, B, D)
        pool = np.empty_like(logical)
        pool[ids] = logical
        pools.append(pool)
    return pools[0], pools[1], table


@pytest.mark.parametrize("partition", [0, 256])
@pytest.mark.parametrize("B", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_block_size_sweep_paged_equals_contiguous(batch, B, partition):
    import torch

    import paged_kv_cache_pa_amd as pa

    b = batch
    if partition and partition % B:
        pytest.skip("partition must be a multiple of the block size")
    dense = _decode_dense(b, partition)
    for scattered in (False, True):
        kp, vp, table = _paged(b, B, scattered)
        out = torch.empty(b["q"].shape, dtype=torch.float16, device="cuda")
        pa.pa_decode(to_dev(b["q"]), to_dev(kp), to_dev(vp), to_dev(table), to_dev(b["lens"]),
                     b["scale"], out, max_context_len=b["ctx"], partition_size=partition,
                     layout="HND")
        torch.cuda.synchronize()
        got = to_host(out, "f16")
        assert same_bits(got, dense), f"B={B} scattered={scattered}"
    if B in (1, 16, 256):
        ref = oracle.decode_dense(b["q"], b["k"], b["v"], b["lens"], b["scale"], "f16",
                                  layout="HND")
        assert_fp_close(f64(dense, "f16"), ref, "f16")
