"""Config 3 at every point of the sweep: paged against dense, and both
against the fp64 oracle.

The sweep is 40/40 heads, head dim 128, fp16, batch {8, 32, 128} x context
{64, 256, 1024, 2048}: the paged-vs-contiguous comparison of [Kwon]
"Ablation Studies and Robustness Checks" (Figure 18a) and of [Res]
"Attention over scattered blocks" (the same kernel with and without the
table).  Each point is generated on the device (torch's seeded generator;
its largest dense tensor is 2.68 GB, so host generation would take minutes)
in the same structure as ``workloads.config3``: the dense [S, n, 40, 128]
buffers cut into 16-token blocks and scattered by a seeded permutation.

At every point and in both layouts:
* pa_decode and pa_decode_dense give the same bits on every row (compared
  on the device);
* sampled (sequence, head) units, two per sequence so that every sequence
  is covered, match the oracle's dense decode within the attention
  tolerance.  Only the sampled units' rows are copied to the host; each
  unit is an independent one-head problem for the oracle.
At 128 x 2048 the dense per-sequence offset passes 2^31 bytes.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from helpers import assert_fp_close

pytestmark = pytest.mark.gpu

H, D = 40, 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def sampled_units(batch):
    """Two heads per sequence (distinct), covering every sequence."""
    s = np.repeat(np.arange(batch), 2)
    h = np.empty_like(s)
    h[0::2] = (13 * np.arange(batch) + 5) % H
    h[1::2] = (29 * np.arange(batch) + 17) % H
    h[1::2] = np.where(h[1::2] == h[0::2], (h[1::2] + 1) % H, h[1::2])
    return s, h


def oracle_units(d, s_idx, h_idx, ctx):
    """fp64 oracle on the sampled units: unit u is sequence s_idx[u] with
    the single head h_idx[u] (its q row, its kv head's dense rows)."""
    import torch

    si = torch.from_numpy(s_idx).long().cuda()
    hi = torch.from_numpy(h_idx).long().cuda()
    # token-major dense [S, n, H, D]: unit rows [U, n, D] -> [U, n, 1, D]
    kd = d["k_dense"][si, :, hi, :].contiguous().cpu().numpy()[:, :, None, :]
    vd = d["v_dense"][si, :, hi, :].contiguous().cpu().numpy()[:, :, None, :]
    q = d["q"][si, hi, :].contiguous().cpu().numpy()[:, None, :]
    lens = np.full(len(s_idx), ctx, np.int32)
    return oracle.decode_dense(q, kd, vd, lens, d["scale"], "f16")[:, 0, :]


@pytest.mark.parametrize("batch,ctx", W.CONFIG3_POINTS)
def test_config3_point(batch, ctx):
    import torch

    import paged_kv_cache_pa_amd as pa

    print(f"config3 {batch}x{ctx}", flush=True)
    d = W.config3_device(batch, ctx)
    s_idx, h_idx = sampled_units(batch)
    assert set(s_idx.tolist()) == set(range(batch))
    ref = oracle_units(d, s_idx, h_idx, ctx)
    seq_bytes = ctx * H * D * 2
    if (batch, ctx) == (128, 2048):
        assert (batch - 1) * seq_bytes >= 2**31  # dense offsets need 64 bits
    for layout in ("NHD", "HND"):
        if layout == "HND":  # the same values, head-major
            for key in ("k_cache", "v_cache", "k_dense", "v_dense"):
                d[key] = d[key].transpose(1, 2).contiguous()
        paged = torch.full_like(d["q"], float("nan"))
        dense = torch.full_like(d["q"], float("nan"))
        pa.pa_decode(d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["context_lens"],
                     d["scale"], paged, max_context_len=ctx, layout=layout)
        pa.pa_decode_dense(d["q"], d["k_dense"], d["v_dense"], d["context_lens"], d["scale"],
                           dense, max_context_len=ctx, layout=layout)
        torch.cuda.synchronize()
        assert torch.equal(paged.view(torch.int16), dense.view(torch.int16)), \
            f"{layout} {batch}x{ctx}: paged and dense differ"
        assert bool(torch.isfinite(paged).all()), f"{layout} {batch}x{ctx}: non-finite output"
        got = paged[torch.from_numpy(s_idx).long().cuda(), torch.from_numpy(h_idx).long().cuda()]
        got = got.float().cpu().numpy().astype(np.float64)
        assert_fp_close(got, ref, "f16", f"config3 {layout} {batch}x{ctx} sampled units")
    del d
    torch.cuda.empty_cache()
