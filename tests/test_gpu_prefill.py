"""Multi-token (prompt / chunked-prefill) attention over the paged cache:
the HIP kernel against the fp64 oracle, element by element, through the C
ABI.  Tolerance as decode (|err| <= 2e-3 + 1e-2 |ref| for fp16 / bf16).

Cases span several 64-row tiles with ragged tails, chunks that are whole
prompts, chunks at the end of a longer context, one-token chunks, empty
chunks, every pool layout, grouped-query heads, head dims 64 and 128, and
block sizes 1 .. 64; plus causality (tokens after a row's position cannot
change it) and the one-row chunk equal to decode within tolerance."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import f64, in_layout, to_dev, to_host
from helpers import assert_fp_close, same_bits

pytestmark = pytest.mark.gpu

MIX = ([100, 300, 17, 1, 64, 200, 80], [100, 37, 1, 1, 64, 130, 0])


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run(p, layout, k=None, v=None, max_query_len=None):
    import torch

    import paged_kv_cache_pa_amd as pa

    out = torch.full(p.q.shape, float("nan"), dtype=torch.float16 if p.dtype == "f16"
                     else torch.bfloat16, device="cuda")
    pa.pa_prefill(to_dev(p.q, p.dtype), to_dev(in_layout(p.k_cache if k is None else k, layout), p.dtype),
                  to_dev(in_layout(p.v_cache if v is None else v, layout), p.dtype),
                  to_dev(p.block_tables), to_dev(p.context_lens), to_dev(p.query_start), p.scale,
                  out, max_query_len=max_query_len or int(p.chunk_lens.max()),
                  max_context_len=int(p.context_lens.max()), layout=layout)
    torch.cuda.synchronize()
    return to_host(out, p.dtype)


def ref(p, k=None, v=None):
    return oracle.prefill(p.q, p.k_cache if k is None else k, p.v_cache if v is None else v,
                          p.block_tables, p.context_lens, p.query_start, p.scale, p.dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("hq,hkv,d", [(4, 4, 128), (12, 2, 128), (8, 2, 64)])
def test_prefill_matches_oracle(dtype, layout, hq, hkv, d):
    p = W.random_prefill(81, dtype, MIX[0], MIX[1], hq, hkv, d)
    got = run(p, layout)
    assert_fp_close(f64(got, dtype), ref(p), dtype)


@pytest.mark.parametrize("B", [1, 2, 8, 32, 64])
def test_prefill_block_sizes(B):
    p = W.random_prefill(82, "bf16", [150, 33, 70], [150, 20, 65], 4, 2, 128, block_size=B)
    assert_fp_close(f64(run(p, "HND"), "bf16"), ref(p), "bf16")


def test_prefill_long_context_chunk():
    """A 192-row chunk at the end of a 2000-token context (several table
    lookups per block and many key tiles per row)."""
    p = W.random_prefill(83, "f16", [2000, 513], [192, 513], 8, 8, 128)
    assert_fp_close(f64(run(p, "HND"), "f16"), ref(p), "f16")


def test_prefill_table_chunks():
    """Block sizes 1 and 2 with contexts past 1024 blocks: the key loop takes
    the block table 1024 entries at a time and restarts its pipeline at each
    such chunk (chunks of 1024 and 2048 keys; the last one ragged)."""
    print("case B=1", flush=True)
    p = W.random_prefill(88, "f16", [2500, 1030], [300, 1030], 4, 2, 128, block_size=1)
    assert_fp_close(f64(run(p, "HND"), "f16"), ref(p), "f16")
    print("case B=2", flush=True)
    p = W.random_prefill(89, "bf16", [2100], [129], 4, 4, 64, block_size=2)
    assert_fp_close(f64(run(p, "NHD"), "bf16"), ref(p), "bf16")


def test_prefill_is_causal():
    p = W.random_prefill(84, "bf16", [90], [40], 4, 4, 128, poison=False)
    before = run(p, "NHD")
    k2, v2 = p.k_cache.copy(), p.v_cache.copy()
    rng = np.random.default_rng(2)
    cut = 90 - 40 + 15                  # tokens after row 15's position change
    for t in range(cut + 1, 90):
        b, o = p.block_tables[0][t // 16], t % 16
        k2[b, o] = W.randn(rng, k2[b, o].shape, "bf16")
        v2[b, o] = W.randn(rng, v2[b, o].shape, "bf16")
    after = run(p, "NHD", k2, v2)
    assert same_bits(after[:16], before[:16])
    assert_fp_close(f64(after, "bf16"), ref(p, k2, v2), "bf16")


def test_prefill_one_row_chunks_match_decode_reference():
    import torch

    import paged_kv_cache_pa_amd as pa

    p = W.random_prefill(85, "f16", [33, 250, 1, 16], [1, 1, 1, 1], 6, 2, 128)
    got = run(p, "HND")
    dec = oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, "f16")
    assert_fp_close(f64(got, "f16"), dec, "f16")
    out = torch.empty(p.q.shape, dtype=torch.float16, device="cuda")
    pa.pa_decode(to_dev(p.q, "f16"), to_dev(in_layout(p.k_cache, "HND"), "f16"),
                 to_dev(in_layout(p.v_cache, "HND"), "f16"), to_dev(p.block_tables),
                 to_dev(p.context_lens), p.scale, out, max_context_len=250, layout="HND")
    torch.cuda.synchronize()
    assert_fp_close(f64(to_host(out, "f16"), "f16"), f64(got, "f16"), "f16")


def test_prefill_grid_bound_larger_than_chunks():
    """max_query_len above every chunk: the extra tiles find no rows."""
    p = W.random_prefill(86, "f16", [70, 10], [70, 3], 2, 2, 64)
    assert_fp_close(f64(run(p, "NHD", max_query_len=70), "f16"), ref(p), "f16")
    p2 = W.random_prefill(86, "f16", [70, 10], [5, 3], 2, 2, 64)
    assert_fp_close(f64(run(p2, "NHD", max_query_len=64), "f16"), ref(p2), "f16")


@pytest.mark.parametrize("label,dtype,S,ctx,chunk,hq,hkv", [
    ("OPT-13B prompt 8 x 1024", "f16", 8, 1024, 1024, 40, 40),
    ("GQA chunk 512 after 3584", "bf16", 4, 4096, 512, 32, 8),
])
def test_prefill_bench_points_sampled(label, dtype, S, ctx, chunk, hq, hkv):
    """The benchmark's two prefill launches at full size (head-major pool),
    checked on sampled rows: row r of a chunk attends to positions 0 ..
    ctx - chunk + r, so its exact value is the single-query result of that
    row over a context of that position + 1, which the oracle's decode
    gives.  Rows at tile edges and the ends of every sequence's chunk."""
    print("case", label, flush=True)
    p = W.random_prefill(84 + S, dtype, [ctx] * S, [chunk] * S, hq, hkv, 128)
    got = run(p, "HND")
    picks = sorted({0, 1, 31, 32, 63, 64, 127, 128, chunk // 2, chunk - 2, chunk - 1})
    rows, seqs, lens = [], [], []
    for s in range(S):
        for r in picks:
            rows.append(int(p.query_start[s]) + r)
            seqs.append(s)
            lens.append(ctx - chunk + r + 1)
    rows, seqs = np.array(rows), np.array(seqs)
    want = oracle.decode(p.q[rows], p.k_cache, p.v_cache, p.block_tables[seqs],
                         np.array(lens, np.int32), p.scale, dtype)
    assert_fp_close(f64(got[rows], dtype), want, dtype, label)
