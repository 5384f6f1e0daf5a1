"""Large pools and long contexts.

* A pool past 4 GiB per tensor, with the batch's blocks at the top of it:
  every byte offset into the pool needs 64 bits.  Decode, decode_append,
  cache_write, copy_blocks and prefill must give bit for bit what they give
  on a compact pool holding the same blocks (results do not depend on where
  blocks sit), and the compact results are checked against the fp64 oracle.
* Contexts of tens of thousands of tokens, with and without split-K (up to
  137 partitions), against the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import empty_out, f64, in_layout, to_dev, to_host, torch_dtype
from helpers import assert_fp_close, same_bits

pytestmark = pytest.mark.gpu

GIB = 1 << 30


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def big_pool(compact, nb_big, ids, dtype):
    """A NaN-filled device pool of nb_big blocks holding compact block c
    (device tensor, block index first) at block ids[c]."""
    import torch

    shape = (nb_big,) + tuple(compact.shape[1:])
    big = torch.full(shape, float("nan"), dtype=torch_dtype(dtype), device=compact.device)
    big[torch.from_numpy(ids).long().to(compact.device)] = compact
    return big


def remap(table, ids):
    return np.where(table >= 0, ids[np.maximum(table, 0)], -1).astype(np.int32)


def blocks_of(big, ids, dtype):
    import torch

    return to_host(big[torch.from_numpy(ids).long().to(big.device)], dtype)


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_pool_past_4gib(layout):
    import torch

    import paged_kv_cache_pa_amd as pa

    dt, Hq, Hkv, D, B = "f16", 8, 4, 128, 16
    p = W.random_paged(71, dt, [1, 37, 300, 1000, 0], Hq, Hkv, D, extra_blocks=8)
    NB = p.num_blocks
    blk_bytes = B * Hkv * D * 2
    nb_big = (5 * GIB) // blk_bytes + NB
    rng = np.random.default_rng(72)
    ids = (nb_big - 1 - rng.permutation(NB)).astype(np.int32)   # the top NB ids, shuffled
    assert int(ids.min()) * blk_bytes >= 4 * GIB
    tb_big = remap(p.block_tables, ids)

    kc, vc = to_dev(in_layout(p.k_cache, layout), dt), to_dev(in_layout(p.v_cache, layout), dt)
    kb, vb = big_pool(kc, nb_big, ids, dt), big_pool(vc, nb_big, ids, dt)
    q, cl = to_dev(p.q, dt), to_dev(p.context_lens)
    mcl = int(p.context_lens.max())

    def decode(k, v, table, ps):
        out = empty_out(p)
        pa.pa_decode(q, k, v, to_dev(table), cl, p.scale, out, max_context_len=mcl,
                     partition_size=ps, layout=layout)
        torch.cuda.synchronize()
        return to_host(out, dt)

    ref = oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, dt)
    for ps in (0, 256):
        small = decode(kc, vc, p.block_tables, ps)
        assert_fp_close(f64(small, dt), ref, dt)
        assert same_bits(decode(kb, vb, tb_big, ps), small)

    # copy-on-write pairs between used and spare blocks, then one new token per
    # non-empty sequence written at its next slot
    used = sorted(set(p.block_tables[p.block_tables >= 0].tolist()))
    spare = [b for b in range(NB) if b not in set(used)]
    pairs = np.array([[used[0], spare[0]], [used[-1], spare[1]], [used[2], spare[2]]], np.int32)
    pa.pa_copy_blocks(kc, vc, to_dev(pairs), layout=layout)
    pa.pa_copy_blocks(kb, vb, to_dev(np.ascontiguousarray(ids[pairs])), layout=layout)
    kh, vh = oracle.copy_blocks(p.k_cache, p.v_cache, pairs, dt)
    lens = p.context_lens.copy()
    slots = np.full(len(lens), -1, np.int32)
    table = p.block_tables.copy()
    for s, n in enumerate(lens):
        if n == 0 or n % B == 0:
            continue                                     # only slots inside a held block
        slots[s] = table[s, n // B] * B + n % B
        lens[s] = n + 1
    kn = W.randn(rng, (len(lens), Hkv, D), dt)
    vn = W.randn(rng, (len(lens), Hkv, D), dt)
    big_slots = np.where(slots >= 0, ids[np.maximum(slots, 0) // B] * B + slots % B, -1)
    big_slots = big_slots.astype(np.int32)
    assert int(big_slots.max()) < 2**31 - 1
    pa.pa_cache_write(to_dev(kn, dt), to_dev(vn, dt), kc, vc, to_dev(slots), layout=layout)
    pa.pa_cache_write(to_dev(kn, dt), to_dev(vn, dt), kb, vb, to_dev(big_slots), layout=layout)
    torch.cuda.synchronize()
    kh, vh = oracle.cache_write(kn, vn, kh, vh, slots, dt)
    assert same_bits(to_host(kc, dt), in_layout(kh, layout))
    assert same_bits(to_host(vc, dt), in_layout(vh, layout))
    assert same_bits(blocks_of(kb, ids, dt), in_layout(kh, layout))
    assert same_bits(blocks_of(vb, ids, dt), in_layout(vh, layout))

    # decode_append on both pools: one more token for the same sequences
    kn2 = W.randn(rng, (len(lens), Hkv, D), dt)
    vn2 = W.randn(rng, (len(lens), Hkv, D), dt)
    grow = (lens > 0) & (lens % B != 0)
    lens2 = np.where(grow, lens + 1, lens).astype(np.int32)
    outs = []
    for k, v, tab in ((kc, vc, table), (kb, vb, tb_big)):
        # the newest token of a sequence that does not grow is rewritten with
        # its own rows, so every non-empty sequence can take part
        kin = to_dev(np.where(grow[:, None, None], kn2, _newest(kh, table, lens2, B)), dt)
        vin = to_dev(np.where(grow[:, None, None], vn2, _newest(vh, table, lens2, B)), dt)
        out = empty_out(p)
        pa.pa_decode_append(q, kin, vin, k, v, to_dev(tab), to_dev(lens2), p.scale, out,
                            max_context_len=mcl + 2, layout=layout)
        torch.cuda.synchronize()
        outs.append(to_host(out, dt))
    assert same_bits(outs[1], outs[0])
    kh2, vh2 = to_host(kc, dt), to_host(vc, dt)      # in the requested layout
    assert same_bits(blocks_of(kb, ids, dt), kh2) and same_bits(blocks_of(vb, ids, dt), vh2)
    ref2 = oracle.decode(p.q, kh2, vh2, table, lens2, p.scale, dt, layout=layout)
    assert_fp_close(f64(outs[0], dt), ref2, dt)

    # prefill: the last rows of every sequence as a chunk
    chunks = np.minimum(lens2, 40).astype(np.int32)
    qs = np.zeros(len(chunks) + 1, np.int32)
    qs[1:] = np.cumsum(chunks)
    qp = W.randn(rng, (int(qs[-1]), Hq, D), dt)
    pres = []
    for k, v, tab in ((kc, vc, table), (kb, vb, tb_big)):
        out = torch.full(qp.shape, float("nan"), dtype=torch.float16, device=kc.device)
        pa.pa_prefill(to_dev(qp, dt), k, v, to_dev(tab), to_dev(lens2), to_dev(qs), p.scale, out,
                      layout=layout)
        torch.cuda.synchronize()
        pres.append(to_host(out, dt))
    assert same_bits(pres[1], pres[0])
    refp = oracle.prefill(qp, kh2, vh2, table, lens2, qs, p.scale, dt, layout=layout)
    assert_fp_close(f64(pres[0], dt), refp, dt)
    del kb, vb
    torch.cuda.empty_cache()


def _newest(pool, table, lens, B):
    """Rows of position n - 1 of each sequence from a token-major host pool
    (zeros for empty sequences)."""
    S = len(lens)
    out = np.zeros((S,) + pool.shape[2:], pool.dtype)
    for s in range(S):
        n = int(lens[s])
        if n:
            out[s] = pool[table[s, (n - 1) // B], (n - 1) % B]
    return out


@pytest.mark.parametrize("dtype,hq,hkv,d", [("f16", 4, 4, 128), ("bf16", 8, 2, 128),
                                            ("f32", 4, 2, 64)])
@pytest.mark.parametrize("ps", [0, 512])
def test_long_context(dtype, hq, hkv, d, ps):
    import torch

    import paged_kv_cache_pa_amd as pa

    p = W.random_paged(73, dtype, [70001, 3, 16384], hq, hkv, d)
    q, k, v = to_dev(p.q, dtype), to_dev(p.k_cache, dtype), to_dev(p.v_cache, dtype)
    bt, cl = to_dev(p.block_tables), to_dev(p.context_lens)
    out = empty_out(p)
    pa.pa_decode(q, k, v, bt, cl, p.scale, out, max_context_len=int(p.context_lens.max()),
                 partition_size=ps)
    torch.cuda.synchronize()
    got = to_host(out, dtype)
    ref = oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, dtype)
    if dtype == "f32":
        rel = np.abs(f64(got, dtype) - ref).max(axis=-1) / np.abs(ref).max(axis=-1)
        assert rel.max() <= 1e-5, rel.max()
    else:
        assert_fp_close(f64(got, dtype), ref, dtype)
