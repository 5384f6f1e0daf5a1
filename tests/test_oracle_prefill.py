"""Pins of the multi-token (prefill / chunked prefill) oracle.

Definition ([Kwon] §3.4: in the prompt phase every token attends to itself
and the tokens before it; the paged kernel reads them through the block
table): row r of sequence s's chunk of T rows sits at position n - T + r of
its n cached tokens and attends to positions 0 .. n - T + r.

Pins: a chunk's last row is the decode of the whole sequence (bit for bit,
the same routine); a one-row chunk at position p is the decode of the first
p + 1 tokens; a scalar route (brute.prefill) on tiny inputs; a numpy route
(gather + masked scipy softmax); causality (changing tokens after a row's
position leaves the row unchanged); equal keys give prefix means of V; and
splitting one chunk into two calls changes nothing."""
from __future__ import annotations

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import workloads as W
from helpers import same_bits
from oracle import brute


def gather(p, s, g):
    B = p.block_size
    n = int(p.context_lens[s])
    K = np.stack([W.to_f64(p.k_cache[p.block_tables[s][t // B], t % B, g], p.dtype)
                  for t in range(n)])
    V = np.stack([W.to_f64(p.v_cache[p.block_tables[s][t // B], t % B, g], p.dtype)
                  for t in range(n)])
    return K, V


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_last_row_is_decode(dtype):
    p = W.random_prefill(71, dtype, [40, 17, 5, 64], [9, 17, 1, 30], 4, 2, 32, block_size=4)
    out = oracle.prefill(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens,
                         p.query_start, p.scale, dtype)
    last = p.query_start[1:] - 1
    dec = oracle.decode(p.q[last], p.k_cache, p.v_cache, p.block_tables, p.context_lens,
                        p.scale, dtype)
    assert same_bits(out[last], dec)


def test_single_row_at_position_is_decode_of_prefix():
    p = W.random_prefill(72, "f16", [50], [12], 2, 1, 16, block_size=8)
    out = oracle.prefill(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens,
                         p.query_start, p.scale, "f16")
    for r in range(12):
        pos = 50 - 12 + r
        dec = oracle.decode(p.q[r:r + 1], p.k_cache, p.v_cache, p.block_tables,
                            np.array([pos + 1], np.int32), p.scale, "f16")
        assert same_bits(out[r:r + 1], dec)


def test_matches_scalar_route():
    p = W.random_prefill(73, "f32", [7, 5], [4, 5], 2, 1, 4, block_size=2, scale=0.3)
    out = oracle.prefill(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens,
                         p.query_start, p.scale, "f32")
    ref = np.array(brute.prefill(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens,
                                 p.query_start, p.scale))
    assert np.allclose(out, ref, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_matches_numpy_masked_softmax(dtype):
    p = W.random_prefill(74, dtype, [33, 70, 16], [33, 20, 3], 6, 2, 16)
    out = oracle.prefill(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens,
                         p.query_start, p.scale, dtype)
    G = 3
    for s in range(3):
        n, lo, hi = int(p.context_lens[s]), int(p.query_start[s]), int(p.query_start[s + 1])
        T = hi - lo
        for g in range(2):
            K, V = gather(p, s, g)
            for h in range(g * G, (g + 1) * G):
                qh = W.to_f64(p.q[lo:hi, h], dtype)          # [T, D]
                sc = p.scale * qh @ K.T                        # [T, n]
                pos = n - T + np.arange(T)
                sc[np.arange(n)[None, :] > pos[:, None]] = -np.inf
                ref = softmax(sc, axis=1) @ V
                np.testing.assert_allclose(out[lo:hi, h], ref, rtol=1e-12, atol=1e-13)


def test_causal_future_tokens_do_not_matter():
    p = W.random_prefill(75, "bf16", [48], [20], 4, 4, 16, block_size=16, poison=False)
    out = oracle.prefill(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens,
                         p.query_start, p.scale, "bf16")
    k2, v2 = p.k_cache.copy(), p.v_cache.copy()
    rng = np.random.default_rng(1)
    cut = 48 - 20 + 7                    # row 7's position: tokens after it change
    for t in range(cut + 1, 48):
        b, o = p.block_tables[0][t // 16], t % 16
        k2[b, o] = W.randn(rng, k2[b, o].shape, "bf16")
        v2[b, o] = W.randn(rng, v2[b, o].shape, "bf16")
    out2 = oracle.prefill(p.q, k2, v2, p.block_tables, p.context_lens, p.query_start, p.scale,
                          "bf16")
    assert same_bits(out2[:8], out[:8])
    assert not np.array_equal(out2[8:], out[8:])


def test_equal_keys_give_prefix_means():
    p = W.random_prefill(76, "f32", [24], [10], 1, 1, 8, block_size=4, poison=False)
    k = p.k_cache.copy()
    k[:] = k[p.block_tables[0][0], 0]     # every key equal
    out = oracle.prefill(p.q, k, p.v_cache, p.block_tables, p.context_lens, p.query_start,
                         p.scale, "f32")
    _, V = gather(p, 0, 0)
    for r in range(10):
        pos = 24 - 10 + r
        np.testing.assert_allclose(out[r, 0], V[:pos + 1].mean(axis=0), rtol=1e-13, atol=1e-14)


def test_split_chunk_equals_whole_chunk():
    p = W.random_prefill(77, "f16", [60], [25], 2, 2, 16, block_size=8)
    whole = oracle.prefill(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens,
                           p.query_start, p.scale, "f16")
    first = oracle.prefill(p.q[:10], p.k_cache, p.v_cache, p.block_tables,
                           np.array([60 - 15], np.int32), np.array([0, 10], np.int32), p.scale,
                           "f16")
    second = oracle.prefill(p.q[10:], p.k_cache, p.v_cache, p.block_tables, p.context_lens,
                            np.array([0, 15], np.int32), p.scale, "f16")
    assert same_bits(np.concatenate([first, second]), whole)


def test_refuses_chunk_longer_than_context():
    p = W.random_prefill(78, "f32", [10], [4], 1, 1, 8)
    with pytest.raises(oracle.OracleError):
        oracle.prefill(p.q, p.k_cache, p.v_cache, p.block_tables, np.array([3], np.int32),
                       p.query_start, p.scale, "f32")
