"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test names what a plausible mistake in the oracle would break:
dropped normalisation, a wrong sign, the exp-of-a-sum misreading of the
block-wise denominator, a transposed index (t % B vs t / B), the wrong
query-head -> kv-head map, a bad fp16/bf16 widening, a broken merge.
CPU only."""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W
from oracle import brute
from helpers import assert_fp_close, bits, empty_pool, np_reference, same_bits


# ---------------------------------------------------------------- widening


def test_half_widening_exhaustive():
    """All 65536 binary16 patterns against numpy's float16 -> float64."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = pats.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(p)) for p in pats])
    nan = np.isnan(want)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == want[~nan]).all()
    assert same_bits(got[~nan], want[~nan])  # signed zeros too


def test_bf16_widening_exhaustive():
    """bf16 is the top half of a binary32: all 65536 patterns."""
    pats = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        want = (pats << 16).view(np.float32).astype(np.float64)
    got = np.array([oracle.bf16_to_double(int(p)) for p in pats])
    nan = np.isnan(want)
    assert (np.isnan(got) == nan).all()
    assert same_bits(got[~nan], want[~nan])


# ---------------------------------------------------------------- pages' fixtures


def _hand_case(g):
    nb, b, d = g["num_blocks"], g["block_size"], g["head_dim"]
    k, v = empty_pool(nb, b, 1, d, "f32")
    for t in range(g["context_len"]):
        blk = g["block_table"][t // b]
        k[blk, t % b, 0] = g["k"][t]
        v[blk, t % b, 0] = g["v"][t]
    q = np.array(g["q"], dtype=np.float32).reshape(1, 1, d)
    table = np.array([g["block_table"]], dtype=np.int32)
    lens = np.array([g["context_len"]], dtype=np.int32)
    return q, k, v, table, lens


def test_hand_weights(golden):
    """Weights 1/7, 2/7, 4/7 and out = [5, 10, 0, 1], derived by hand."""
    g = golden("hand_weights.json")
    q, k, v, table, lens = _hand_case(g)
    out, w = oracle.decode(q, k, v, table, lens, g["scale"], "f32", want_weights=True)
    want_w = [float(Fraction(x)) for x in g["weights"]]
    assert np.allclose(w[0, 0, :3], want_w, rtol=0, atol=1e-15)
    assert (w[0, 0, 3:] == 0).all()
    assert np.allclose(out[0, 0], g["out"], rtol=0, atol=1e-14)
    bo, bw = brute.decode(q, k, v, table, lens, g["scale"])
    assert np.allclose(bo[0][0], g["out"], rtol=0, atol=1e-14)
    assert np.allclose(bw[0][0], want_w, rtol=0, atol=1e-15)


def test_fig6_slots_and_gather(golden):
    """Fig. 6 at block size 4: cache_write places token i at the printed
    slot, and decode reads token j from exactly that slot."""
    g = golden("fig6_block_table.json")
    B, NB, n = g["block_size"], g["num_blocks"], g["context_len"]
    table = np.array(g["block_table"], dtype=np.int32)
    slots = W.slots_of(table, np.arange(n), B)
    assert slots.tolist() == g["slots"]
    D = 8
    k, v = empty_pool(NB, B, 1, D, "f32")
    rng = np.random.default_rng(6)
    k_new = rng.standard_normal((n, 1, D)).astype(np.float32)
    v_new = np.repeat(np.arange(n, dtype=np.float32)[:, None, None], D, axis=2)
    kc, vc = oracle.cache_write(k_new, v_new, k, v, np.array(g["slots"], np.int32), "f32")
    for i, s in enumerate(g["slots"]):
        assert same_bits(kc[s // B, s % B], k_new[i])
        assert (vc[s // B, s % B] == i).all()
    # filled counts: 4, 4, 1 -> the slots not listed stay NaN
    filled = {b: c for b, c in zip(g["block_table"], g["filled"])}
    for b in range(NB):
        assert np.isnan(kc[b, filled.get(b, 0):]).all()
    # one-hot attention on token j must return v_j = j
    for j in range(n):
        kk = np.zeros((n, 1, D), dtype=np.float32)
        kk[j, 0, 0] = 60.0
        kc2, _ = oracle.cache_write(kk, v_new, k, v, np.array(g["slots"], np.int32), "f32")
        q = np.zeros((1, 1, D), np.float32)
        q[0, 0, 0] = 1.0
        out = oracle.decode(q, kc2, vc, table[None], np.array([n], np.int32), 1.0, "f32")
        assert np.allclose(out[0, 0], j, rtol=0, atol=1e-20), (j, out[0, 0])


def test_internals_flowchart(golden):
    """Two sequences sharing blocks 7 and 1: each reads its own third block."""
    g = golden("internals_flowchart.json")
    B, NB = g["block_size"], g["num_blocks"]
    lens = np.array(g["context_lens"], np.int32)
    assert lens.tolist() == [sum(f) for f in g["filled"]]
    table = np.array(g["tables"], np.int32)
    used = set(table.ravel().tolist())
    assert sorted(set(range(NB)) - used) == g["free"]
    rng = np.random.default_rng(7)
    D, H = 16, 2
    k = W.randn(rng, (NB, B, H, D), "f16")
    v = W.randn(rng, (NB, B, H, D), "f16")
    q = W.randn(rng, (1, H, D), "f16").repeat(2, axis=0)
    p = W.Paged("f16", q, k, v, table, lens, 0.25, B)
    out = oracle.decode(q, k, v, table, lens, 0.25, "f16")
    assert np.allclose(out, np_reference(p), rtol=1e-12, atol=1e-13)
    # the shared 32-token prefix is the same data for both sequences
    short = oracle.decode(q, k, v, table, np.array([32, 32], np.int32), 0.25, "f16")
    assert same_bits(short[0], short[1])
    assert not np.allclose(out[0], out[1])


def test_internals_cow_trace(golden):
    """copy 1 -> 3, then A1 writes into the copy and A2 into block 1 in place."""
    g = golden("internals_cow_trace.json")
    B, NB = g["block_size"], g["num_blocks"]
    rng = np.random.default_rng(8)
    H, D = 2, 8
    k, v = empty_pool(NB, B, H, D, "f16")
    n0 = g["context_len_before"]
    for t in range(n0):
        b = g["shared_table"][t // B]
        k[b, t % B] = W.randn(rng, (H, D), "f16")
        v[b, t % B] = W.randn(rng, (H, D), "f16")
    kc, vc = oracle.copy_blocks(k, v, np.array(g["copy_pairs"], np.int32), "f16")
    assert same_bits(kc[3], k[1])
    assert same_bits(kc[1], k[1])
    new_k = W.randn(rng, (2, H, D), "f16")
    new_v = W.randn(rng, (2, H, D), "f16")
    slots = np.array([g["write_slots"]["A1"], g["write_slots"]["A2"]], np.int32)
    kc, vc = oracle.cache_write(new_k, new_v, kc, vc, slots, "f16")
    tables = np.array([g["tables_after"]["A1"], g["tables_after"]["A2"]], np.int32)
    lens = np.array([n0 + 1, n0 + 1], np.int32)
    q = W.randn(rng, (1, H, D), "f16").repeat(2, axis=0)
    p = W.Paged("f16", q, kc, vc, tables, lens, 0.5, B)
    out = oracle.decode(q, kc, vc, tables, lens, 0.5, "f16")
    assert np.isfinite(out).all()
    assert np.allclose(out, np_reference(p), rtol=1e-12, atol=1e-13)
    # before the divergent token both samples see identical history
    pre = oracle.decode(q, kc, vc, tables, np.array([n0, n0], np.int32), 0.5, "f16")
    assert same_bits(pre[0], pre[1])


def _replay_share(prompt_len, samples, steps, B):
    """The sampling run of the fixture, replayed with an ascending allocator:
    fork shares every block; a sample about to write into a shared, partly
    filled last block copies it first; blocks are added on demand."""
    nxt = [0]
    refs = {}

    def alloc():
        b = nxt[0]
        nxt[0] += 1
        refs[b] = 1
        return b

    first = [alloc() for _ in range(-(-prompt_len // B))]
    tables = [list(first)] + [list(first) for _ in range(samples - 1)]
    for b in first:
        refs[b] += samples - 1
    n = [prompt_len] * samples
    pairs = []
    for _ in range(steps):
        for i in range(samples):
            t = tables[i]
            if n[i] % B and refs[t[-1]] > 1:
                old, new = t[-1], alloc()
                pairs.append((old, new))
                refs[old] -= 1
                t[-1] = new
            while len(t) * B < n[i] + 1:
                t.append(alloc())
            n[i] += 1
    return tables, pairs, nxt[0], n


def test_share_py_tables(golden):
    g = golden("share_py_tables.json")
    B = g["block_size"]
    steps = g["final_context_len"] - g["prompt_len"]
    tables, pairs, used, n = _replay_share(g["prompt_len"], g["samples"], steps, B)
    assert tables == g["tables"]
    assert [list(p) for p in pairs] == g["copy_pairs"]
    assert used == g["blocks_in_use"] and len(pairs) == g["copies"]
    assert g["samples"] * len(g["tables"][0]) == g["blocks_without_sharing"]
    # 108 cached tokens give the same tables (the reading's alternative)
    assert _replay_share(g["prompt_len"], g["samples"], steps + 1, B)[0] == g["tables"]

    # copy + write + decode on random data through the fixture's tables
    rng = np.random.default_rng(44)
    H, D, NB = 2, 16, used
    k, v = empty_pool(NB, B, H, D, "bf16")
    P = g["prompt_len"]
    for t in range(P):
        b = g["prompt_blocks"][t // B]
        k[b, t % B] = W.randn(rng, (H, D), "bf16")
        v[b, t % B] = W.randn(rng, (H, D), "bf16")
    kc, vc = oracle.copy_blocks(k, v, np.array(g["copy_pairs"], np.int32), "bf16")
    tab = np.array(g["tables"], np.int32)
    N = g["final_context_len"]
    slots = np.concatenate([W.slots_of(tab[i], np.arange(P, N), B) for i in range(g["samples"])])
    k_new = W.randn(rng, (len(slots), H, D), "bf16")
    v_new = W.randn(rng, (len(slots), H, D), "bf16")
    kc, vc = oracle.cache_write(k_new, v_new, kc, vc, slots, "bf16")
    assert same_bits(kc[:2], k[:2])       # full prompt blocks untouched
    for dst in (3, 4, 5):                                      # copies keep the 12 prompt slots
        assert same_bits(kc[dst, :12], k[2, :12])
    assert same_bits(kc[2, :12], k[2, :12])
    lens = np.full(g["samples"], N, np.int32)
    valid = W.valid_slots(tab, lens, NB, B)                    # every valid slot now written
    assert not np.isnan(W.to_f64(kc[valid], "bf16")).any()
    assert np.isnan(W.to_f64(kc[~valid], "bf16")).all()
    q = W.randn(rng, (g["samples"], H, D), "bf16")
    p = W.Paged("bf16", q, kc, vc, tab, lens, 0.25, B)
    out = oracle.decode(q, kc, vc, tab, lens, 0.25, "bf16")
    assert np.allclose(out, np_reference(p), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- closed forms


def _single(n, D=8, seed=0, dtype="f32", hkv=1, hq=1, B=4):
    return W.random_paged(seed, dtype, [n], hq, hkv, D, block_size=B)


def test_one_token_returns_its_value_exactly():
    for dt in W.DTYPES:
        p = _single(1, dtype=dt, seed=3)
        out = oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, dt)
        b = p.block_tables[0, 0]
        assert same_bits(out[0, 0], W.to_f64(p.v_cache[b, 0, 0], dt))


def test_equal_keys_and_zero_query_give_the_mean():
    p = _single(37, D=16, seed=4)
    k = p.k_cache.copy()
    k[:] = np.float32(0.75)
    out = oracle.decode(p.q, k, p.v_cache, p.block_tables, p.context_lens, 1.0, "f32")
    V = np.stack([W.to_f64(p.v_cache[p.block_tables[0, t // 4], t % 4, 0], "f32") for t in range(37)])
    assert np.allclose(out[0, 0], V.mean(axis=0), rtol=0, atol=1e-14)
    out0 = oracle.decode(np.zeros_like(p.q), p.k_cache, p.v_cache, p.block_tables,
                         p.context_lens, 1.0, "f32")
    assert np.allclose(out0[0, 0], V.mean(axis=0), rtol=0, atol=1e-14)


def test_two_tokens_logistic():
    """n = 2: out = sigma(x0 - x1) v0 + sigma(x1 - x0) v1."""
    p = _single(2, D=8, seed=5, B=1)
    out = oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, "f32")
    b0, b1 = p.block_tables[0, :2]
    q = p.q[0, 0].astype(np.float64)
    k0, k1 = p.k_cache[b0, 0, 0].astype(np.float64), p.k_cache[b1, 0, 0].astype(np.float64)
    v0, v1 = p.v_cache[b0, 0, 0].astype(np.float64), p.v_cache[b1, 0, 0].astype(np.float64)
    dx = p.scale * (q @ k0 - q @ k1)
    s0 = 1.0 / (1.0 + math.exp(-dx))
    assert np.allclose(out[0, 0], s0 * v0 + (1 - s0) * v1, rtol=1e-14, atol=1e-15)


def test_large_gap_is_one_hot():
    p = _single(50, D=8, seed=6)
    k = np.zeros_like(p.k_cache)
    j = 33
    k[p.block_tables[0, j // 4], j % 4, 0, 0] = 1000.0
    q = np.zeros_like(p.q)
    q[0, 0, 0] = 1.0
    out = oracle.decode(q, k, p.v_cache, p.block_tables, p.context_lens, 1.0, "f32")
    assert same_bits(out[0, 0], p.v_cache[p.block_tables[0, j // 4], j % 4, 0].astype(np.float64))


def test_empty_sequence_gives_zeros():
    p = W.random_paged(9, "f16", [0, 5, 0], 4, 2, 16)
    out = oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, "f16")
    assert (out[0] == 0).all() and (out[2] == 0).all() and np.isfinite(out[1]).all()


def test_gqa_head_map_contiguous_groups():
    """Constant V per kv head: query head h must return kv head h // G's value."""
    Hq, Hkv = 12, 2
    p = W.random_paged(10, "bf16", [40, 17], Hq, Hkv, 16)
    v = p.v_cache.copy()
    for g in range(Hkv):
        v[:, :, g, :] = W.to_storage(np.full((1,), g + 1.0, np.float32), "bf16")[0]
    out = oracle.decode(p.q, p.k_cache, v, p.block_tables, p.context_lens, p.scale, "bf16")
    for h in range(Hq):
        assert np.allclose(out[:, h], h // (Hq // Hkv) + 1, rtol=0, atol=1e-14), h


def test_exact_result_mpmath():
    """Within 1e-14 of a 50-digit evaluation of the defining equation."""
    import mpmath

    mpmath.mp.dps = 50
    p = W.random_paged(11, "f16", [23], 2, 1, 8, block_size=4)
    out = oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, "f16")
    for h in range(2):
        qv = [mpmath.mpf(float(x)) for x in p.q[0, h]]
        rows = [(p.block_tables[0, t // 4], t % 4) for t in range(23)]
        xs = [mpmath.mpf(p.scale) * mpmath.fsum(qv[d] * mpmath.mpf(float(p.k_cache[b, o, 0, d]))
                                               for d in range(8)) for b, o in rows]
        es = [mpmath.exp(x) for x in xs]
        Z = mpmath.fsum(es)
        for d in range(8):
            ref = mpmath.fsum(e * mpmath.mpf(float(p.v_cache[b, o, 0, d])) for e, (b, o) in zip(es, rows)) / Z
            assert abs(out[0, h, d] - float(ref)) <= 1e-14 * max(1.0, abs(float(ref)))


# ---------------------------------------------------------------- invariants


def test_weights_convex():
    p = W.config1()
    kc, vc = oracle.cache_write(p.k_new, p.v_new, p.k_cache, p.v_cache, p.slot_mapping, "f32")
    out, w = oracle.decode(p.q, kc, vc, p.block_tables, p.context_lens, p.scale, "f32",
                           want_weights=True)
    for s, n in enumerate(p.context_lens):
        assert np.allclose(w[s, :, :n].sum(axis=-1), 1.0, rtol=0, atol=1e-14)
        assert (w[s, :, :n] >= 0).all() and (w[s, :, n:] == 0).all()
    assert np.isfinite(out).all()


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_block_permutation_invariance(dtype):
    """Relabelling physical blocks leaves the result bitwise unchanged."""
    p = W.random_paged(12, dtype, [1, 16, 17, 63, 100], 6, 3, 32, extra_blocks=11)
    out = oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, dtype)
    rng = np.random.default_rng(99)
    pi = rng.permutation(p.num_blocks).astype(np.int32)
    k2 = np.empty_like(p.k_cache)
    v2 = np.empty_like(p.v_cache)
    k2[pi] = p.k_cache
    v2[pi] = p.v_cache
    t2 = np.where(p.block_tables >= 0, pi[np.maximum(p.block_tables, 0)], -1).astype(np.int32)
    out2 = oracle.decode(p.q, k2, v2, t2, p.context_lens, p.scale, dtype)
    assert same_bits(out, out2)


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_paged_equals_dense(dtype):
    p = W.random_with_dense(13, dtype, [5, 0, 33, 80, 16], 8, 2, 64)
    out = oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, dtype)
    outd = oracle.decode_dense(p.q, p.k_dense, p.v_dense, p.context_lens, p.scale, dtype)
    assert same_bits(out, outd)


def to_head_major(a):
    """[X, tokens, Hkv, D] -> [X, Hkv, tokens, D] (numpy transpose)."""
    return np.ascontiguousarray(np.swapaxes(a, 1, 2))


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_head_major_layout_matches_transpose(dtype):
    """The head-major pool holds the same values, transposed inside each
    block: decode, dense decode and cache_write must agree bitwise."""
    p = W.random_with_dense(33, dtype, [7, 0, 40, 95], 6, 3, 32, block_size=8)
    ref = oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, dtype)
    hm = oracle.decode(p.q, to_head_major(p.k_cache), to_head_major(p.v_cache), p.block_tables,
                       p.context_lens, p.scale, dtype, layout="HND")
    assert same_bits(ref, hm)
    dh = oracle.decode_dense(p.q, to_head_major(p.k_dense), to_head_major(p.v_dense),
                             p.context_lens, p.scale, dtype, layout="HND")
    assert same_bits(ref, dh)
    sp = oracle.decode_split(p.q, to_head_major(p.k_cache), to_head_major(p.v_cache),
                             p.block_tables, p.context_lens, p.scale, dtype, 16, layout="HND")
    assert np.allclose(sp, ref, rtol=1e-13, atol=1e-14)
    rng = np.random.default_rng(34)
    slots = rng.permutation(p.num_blocks * 8)[:20].astype(np.int32)
    kn, vn = W.randn(rng, (20, 3, 32), dtype), W.randn(rng, (20, 3, 32), dtype)
    kc, vc = oracle.cache_write(kn, vn, p.k_cache, p.v_cache, slots, dtype)
    kh, vh = oracle.cache_write(kn, vn, to_head_major(p.k_cache), to_head_major(p.v_cache), slots,
                                dtype, layout="HND")
    assert same_bits(to_head_major(kc), kh) and same_bits(to_head_major(vc), vh)


@pytest.mark.parametrize("P", [16, 32, 48, 512])
def test_split_merge_identity(P):
    p = W.random_paged(14, "bf16", [0, 1, 15, 16, 17, 47, 48, 49, 300, 700], 6, 2, 32)
    out = oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, "bf16")
    outs = oracle.decode_split(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens,
                               p.scale, "bf16", P)
    den = np.maximum(np.abs(out).max(axis=-1, keepdims=True), 1e-300)
    assert (np.abs(outs - out) / den <= 1e-14).all()


@pytest.mark.parametrize("dtype,hq,hkv,d", [("f32", 4, 4, 8), ("f16", 6, 2, 8), ("bf16", 4, 1, 16)])
def test_brute_force_tiny(dtype, hq, hkv, d):
    p = W.random_paged(15, dtype, [1, 6, 9, 0, 13], hq, hkv, d, block_size=4)
    out = oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, dtype)
    widen = (lambda x: float(W.to_f64(np.array([x], np.uint16), "bf16")[0])) if dtype == "bf16" else float
    bo, _ = brute.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, widen)
    assert np.allclose(out, np.array(bo), rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_numpy_scipy_route(dtype):
    p = W.random_paged(16, dtype, [3, 77, 128, 129, 250], 8, 4, 64)
    out = oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, dtype)
    assert np.allclose(out, np_reference(p), rtol=1e-12, atol=1e-13)


def test_units_subset_matches_full():
    p = W.random_paged(17, "f16", [30, 90, 7], 8, 8, 32)
    full = oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, "f16")
    units = np.array([[1, 3], [2, 7], [0, 0]], np.int32)
    part = oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale,
                         "f16", units=units)
    for s, h in units:
        assert same_bits(part[s, h], full[s, h])


# ---------------------------------------------------------------- cache_write / copy_blocks


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_cache_write_matches_numpy_scatter(dtype):
    rng = np.random.default_rng(18)
    NB, B, H, D = 12, 16, 3, 32
    k, v = empty_pool(NB, B, H, D, dtype)
    N = 70
    slots = rng.permutation(NB * B)[:N].astype(np.int32)
    slots[::9] = -1
    k_new = W.randn(rng, (N, H, D), dtype)
    v_new = W.randn(rng, (N, H, D), dtype)
    kc, vc = oracle.cache_write(k_new, v_new, k, v, slots, dtype)
    ke, ve = k.copy().reshape(NB * B, H, D), v.copy().reshape(NB * B, H, D)
    ok = slots >= 0
    ke[slots[ok]] = k_new[ok]
    ve[slots[ok]] = v_new[ok]
    assert same_bits(kc, ke.reshape(kc.shape))
    assert same_bits(vc, ve.reshape(vc.shape))


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_copy_blocks_matches_numpy(dtype):
    rng = np.random.default_rng(19)
    NB, B, H, D = 20, 16, 2, 64
    k = W.randn(rng, (NB, B, H, D), dtype)
    v = W.randn(rng, (NB, B, H, D), dtype)
    perm = rng.permutation(NB)
    src, dst = perm[:6], perm[6:12]
    pairs = np.stack([src, dst], axis=1).astype(np.int32)
    kc, vc = oracle.copy_blocks(k, v, pairs, dtype)
    ke, ve = k.copy(), v.copy()
    ke[dst] = k[src]
    ve[dst] = v[src]
    assert same_bits(kc, ke) and same_bits(vc, ve)


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_swap_blocks_matches_byte_gather(dtype):
    """Host <-> GPU pool moves: each destination block holds the source
    block's bytes; ids outside either pool are skipped; a swap-out followed
    by the reverse swap-in brings every moved block back unchanged."""
    rng = np.random.default_rng(23)
    L, B, H, D = 3, 8, 2, 32
    gk = [W.randn(rng, (20, B, H, D), dtype) for _ in range(L)]
    gv = [W.randn(rng, (20, B, H, D), dtype) for _ in range(L)]
    hk = [W.randn(rng, (9, B, H, D), dtype) for _ in range(L)]
    hv = [W.randn(rng, (9, B, H, D), dtype) for _ in range(L)]
    pairs = np.array([[4, 0], [17, 8], [2, 3], [25, 1], [5, 9], [11, 5]], np.int32)
    ok_, ov_ = oracle.swap_blocks(hk, hv, gk, gv, pairs)
    valid = pairs[(pairs[:, 0] < 20) & (pairs[:, 1] < 9)]
    for layer in range(L):
        nbytes = gk[layer][0].nbytes
        src = gk[layer].view(np.uint8).reshape(20, nbytes)
        want = hk[layer].view(np.uint8).reshape(9, nbytes).copy()
        want[valid[:, 1]] = src[valid[:, 0]]
        assert np.array_equal(ok_[layer].view(np.uint8).reshape(9, nbytes), want)
        untouched = np.setdiff1d(np.arange(9), valid[:, 1])
        assert same_bits(ov_[layer][untouched], hv[layer][untouched])
    # round trip: wipe the GPU blocks, then swap back in
    wiped = [x.copy() for x in gk]
    for layer in range(L):
        wiped[layer][valid[:, 0]] = W.nan_fill(wiped[layer][valid[:, 0]].shape, dtype)
    back_k, _ = oracle.swap_blocks(wiped, [x.copy() for x in gv], ok_, ov_, valid[:, ::-1])
    for layer in range(L):
        assert same_bits(back_k[layer], gk[layer])


def test_copy_blocks_layers_is_per_layer_copy():
    rng = np.random.default_rng(24)
    ks = [W.randn(rng, (10, 4, 2, 16), "f16") for _ in range(4)]
    vs = [W.randn(rng, (10, 4, 2, 16), "f16") for _ in range(4)]
    pairs = np.array([[1, 7], [3, 2]], np.int32)
    kc, vc = oracle.copy_blocks_layers(ks, vs, pairs, "f16")
    for layer in range(4):
        ke, ve = ks[layer].copy(), vs[layer].copy()
        ke[[7, 2]] = ks[layer][[1, 3]]
        ve[[7, 2]] = vs[layer][[1, 3]]
        assert same_bits(kc[layer], ke) and same_bits(vc[layer], ve)


def test_cache_write_layers_fig6(golden):
    """Fig. 6's slots in three layers at once: layer l's token i lands at the
    printed slot of layer l's pools only (values 100 l + i), every other
    slot of every layer stays NaN."""
    g = golden("fig6_block_table.json")
    B, NB, n = g["block_size"], g["num_blocks"], g["context_len"]
    slots = np.array(g["slots"], np.int32)
    D, L = 8, 3
    pools = [empty_pool(NB, B, 1, D, "f32") for _ in range(L)]
    news = [np.full((n, 1, D), 100.0 * layer, np.float32) + np.arange(n, dtype=np.float32)[:, None, None]
            for layer in range(L)]
    kc, vc = oracle.cache_write_layers(news, [-x for x in news], [k for k, _ in pools],
                                       [v for _, v in pools], slots, "f32")
    for layer in range(L):
        written = np.zeros((NB, B), bool)
        for i, sl in enumerate(g["slots"]):
            assert (kc[layer][sl // B, sl % B] == 100.0 * layer + i).all()
            assert (vc[layer][sl // B, sl % B] == -(100.0 * layer + i)).all()
            written[sl // B, sl % B] = True
        assert np.isnan(kc[layer][~written]).all() and np.isnan(vc[layer][~written]).all()


def test_index_errors_write_nothing():
    k, v = empty_pool(4, 4, 1, 8, "f32")
    new = np.ones((2, 1, 8), np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.cache_write(new, new, k, v, np.array([3, 16], np.int32), "f32")
    with pytest.raises(oracle.OracleError):
        oracle.copy_blocks(k, v, np.array([[0, 4]], np.int32), "f32")
    with pytest.raises(oracle.OracleError):
        oracle.decode(np.ones((1, 1, 8), np.float32), k, v, np.array([[0, -1]], np.int32),
                      np.array([5], np.int32), 1.0, "f32")


# ---------------------------------------------------------------- the configurations


def test_config1_write_then_decode():
    p = W.config1()
    assert np.isnan(p.k_cache).any()
    kc, vc = oracle.cache_write(p.k_new, p.v_new, p.k_cache, p.v_cache, p.slot_mapping, "f32")
    for s in range(p.num_seqs):
        n = p.context_lens[s]
        b, o = divmod(int(p.slot_mapping[s]), 16)
        assert b == p.block_tables[s, (n - 1) // 16] and o == (n - 1) % 16
        assert same_bits(kc[b, o], p.k_new[s])
    out = oracle.decode(p.q, kc, vc, p.block_tables, p.context_lens, p.scale, "f32")
    q = W.Paged("f32", p.q, kc, vc, p.block_tables, p.context_lens, p.scale, 16)
    assert np.isfinite(out).all()
    assert np.allclose(out, np_reference(q), rtol=1e-12, atol=1e-13)


def test_config4_scenario_invariants():
    sc = W.config4()
    p = sc.paged
    B, P = 16, sc.prompt_len // 16
    # block count: 16*32 shared prompt blocks + per beam its stem block and suffix blocks
    want = sc.groups * P + sum(
        1 + -(-max(0, int(sb) - (B - int(sc.stem[i // sc.beams]))) // B)
        for i, sb in enumerate(sc.suffix))
    assert sc.blocks_in_use == want
    assert len(p.block_pairs) == sc.groups * (sc.beams - 1)
    dst = p.block_pairs[:, 1]
    assert len(set(dst.tolist())) == len(dst) and not set(dst.tolist()) & set(p.block_pairs[:, 0].tolist())
    sm = p.slot_mapping
    assert len(set(sm.tolist())) == len(sm)
    kc, vc = oracle.copy_blocks(p.k_cache, p.v_cache, p.block_pairs, "f16")
    kc, vc = oracle.cache_write(p.k_new, p.v_new, kc, vc, sm, "f16")
    assert same_bits(kc[sc.prompt_blocks.ravel()], p.k_cache[sc.prompt_blocks.ravel()])
    for gi in range(sc.groups):
        t0 = int(sc.stem[gi])
        for bi in range(sc.beams):
            blk = p.block_tables[gi * sc.beams + bi, P]
            assert same_bits(kc[blk, :t0], p.k_cache[sc.stem_block[gi], :t0])
    rng = np.random.default_rng(0)
    units = [(int(s), int(h)) for s, h in zip(rng.integers(0, 96, 24), rng.integers(0, 40, 24))]
    out = oracle.decode(p.q, kc, vc, p.block_tables, p.context_lens, p.scale, "f16",
                        units=np.array(units, np.int32))
    ref = np_reference(W.Paged("f16", p.q, kc, vc, p.block_tables, p.context_lens, p.scale, 16),
                       units=units)
    for s, h in units:
        assert np.isfinite(out[s, h]).all()
        assert np.allclose(out[s, h], ref[s, h], rtol=1e-12, atol=1e-13)


def test_tolerance_helper_rejects_a_planted_error():
    """The tolerance check itself must fail on a wrong result."""
    ref = np.linspace(-1, 1, 64).reshape(2, 32)
    assert_fp_close(ref + 1e-4, ref, "f16")
    with pytest.raises(AssertionError):
        assert_fp_close(ref + 5e-3, ref, "f16")
    with pytest.raises(AssertionError):
        assert_fp_close(ref * (1 + 3e-5), ref, "f32")
