"""Parity of the HIP library with the fp64 oracle, through the C ABI.

Bit-exact for cache_write / copy_blocks and for every property that is
exact by construction (paged == dense, block placement, n = 1,
determinism); the attention tolerance otherwise (fp16/bf16: |err| <=
2e-3 + 1e-2 |ref| elementwise; fp32: 1e-5 row-normwise)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import empty_out, f64, head_major, in_layout, run_decode, to_dev, to_host, upload
from helpers import assert_fp_close, same_bits

pytestmark = pytest.mark.gpu
LAYOUTS = ["NHD", "HND"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_pa_amd as pa

    print("library:", pa.lib().pa_build_info().decode(), flush=True)


def ref_decode(p: W.Paged, units=None):
    return oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale,
                         p.dtype, units=units)


def check(p, got, ref, what, units=None):
    g = f64(got, p.dtype)
    if units is not None:
        idx = tuple(np.array(units).T)
        g, ref = g[idx], ref[idx]
    assert_fp_close(g, ref, p.dtype, what)


# ---------------------------------------------------------------- the configurations


@pytest.mark.parametrize("layout", LAYOUTS)
def test_config1_write_then_decode(layout):
    import torch

    import paged_kv_cache_pa_amd as pa

    p = W.config1()
    q, k, v, bt, cl = upload(p, layout)
    pa.pa_cache_write(to_dev(p.k_new), to_dev(p.v_new), k, v, to_dev(p.slot_mapping), layout=layout)
    torch.cuda.synchronize()
    kc, vc = oracle.cache_write(p.k_new, p.v_new, in_layout(p.k_cache, layout),
                                in_layout(p.v_cache, layout), p.slot_mapping, "f32", layout=layout)
    assert same_bits(to_host(k, "f32"), kc) and same_bits(to_host(v, "f32"), vc)
    ref = oracle.decode(p.q, kc, vc, p.block_tables, p.context_lens, p.scale, "f32", layout=layout)
    pw = W.Paged("f32", p.q, kc, vc, p.block_tables, p.context_lens, p.scale, 16)
    for ps in (0, 16, 32, 64):
        got = run_decode(pw, partition_size=ps, tensors=(q, k, v, bt, cl), layout=layout)
        check(pw, got, ref, f"config1 {layout} partition {ps}")


@pytest.fixture(scope="module")
def cfg2():
    p = W.config2()
    return p, ref_decode(p)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_config2_full(cfg2, layout):
    p, ref = cfg2
    t = upload(p, layout)
    outs = {}
    for ps in (0, 256, 512):
        outs[ps] = run_decode(p, partition_size=ps, tensors=t, layout=layout)
        check(p, outs[ps], ref, f"config2 {layout} partition {ps}")
    # with 1024 <= partition, one partition covers every sequence: same bits as no split
    assert same_bits(run_decode(p, partition_size=2048, tensors=t, layout=layout), outs[0])


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("batch,ctx", [(8, 64), (8, 256), (32, 256), (8, 1024), (8, 2048), (32, 64),
                                       (128, 64)])
def test_config3_paged_vs_dense(batch, ctx, layout):
    import torch

    import paged_kv_cache_pa_amd as pa

    p = W.config3(batch, ctx)
    ref = oracle.decode_dense(p.q, p.k_dense, p.v_dense, p.context_lens, p.scale, "f16")
    t = upload(p, layout)
    got = run_decode(p, partition_size=0, tensors=t, layout=layout)
    check(p, got, ref, f"config3 paged {layout} {batch}x{ctx}")
    out = empty_out(p)
    pa.pa_decode_dense(t[0], to_dev(in_layout(p.k_dense, layout)), to_dev(in_layout(p.v_dense, layout)),
                       t[4], p.scale, out, max_context_len=ctx, layout=layout)
    torch.cuda.synchronize()
    assert same_bits(to_host(out, "f16"), got), "paged and dense differ"


@pytest.mark.parametrize("layout", LAYOUTS)
def test_config4_cow_write_decode(layout):
    import torch

    import paged_kv_cache_pa_amd as pa

    sc = W.config4()
    p = sc.paged
    q, k, v, bt, cl = upload(p, layout)
    pa.pa_copy_blocks(k, v, to_dev(p.block_pairs), layout=layout)
    pa.pa_cache_write(to_dev(p.k_new, "f16"), to_dev(p.v_new, "f16"), k, v, to_dev(p.slot_mapping),
                      layout=layout)
    torch.cuda.synchronize()
    kc, vc = oracle.copy_blocks(in_layout(p.k_cache, layout), in_layout(p.v_cache, layout),
                                p.block_pairs, "f16", layout=layout)
    kc, vc = oracle.cache_write(p.k_new, p.v_new, kc, vc, p.slot_mapping, "f16", layout=layout)
    assert same_bits(to_host(k, "f16"), kc) and same_bits(to_host(v, "f16"), vc)
    ref = oracle.decode(p.q, kc, vc, p.block_tables, p.context_lens, p.scale, "f16", layout=layout)
    pw = W.Paged("f16", p.q, kc, vc, p.block_tables, p.context_lens, p.scale, 16)
    for ps in (0, 256):
        got = run_decode(pw, partition_size=ps, tensors=(q, k, v, bt, cl), layout=layout)
        check(pw, got, ref, f"config4 {layout} partition {ps}")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_config5_gqa_split(layout):
    p = W.config5()
    ref = ref_decode(p)
    t = upload(p, layout)
    # 512: the configured split (512 workgroups); 384 and 336: grids of 688
    # and 784 workgroups, more than fit at once, on 4-wave workgroups
    for ps in (512, 384, 336):
        got = run_decode(p, partition_size=ps, tensors=t, layout=layout)
        check(p, got, ref, f"config5 {layout} partition {ps}")
    got0 = run_decode(p, partition_size=0, tensors=t, layout=layout)
    check(p, got0, ref, f"config5 {layout} no split")


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("n", [4096, 10000, 12000, 16384])
def test_config5_uniform_batches(n, layout):
    """Every row (8 sequences x 12 query heads) of each uniform batch."""
    p = W.config5(uniform_len=n)
    ref = ref_decode(p)
    t = upload(p, layout)
    got = run_decode(p, partition_size=512, tensors=t, layout=layout)
    check(p, got, ref, f"config5 uniform {n} {layout}")


# ---------------------------------------------------------------- the pages' fixtures


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_hand_weights_gpu(golden, dtype):
    """Weights 1/7, 2/7, 4/7 -> out [5, 10, 0, 1] (head_dim padded with zeros to 64)."""
    g = golden("hand_weights.json")
    B, NB, D = g["block_size"], g["num_blocks"], 64
    k, v = W.nan_fill((NB, B, 1, D), dtype), W.nan_fill((NB, B, 1, D), dtype)
    for t in range(g["context_len"]):
        blk = g["block_table"][t // B]
        row_k = np.zeros(D, np.float32)
        row_v = np.zeros(D, np.float32)
        row_k[:4] = g["k"][t]
        row_v[:4] = g["v"][t]
        k[blk, t % B, 0] = W.to_storage(row_k, dtype)
        v[blk, t % B, 0] = W.to_storage(row_v, dtype)
    qv = np.zeros((1, 1, D), np.float32)
    qv[0, 0, :4] = g["q"]
    p = W.Paged(dtype, W.to_storage(qv, dtype), k, v, np.array([g["block_table"]], np.int32),
                np.array([g["context_len"]], np.int32), g["scale"], B)
    got = f64(run_decode(p), dtype)[0, 0]
    want = np.zeros(D)
    want[:4] = g["out"]
    assert_fp_close(got[None], want[None], dtype, f"hand weights {dtype}")


def test_fig6_write_and_gather_gpu(golden):
    import torch

    import paged_kv_cache_pa_amd as pa

    g = golden("fig6_block_table.json")
    B, NB, n, D = g["block_size"], g["num_blocks"], g["context_len"], 64
    slots = np.array(g["slots"], np.int32)
    k0, v0 = W.nan_fill((NB, B, 1, D), "f32"), W.nan_fill((NB, B, 1, D), "f32")
    v_new = np.repeat(np.arange(n, dtype=np.float32)[:, None, None], D, axis=2)
    table = np.array([g["block_table"]], np.int32)
    for j in range(n):
        k_new = np.zeros((n, 1, D), np.float32)
        k_new[j, 0, 0] = 60.0
        k, v = to_dev(k0), to_dev(v0)
        pa.pa_cache_write(to_dev(k_new), to_dev(v_new), k, v, to_dev(slots))
        torch.cuda.synchronize()
        kc, vc = oracle.cache_write(k_new, v_new, k0, v0, slots, "f32")
        assert same_bits(to_host(k, "f32"), kc) and same_bits(to_host(v, "f32"), vc)
        q = np.zeros((1, 1, D), np.float32)
        q[0, 0, 0] = 1.0
        p = W.Paged("f32", q, kc, vc, table, np.array([n], np.int32), 1.0, B)
        got = run_decode(p, tensors=(to_dev(q), k, v, to_dev(table), to_dev(p.context_lens)))
        assert np.allclose(got[0, 0], j, rtol=0, atol=1e-6), (j, got[0, 0, :4])


# ---------------------------------------------------------------- edge cases

EDGE_LENS = [0, 1, 15, 16, 17, 31, 32, 33, 511, 512, 513, 1000]


@pytest.mark.parametrize("dtype,hq,hkv,d", [("f32", 8, 8, 64), ("f32", 4, 2, 128),
                                            ("f16", 8, 8, 128), ("f16", 6, 3, 64),
                                            ("bf16", 12, 2, 128), ("bf16", 8, 1, 64)])
@pytest.mark.parametrize("ps", [0, 32, 512])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_edge_lengths(dtype, hq, hkv, d, ps, layout):
    p = W.random_paged(21, dtype, EDGE_LENS, hq, hkv, d)
    got = run_decode(p, partition_size=ps, layout=layout)
    check(p, got, ref_decode(p), f"edge lengths {layout} {dtype} {hq}/{hkv} D{d} ps{ps}")
    assert (f64(got[0], dtype) == 0).all(), "empty sequence must give zeros"


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("B", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_block_sizes(B, layout):
    p = W.random_paged(22, "f16", [1, B - 1 if B > 1 else 1, B, B + 1, 3 * B + 5, 700], 4, 2, 128,
                       block_size=B)
    for ps in (0, max(B, 256)):
        got = run_decode(p, partition_size=ps, layout=layout)
        check(p, got, ref_decode(p), f"block size {B} {layout} ps {ps}")


@pytest.mark.parametrize("G", range(1, 17))
def test_head_groups(G):
    p = W.random_paged(23, "bf16", [5, 77, 300], 2 * G, 2, 64)
    check(p, run_decode(p), ref_decode(p), f"G={G}")
    check(p, run_decode(p, partition_size=64), ref_decode(p), f"G={G} split")


@pytest.mark.parametrize("G", [12, 16])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_wide_head_groups_f16_d128(G, layout):
    """9..16 query heads per kv head (16-bit types, matrix cores), head dim
    128, with split-K and a ragged batch."""
    p = W.random_paged(29, "f16", [1, 16, 17, 513, 1000], 4 * G, 4, 128)
    for ps in (0, 256):
        check(p, run_decode(p, partition_size=ps, layout=layout), ref_decode(p),
              f"G={G} {layout} ps {ps}")


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_single_token_is_exact(dtype):
    p = W.random_paged(24, dtype, [1, 1, 1], 8, 4, 128)
    got = run_decode(p)
    for s in range(3):
        b = p.block_tables[s, 0]
        for h in range(8):
            assert same_bits(got[s, h], p.v_cache[b, 0, h // 2]), (s, h)


# ---------------------------------------------------------------- exact properties


@pytest.mark.parametrize("dtype", W.DTYPES)
@pytest.mark.parametrize("ps", [0, 32])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_paged_equals_dense_bitwise(dtype, ps, layout):
    import torch

    import paged_kv_cache_pa_amd as pa

    p = W.random_with_dense(25, dtype, [0, 1, 16, 17, 100, 333], 8, 4, 128)
    smax = p.k_dense.shape[1]
    paged = run_decode(p, partition_size=ps, max_context_len=smax, layout=layout)
    out = empty_out(p)
    pa.pa_decode_dense(to_dev(p.q, dtype), to_dev(in_layout(p.k_dense, layout), dtype),
                       to_dev(in_layout(p.v_dense, layout), dtype), to_dev(p.context_lens),
                       p.scale, out, max_context_len=smax, partition_size=ps, layout=layout)
    torch.cuda.synchronize()
    dense = to_host(out, dtype)
    assert same_bits(paged, dense)
    check(p, dense, oracle.decode_dense(p.q, p.k_dense, p.v_dense, p.context_lens, p.scale, dtype),
          "dense")


def test_block_placement_invariance_bitwise():
    p = W.random_paged(26, "f16", [3, 64, 129, 1000], 8, 8, 128, extra_blocks=20)
    base = run_decode(p, partition_size=256)
    rng = np.random.default_rng(5)
    pi = rng.permutation(p.num_blocks).astype(np.int32)
    k2, v2 = np.empty_like(p.k_cache), np.empty_like(p.v_cache)
    k2[pi], v2[pi] = p.k_cache, p.v_cache
    t2 = np.where(p.block_tables >= 0, pi[np.maximum(p.block_tables, 0)], -1).astype(np.int32)
    p2 = W.Paged("f16", p.q, k2, v2, t2, p.context_lens, p.scale, 16)
    assert same_bits(run_decode(p2, partition_size=256), base)


def test_determinism():
    p = W.random_paged(27, "bf16", [4000, 17, 2500], 12, 2, 128)
    t = upload(p)
    first = run_decode(p, partition_size=512, tensors=t)
    for _ in range(9):
        assert same_bits(run_decode(p, partition_size=512, tensors=t), first)


def test_poison_is_never_read():
    """NaN in every unused slot and unassigned block; NaN-free output."""
    p = W.random_paged(28, "f16", [1, 17, 250], 8, 8, 128, extra_blocks=30, mbs=40)
    got = run_decode(p)
    assert np.isfinite(f64(got, "f16")).all()
    check(p, got, ref_decode(p), "poisoned pool")


# ---------------------------------------------------------------- indexing kernels


@pytest.mark.parametrize("dtype", W.DTYPES)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_cache_write_bit_exact(dtype, layout):
    import torch

    import paged_kv_cache_pa_amd as pa

    rng = np.random.default_rng(29)
    NB, B, H, D = 40, 16, 4, 64
    k0, v0 = W.nan_fill((NB, B, H, D), dtype), W.nan_fill((NB, B, H, D), dtype)
    k0, v0 = in_layout(k0, layout), in_layout(v0, layout)
    N = 300
    slots = rng.permutation(NB * B)[:N].astype(np.int32)
    slots[::7] = -1
    kn, vn = W.randn(rng, (N, H, D), dtype), W.randn(rng, (N, H, D), dtype)
    k, v = to_dev(k0, dtype), to_dev(v0, dtype)
    pa.pa_cache_write(to_dev(kn, dtype), to_dev(vn, dtype), k, v, to_dev(slots), layout=layout)
    torch.cuda.synchronize()
    kc, vc = oracle.cache_write(kn, vn, k0, v0, slots, dtype, layout=layout)
    assert same_bits(to_host(k, dtype), kc) and same_bits(to_host(v, dtype), vc)


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_copy_blocks_bit_exact(dtype):
    import torch

    import paged_kv_cache_pa_amd as pa

    rng = np.random.default_rng(30)
    NB, B, H, D = 64, 16, 8, 128
    k0, v0 = W.randn(rng, (NB, B, H, D), dtype), W.randn(rng, (NB, B, H, D), dtype)
    perm = rng.permutation(NB)
    pairs = np.stack([perm[:20], perm[20:40]], axis=1).astype(np.int32)
    k, v = to_dev(k0, dtype), to_dev(v0, dtype)
    pa.pa_copy_blocks(k, v, to_dev(pairs))
    torch.cuda.synchronize()
    kc, vc = oracle.copy_blocks(k0, v0, pairs, dtype)
    assert same_bits(to_host(k, dtype), kc) and same_bits(to_host(v, dtype), vc)


def test_share_fixture_end_to_end(golden):
    """The four-sample fixture: copy, write, decode on the GPU vs the oracle."""
    import torch

    import paged_kv_cache_pa_amd as pa

    g = golden("share_py_tables.json")
    B, P, N = g["block_size"], g["prompt_len"], g["final_context_len"]
    NB, H, D = g["blocks_in_use"], 2, 128
    rng = np.random.default_rng(31)
    k0, v0 = W.nan_fill((NB, B, H, D), "bf16"), W.nan_fill((NB, B, H, D), "bf16")
    for t in range(P):
        b = g["prompt_blocks"][t // B]
        k0[b, t % B] = W.randn(rng, (H, D), "bf16")
        v0[b, t % B] = W.randn(rng, (H, D), "bf16")
    tab = np.array(g["tables"], np.int32)
    pairs = np.array(g["copy_pairs"], np.int32)
    slots = np.concatenate([W.slots_of(tab[i], np.arange(P, N), B) for i in range(g["samples"])])
    kn = W.randn(rng, (len(slots), H, D), "bf16")
    vn = W.randn(rng, (len(slots), H, D), "bf16")
    k, v = to_dev(k0, "bf16"), to_dev(v0, "bf16")
    pa.pa_copy_blocks(k, v, to_dev(pairs))
    pa.pa_cache_write(to_dev(kn, "bf16"), to_dev(vn, "bf16"), k, v, to_dev(slots))
    torch.cuda.synchronize()
    kc, vc = oracle.copy_blocks(k0, v0, pairs, "bf16")
    kc, vc = oracle.cache_write(kn, vn, kc, vc, slots, "bf16")
    assert same_bits(to_host(k, "bf16"), kc) and same_bits(to_host(v, "bf16"), vc)
    q = W.randn(rng, (g["samples"], 6 * H, D), "bf16")
    p = W.Paged("bf16", q, kc, vc, tab, np.full(g["samples"], N, np.int32), 0.088, B)
    got = run_decode(p, tensors=(to_dev(q, "bf16"), k, v, to_dev(tab), to_dev(p.context_lens)))
    check(p, got, ref_decode(p), "share fixture")


@pytest.mark.parametrize("S", [1, 2, 255, 256, 257, 600])
def test_batch_sizes_and_scheduling(S):
    """Batch sizes around the 256-sequence limit of longest-first order, with
    ties: every row must match (at these grids, 2 kv heads, at most 512
    workgroups, so the order is the natural one; the ranked order is
    test_longest_first_order_every_kernel's)."""
    rng = np.random.default_rng(40 + S)
    lens = rng.integers(0, 90, size=S)
    lens[::5] = 33  # many ties
    p = W.random_paged(41, "bf16", lens, 4, 2, 64, extra_blocks=2)
    for layout in LAYOUTS:
        check(p, run_decode(p, layout=layout), ref_decode(p), f"S={S} {layout}")
    check(p, run_decode(p, partition_size=32), ref_decode(p), f"S={S} split")


@pytest.mark.parametrize("dtype,S,hq,hkv,d", [
    ("bf16", 200, 16, 4, 128),   # matrix-core kernel (G 4), 800 workgroups
    ("f32", 130, 8, 4, 64),      # VALU kernel with G 2, 520 workgroups
    ("f16", 256, 3, 3, 128),     # VALU kernel, MHA, 768 workgroups, 256 sequences
    # up to 64 sequences every wave ranks on its own
    ("f16", 64, 16, 16, 128),    # VALU kernel, MHA, 1024 workgroups
    ("bf16", 33, 64, 16, 64),    # matrix-core kernel (G 4), 528 workgroups
    ("f16", 2, 300, 300, 64),    # two sequences, 600 workgroups
])
def test_longest_first_order_every_kernel(dtype, S, hq, hkv, d):
    """Longest-first order (more than 512 workgroups, at most 256 sequences,
    no split) in each decode kernel form, with many tied lengths, empty and
    one-token sequences: every row must match the oracle."""
    rng = np.random.default_rng(4000 + S)
    lens = rng.integers(0, 120, size=S)
    lens[::7] = 33
    lens[3::11] = 0
    lens[5::13] = 1
    print("case", dtype, S, hq, hkv, d, flush=True)
    p = W.random_paged(4100 + S, dtype, lens, hq, hkv, d, extra_blocks=2)
    for layout in LAYOUTS:
        check(p, run_decode(p, layout=layout), ref_decode(p), f"ranked {dtype} {layout}")


def test_side_stream():
    import torch

    import paged_kv_cache_pa_amd as pa

    p = W.random_paged(32, "f16", [100, 200], 8, 8, 128)
    q, k, v, bt, cl = upload(p)
    out = empty_out(p)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        pa.pa_decode(q, k, v, bt, cl, p.scale, out, max_context_len=200, partition_size=64)
    s.synchronize()
    check(p, to_host(out, "f16"), ref_decode(p), "side stream")


def test_binding_refuses_mismatched_head_dim():
    """q and the pool must share the head dim: the binding raises before any
    launch (decode, append, dense and prefill)."""
    import torch

    import paged_kv_cache_pa_amd as pa

    dev = "cuda"
    q = torch.zeros((2, 4, 128), dtype=torch.float16, device=dev)
    k = torch.zeros((8, 16, 4, 64), dtype=torch.float16, device=dev)
    bt = torch.zeros((2, 4), dtype=torch.int32, device=dev)
    cl = torch.ones((2,), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    with pytest.raises(ValueError, match="head dim"):
        pa.pa_decode(q, k, k, bt, cl, 1.0, out)
    kn = torch.zeros((2, 4, 64), dtype=torch.float16, device=dev)
    with pytest.raises(ValueError, match="head dim"):
        pa.pa_decode_append(q, kn, kn, k, k, bt, cl, 1.0, out)
    kd = torch.zeros((2, 32, 4, 64), dtype=torch.float16, device=dev)
    with pytest.raises(ValueError, match="head dim"):
        pa.pa_decode_dense(q, kd, kd, cl, 1.0, out)
    qs = torch.tensor([0, 1, 2], dtype=torch.int32, device=dev)
    with pytest.raises(ValueError, match="head dim"):
        pa.pa_prefill(q, k, k, bt, cl, qs, 1.0, out)


@pytest.mark.parametrize("dtype,hq,hkv", [("f16", 16, 16), ("bf16", 64, 16)])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_order_does_not_change_bits(dtype, hq, hkv, layout):
    """The same 64 sequences decoded with longest-first order (1024
    workgroups) in their own order, reversed and in a random order: the
    ranking hands each sequence to a different workgroup in each launch,
    which never changes its arithmetic at one launch shape (the wave count,
    which splits a sequence's steps among waves, is the same), so every row
    has the same bits in all three, and they match the oracle."""
    rng = np.random.default_rng(4200 + hq)
    S = 64
    lens = rng.integers(0, 200, size=S)
    lens[::9] = 64
    lens[4::11] = 0
    lens[6::13] = 1
    p = W.random_paged(4300 + hq, dtype, lens, hq, hkv, 128, extra_blocks=2)

    def sub(idx):
        return W.Paged(dtype, np.ascontiguousarray(p.q[idx]), p.k_cache, p.v_cache,
                       np.ascontiguousarray(p.block_tables[idx]),
                       np.ascontiguousarray(p.context_lens[idx]), p.scale, p.block_size)

    mcl = int(lens.max())
    whole = run_decode(p, max_context_len=mcl, layout=layout)
    for name, perm in (("reversed", np.arange(S)[::-1]), ("shuffled", rng.permutation(S))):
        got = np.empty_like(whole)
        got[perm] = run_decode(sub(perm), max_context_len=mcl, layout=layout)
        assert same_bits(whole, got), f"{dtype} {layout}: batch {name}"
    check(p, whole, ref_decode(p), f"order {dtype} {layout}")
