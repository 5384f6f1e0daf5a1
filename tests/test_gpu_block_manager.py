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


def _pinned(a: np.ndarray, dtype: str):
    import torch

    from gpu_util import torch_dtype

    t = torch.empty(a.shape, dtype=torch_dtype(dtype), pin_memory=True)
    src = torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if dtype == "bf16" else a)
    t.copy_(src.view(t.dtype) if dtype == "bf16" else src)
    return t


def _host(t, dtype):
    x = t.detach().contiguous()
    if dtype == "bf16":
        import torch

        return x.view(torch.int16).numpy().view(np.uint16).copy()
    return x.numpy().copy()


@pytest.mark.parametrize("layers", [3, 70])
def test_copy_blocks_layers_bit_exact(layers):
    import torch

    import paged_kv_cache_pa_amd as pa

    rng = np.random.default_rng(51)
    NB, B, H, D, dt = 24, 16, 2, 64, "f16"
    ks = [W.randn(rng, (NB, B, H, D), dt) for _ in range(layers)]
    vs = [W.randn(rng, (NB, B, H, D), dt) for _ in range(layers)]
    perm = rng.permutation(NB)
    pairs = np.stack([perm[:7], perm[7:14]], axis=1).astype(np.int32)
    pairs[3] = [NB + 5, perm[20]]            # out of range: skipped
    kd, vd = [to_dev(k, dt) for k in ks], [to_dev(v, dt) for v in vs]
    pa.pa_copy_blocks_layers(kd, vd, to_dev(pairs))
    torch.cuda.synchronize()
    kc, vc = oracle.copy_blocks_layers(ks, vs, np.delete(pairs, 3, axis=0), dt)
    for layer in range(layers):
        assert same_bits(to_host(kd[layer], dt), kc[layer])
        assert same_bits(to_host(vd[layer], dt), vc[layer])


@pytest.mark.parametrize("layers,dtype,layout,B", [(3, "f16", "HND", 16), (70, "bf16", "NHD", 4),
                                                   (5, "f32", "HND", 1)])
def test_cache_write_layers_bit_exact(layers, dtype, layout, B):
    """Every layer's new rows in one call (70 layers: two launches), against
    the oracle layer by layer; padding slots (-1) and slots past the pool are
    skipped (the oracle gets only the valid ones)."""
    import torch

    import paged_kv_cache_pa_amd as pa

    rng = np.random.default_rng(54)
    NB, H, D, N = 40, 2, 64, 23   # NB * B >= N at every block size
    ks = [in_layout(W.nan_fill((NB, B, H, D), dtype), layout) for _ in range(layers)]
    vs = [in_layout(W.nan_fill((NB, B, H, D), dtype), layout) for _ in range(layers)]
    kn = [W.randn(rng, (N, H, D), dtype) for _ in range(layers)]
    vn = [W.randn(rng, (N, H, D), dtype) for _ in range(layers)]
    slots = rng.permutation(NB * B)[:N].astype(np.int32)
    slots[3], slots[9], slots[17] = -1, NB * B, NB * B + 7
    kd, vd = [to_dev(x, dtype) for x in ks], [to_dev(x, dtype) for x in vs]
    pa.pa_cache_write_layers([to_dev(x, dtype) for x in kn], [to_dev(x, dtype) for x in vn],
                             kd, vd, to_dev(slots), layout=layout)
    torch.cuda.synchronize()
    keep = (slots >= 0) & (slots < NB * B)
    kc, vc = oracle.cache_write_layers([x[keep] for x in kn], [x[keep] for x in vn], ks, vs,
                                       slots[keep], dtype, layout=layout)
    for layer in range(layers):
        assert same_bits(to_host(kd[layer], dtype), kc[layer]), layer
        assert same_bits(to_host(vd[layer], dtype), vc[layer]), layer


@pytest.mark.parametrize("dtype,layout", [("bf16", "HND"), ("f32", "NHD")])
def test_swap_out_and_in_through_pinned_host_pools(dtype, layout):
    import torch

    import paged_kv_cache_pa_amd as pa

    rng = np.random.default_rng(52)
    L, NBG, NBH, B, H, D = 2, 30, 12, 16, 4, 64
    gk = [in_layout(W.randn(rng, (NBG, B, H, D), dtype), layout) for _ in range(L)]
    gv = [in_layout(W.randn(rng, (NBG, B, H, D), dtype), layout) for _ in range(L)]
    hk = [in_layout(W.nan_fill((NBH, B, H, D), dtype), layout) for _ in range(L)]
    hv = [in_layout(W.nan_fill((NBH, B, H, D), dtype), layout) for _ in range(L)]
    kd, vd = [to_dev(x, dtype) for x in gk], [to_dev(x, dtype) for x in gv]
    kh, vh = [_pinned(x, dtype) for x in hk], [_pinned(x, dtype) for x in hv]
    out_pairs = np.array([[5, 0], [29, 11], [7, 3], [31, 2], [0, 7]], np.int32)  # one skipped
    pa.pa_swap_blocks(kh, vh, kd, vd, to_dev(out_pairs), layout=layout)
    torch.cuda.synchronize()
    ek, ev = oracle.swap_blocks(hk, hv, gk, gv, out_pairs)
    for layer in range(L):
        assert same_bits(_host(kh[layer], dtype), ek[layer])
        assert same_bits(_host(vh[layer], dtype), ev[layer])
    # the GPU blocks are reused by someone else, then the group comes back
    valid = out_pairs[[0, 1, 2, 4]]
    for layer in range(L):
        kd[layer][torch.from_numpy(valid[:, 0]).long().cuda()] = 0
    in_pairs = np.ascontiguousarray(valid[:, ::-1])
    pa.pa_swap_blocks(kd, vd, kh, vh, to_dev(in_pairs), layout=layout)
    torch.cuda.synchronize()
    for layer in range(L):
        assert same_bits(to_host(kd[layer], dtype), gk[layer])
        assert same_bits(to_host(vd[layer], dtype), gv[layer])


def test_manager_swap_then_decode():
    """A beam group is swapped out by the manager, its GPU blocks are taken
    by another request, and after swap-in the group attends exactly as
    before."""
    import torch

    import paged_kv_cache_pa_amd as pa
    from paged_kv_cache_pa_amd.block_manager import BlockManager

    rng = np.random.default_rng(53)
    dt, lay = "f16", "HND"
    NBG, NBH, B, Hq, Hkv, D, MBS = 40, 40, 16, 8, 2, 128, 16
    scale = 1 / np.sqrt(D)
    bm = BlockManager(NBG, NBH, B)
    kd = to_dev(in_layout(W.nan_fill((NBG, B, Hkv, D), dt), lay), dt)
    vd = to_dev(in_layout(W.nan_fill((NBG, B, Hkv, D), dt), lay), dt)
    kh = _pinned(in_layout(W.nan_fill((NBH, B, Hkv, D), dt), lay), dt)
    vh = _pinned(in_layout(W.nan_fill((NBH, B, Hkv, D), dt), lay), dt)

    def write(seqs, ks):
        slots, pairs = bm.reserve(seqs, ks)
        if len(pairs):
            pa.pa_copy_blocks(kd, vd, to_dev(np.ascontiguousarray(pairs)), layout=lay)
        n = int(sum(ks))
        pa.pa_cache_write(to_dev(W.randn(rng, (n, Hkv, D), dt), dt),
                          to_dev(W.randn(rng, (n, Hkv, D), dt), dt), kd, vd, to_dev(slots),
                          layout=lay)

    root = bm.new_seq()
    write([root], [70])
    group = [root, bm.fork(root), bm.fork(root)]
    for _ in range(5):
        write(group, [1, 1, 1])
    q = W.randn(rng, (3, Hq, D), dt)

    def attend(seqs):
        bt, cl = bm.tables(seqs, MBS)
        out = torch.empty((len(seqs), Hq, D), dtype=kd.dtype, device=kd.device)
        pa.pa_decode(to_dev(q, dt), kd, vd, to_dev(bt), to_dev(cl), scale, out,
                     max_context_len=int(cl.max()), layout=lay)
        torch.cuda.synchronize()
        return to_host(out, dt), bt, cl

    before, bt, cl = attend(group)
    ref = oracle.decode(q, to_host(kd, dt), to_host(vd, dt), bt, cl, scale, dt, layout=lay)
    assert_fp_close(f64(before, dt), ref, dt)
    out_pairs = bm.swap_out(group)
    pa.pa_swap_blocks([kh], [vh], [kd], [vd], to_dev(np.ascontiguousarray(out_pairs)), layout=lay)
    other = bm.new_seq()                      # takes the freed GPU blocks
    write([other], [bm.num_free()[0] * B])
    assert bm.num_free()[0] == 0
    bm.free([other])
    in_pairs = bm.swap_in(group)
    pa.pa_swap_blocks([kd], [vd], [kh], [vh], to_dev(np.ascontiguousarray(in_pairs)), layout=lay)
    after, bt2, cl2 = attend(group)
    assert np.array_equal(cl2, cl)
    ref2 = oracle.decode(q, to_host(kd, dt), to_host(vd, dt), bt2, cl2, scale, dt, layout=lay)
    assert_fp_close(f64(after, dt), ref2, dt)
    assert same_bits(after, before)  # moved blocks, same bytes: the same attention
