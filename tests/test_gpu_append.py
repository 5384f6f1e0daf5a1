"""pa_decode_append (the newest token's write and the attention in one
launch) against the two-launch path it replaces (pa_cache_write of each
sequence's newest slot, then pa_decode) and against the fp64 oracle.

Pools must match bit for bit.  Outputs: the matrix-core kernel (grouped
query heads, 16-bit types) reads the newest token inside its loop, in the
same order as pa_decode, so its outputs match bit for bit too; the VALU
kernel adds that token after its loop (one more online-softmax step), so
its outputs differ from pa_decode's only in rounding order and are checked
to the same tolerance as against the oracle.  Covers the VALU kernel (fp32,
MHA fp16), the matrix-core kernel (grouped-query bf16, split-K), narrow
blocks, empty and one-token sequences, both pool layouts."""
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


def newest(p: W.Paged):
    """The newest token's rows (taken out of the pool, whose slot is then
    NaN) and the slot of each sequence (-1 for empty ones)."""
    S = p.q.shape[0]
    NB, B, Hkv, D = p.k_cache.shape
    k, v = p.k_cache.copy(), p.v_cache.copy()
    kn = W.nan_fill((S, Hkv, D), p.dtype)
    vn = W.nan_fill((S, Hkv, D), p.dtype)
    slots = np.full(S, -1, np.int32)
    poison = W.nan_fill((Hkv, D), p.dtype)
    for s in range(S):
        n = int(p.context_lens[s])
        if n == 0:
            continue
        b, o = int(p.block_tables[s][(n - 1) // B]), (n - 1) % B
        kn[s], vn[s] = k[b, o], v[b, o]
        k[b, o], v[b, o] = poison, poison
        slots[s] = b * B + o
    return k, v, kn, vn, slots


CASES = [
    ("f32 mha", lambda: W.random_paged(91, "f32", [37, 1, 0, 64, 100], 4, 4, 64)),
    ("f16 mha", lambda: W.random_paged(92, "f16", [300, 17, 1, 0, 129], 8, 8, 128)),
    ("bf16 gqa", lambda: W.random_paged(93, "bf16", [700, 1, 512, 33, 0, 1030], 12, 2, 128)),
    ("f16 gqa narrow", lambda: W.random_paged(94, "f16", [45, 3, 16, 0], 8, 2, 64, block_size=4)),
]


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("partition", [0, 256])
def test_append_equals_write_then_decode(name, make, layout, partition):
    import torch

    import paged_kv_cache_pa_amd as pa

    p = make()
    if partition and partition % p.block_size:
        pytest.skip("partition must be a multiple of the block size")
    k0, v0, kn, vn, slots = newest(p)
    dt = p.dtype
    mcl = int(p.context_lens.max())
    q, bt, cl = to_dev(p.q, dt), to_dev(p.block_tables), to_dev(p.context_lens)
    knd, vnd = to_dev(kn, dt), to_dev(vn, dt)

    # two launches
    k1, v1 = to_dev(in_layout(k0, layout), dt), to_dev(in_layout(v0, layout), dt)
    pa.pa_cache_write(knd, vnd, k1, v1, to_dev(slots), layout=layout)
    o1 = empty_out(p)
    pa.pa_decode(q, k1, v1, bt, cl, p.scale, o1, max_context_len=mcl, partition_size=partition,
                 layout=layout)
    # one launch
    k2, v2 = to_dev(in_layout(k0, layout), dt), to_dev(in_layout(v0, layout), dt)
    o2 = empty_out(p)
    pa.pa_decode_append(q, knd, vnd, k2, v2, bt, cl, p.scale, o2, max_context_len=mcl,
                        partition_size=partition, layout=layout)
    torch.cuda.synchronize()
    if "gqa" in name:   # dispatched to the matrix-core kernel
        assert same_bits(to_host(o2, dt), to_host(o1, dt))
    else:
        assert_fp_close(f64(to_host(o2, dt), dt), f64(to_host(o1, dt), dt), dt)
    assert same_bits(to_host(k2, dt), to_host(k1, dt))
    assert same_bits(to_host(v2, dt), to_host(v1, dt))
    # and the oracle of the same two steps
    kc, vc = oracle.cache_write(kn, vn, k0, v0, slots, dt)
    ref = oracle.decode(p.q, kc, vc, p.block_tables, p.context_lens, p.scale, dt)
    assert_fp_close(f64(to_host(o2, dt), dt), ref, dt)
    assert same_bits(to_host(k2, dt), in_layout(kc, layout))


def test_config2_append_as_benchmarked():
    """The benchmark's launch at full size: the OPT-13B-shape batch (64
    sequences, 40/40 heads, D 128, fp16), head-major pool, no split, one
    pa_decode_append launch; every sequence's newest row comes from k_new /
    v_new with its pool slot poisoned.  Pools bit-exact against the oracle's
    write; every output row against the fp64 oracle on the original pool."""
    import torch

    import paged_kv_cache_pa_amd as pa

    p = W.config2()
    k, v, kn, vn, slots = newest(p)
    print("config2 append: sum n", int(p.context_lens.sum()), flush=True)
    kd, vd = to_dev(in_layout(k, "HND"), "f16"), to_dev(in_layout(v, "HND"), "f16")
    out = empty_out(p)
    pa.pa_decode_append(to_dev(p.q, "f16"), to_dev(kn, "f16"), to_dev(vn, "f16"), kd, vd,
                        to_dev(p.block_tables), to_dev(p.context_lens), p.scale, out,
                        max_context_len=int(p.context_lens.max()), layout="HND")
    torch.cuda.synchronize()
    kw, vw = oracle.cache_write(kn, vn, k, v, slots, "f16")
    assert same_bits(to_host(kd, "f16"), in_layout(kw, "HND"))
    assert same_bits(to_host(vd, "f16"), in_layout(vw, "HND"))
    ref = oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale, "f16")
    assert_fp_close(f64(to_host(out, "f16"), "f16"), ref, "f16", "config2 decode_append HND")
