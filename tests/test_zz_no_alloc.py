"""pa_decode_no_alloc: pa_decode with its split-K partials in the library's
fixed device array instead of a caller's workspace.

Through the C ABI, against pa_decode (same kernels: the outputs must be
bitwise equal) and against the fp64 oracle (the attention tolerance), on
calls in a row where each later call is smaller than the one before, so a
call that read partials the previous one left in the array would show."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import empty_out, f64, to_dev, to_host, upload
from helpers import assert_fp_close, same_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def both(p, ps, layout="NHD"):
    """(no_alloc output, pa_decode output) on the same device inputs."""
    import torch

    import paged_kv_cache_pa_amd as pa

    q, k, v, bt, cl = upload(p, layout)
    mcl = int(p.context_lens.max(initial=0))
    a, b = empty_out(p), empty_out(p)
    pa.pa_decode_no_alloc(q, k, v, bt, cl, p.scale, a, max_context_len=mcl, partition_size=ps,
                          layout=layout)
    torch.cuda.synchronize()
    pa.pa_decode(q, k, v, bt, cl, p.scale, b, max_context_len=mcl, partition_size=ps,
                 layout=layout)
    torch.cuda.synchronize()
    return to_host(a, p.dtype), to_host(b, p.dtype)


def ref(p, layout="NHD"):
    return oracle.decode(p.q, p.k_cache, p.v_cache, p.block_tables, p.context_lens, p.scale,
                         p.dtype)


def check(p, ps, what, layout="NHD"):
    print(what, flush=True)
    got, want = both(p, ps, layout)
    assert same_bits(got, want), f"{what}: pa_decode_no_alloc differs from pa_decode"
    assert_fp_close(f64(got, p.dtype), ref(p), p.dtype, what)


def test_no_alloc_calls_in_a_row():
    import paged_kv_cache_pa_amd as pa

    import workloads

    # 1: the grouped-query long-context batch, 8 x 12 heads x 32 partitions
    p1 = W.config5()
    need1 = pa.pa_decode_workspace_size(pa.DecodeParams(
        8, 12, 2, 128, 16, p1.max_blocks_per_seq, p1.num_blocks, int(p1.context_lens.max()), 512,
        2, 0))
    assert 0 < need1 <= pa.NO_ALLOC_SCRATCH_BYTES
    check(p1, 512, "call 1: grouped-query bf16, 8 seqs to 16384 tokens, split 512")
    # 2: smaller, fp16 with 4 query heads per kv head and short partitions,
    # an empty sequence and a single-token one
    p2 = workloads.random_paged(811, "f16", [1, 300, 77, 0, 1000], 8, 2, 128)
    check(p2, 64, "call 2: fp16 G 4, 5 seqs, split 64", layout="NHD")
    # 3: smaller still, fp32 multi-head on the other decode kernel, head-major pool
    p3 = workloads.random_paged(812, "f32", [40, 3, 129], 4, 4, 64)
    check(p3, 32, "call 3: fp32 MHA, 3 seqs, split 32", layout="HND")
    # 4: no split (no scratch use at all)
    check(p2, 0, "call 4: no split")


def test_no_alloc_largest_fitting_split():
    """A split whose partials fill most of the 16 MiB array (64 sequences x
    40 heads x 12 partitions), then a small call."""
    import paged_kv_cache_pa_amd as pa

    lens = np.random.default_rng(813).integers(1, 12 * 128 + 1, size=64)
    lens[0] = 12 * 128
    p = W.random_paged(813, "f16", lens, 40, 40, 128, poison=False)
    need = pa.pa_decode_workspace_size(pa.DecodeParams(
        64, 40, 40, 128, 16, p.max_blocks_per_seq, p.num_blocks, 12 * 128, 128, 1, 1))
    assert need > 15 << 20 and need <= pa.NO_ALLOC_SCRATCH_BYTES
    check(p, 128, "64 x 40 heads, 12 partitions of 128", layout="HND")
    small = W.random_paged(814, "f16", [200, 5], 40, 40, 128)
    check(small, 128, "then 2 seqs, 2 partitions", layout="HND")


def test_no_alloc_in_a_hip_graph():
    """Captured into a HIP graph and replayed (the use it is made for): every
    replay, with the program's own eager work between replays, gives the
    eager result bit for bit."""
    import torch

    import paged_kv_cache_pa_amd as pa

    p = W.config5()
    q, k, v, bt, cl = upload(p)
    mcl = int(p.context_lens.max())
    eager = empty_out(p)
    pa.pa_decode_no_alloc(q, k, v, bt, cl, p.scale, eager, max_context_len=mcl, partition_size=512)
    torch.cuda.synchronize()
    want = to_host(eager, p.dtype)
    out = empty_out(p)
    st = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        pa.pa_decode_no_alloc(q, k, v, bt, cl, p.scale, out, max_context_len=mcl,
                              partition_size=512)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=st):
        pa.pa_decode_no_alloc(q, k, v, bt, cl, p.scale, out, max_context_len=mcl,
                              partition_size=512, stream=st)
    other = W.random_paged(815, "bf16", [700, 33], 12, 2, 128)
    for i in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert same_bits(to_host(out, p.dtype), want), f"replay {i}"
        # eager work between replays, on the same scratch array
        a, b = both(other, 256)
        assert same_bits(a, b)
    del g
