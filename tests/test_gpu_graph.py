"""The hot path captured in a HIP graph (torch.cuda.CUDAGraph) and replayed,
as a serving loop replays one captured step per iteration.

One graph holds a whole iteration: pa_copy_blocks (copy-on-write pairs),
pa_cache_write (the new tokens), pa_decode (split-K and merge, or not),
pa_decode_append on a second pool, and pa_prefill.  Between replays eager
work poisons every output and every location the graph writes (NaN), with
synchronisations in between; each replay must then give, bit for bit, what
the same calls give eagerly, and what the fp64 oracle computes for the same
iteration (pools bit-exact, attention outputs within the stated tolerance).
The library issues kernel launches only (no memsets, copies or
allocations), so a graph holds exactly its kernels.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import f64, in_layout, to_dev, to_host, torch_dtype
from helpers import assert_fp_close, same_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _newest_slots(p):
    """Slot of position n - 1 of each sequence (-1 for an empty one)."""
    B = p.block_size
    return np.array([p.block_tables[s, (n - 1) // B] * B + (n - 1) % B if n else -1
                     for s, n in enumerate(p.context_lens)], np.int32)


def _oracle_iteration(p, layout, dtype, pairs, kn, vn, slots, qp, qs):
    """The iteration below computed by the oracle: pools and outputs."""
    k0, v0 = in_layout(p.k_cache, layout), in_layout(p.v_cache, layout)
    k1, v1 = oracle.copy_blocks(k0, v0, pairs, dtype, layout=layout)
    k, v = oracle.cache_write(kn, vn, k1, v1, slots, dtype, layout=layout)
    out = oracle.decode(p.q, k, v, p.block_tables, p.context_lens, p.scale, dtype, layout=layout)
    k2, v2 = oracle.cache_write(kn, vn, k0, v0, slots, dtype, layout=layout)
    out2 = oracle.decode(p.q, k2, v2, p.block_tables, p.context_lens, p.scale, dtype,
                         layout=layout)
    res = dict(k=k, v=v, k2=k2, v2=v2, out=out, out2=out2)
    if dtype != "f32":
        res["outp"] = oracle.prefill(qp, k, v, p.block_tables, p.context_lens, qs, p.scale,
                                     dtype, layout=layout)
    return res


@pytest.mark.parametrize("dtype,hq,hkv", [("f16", 8, 8), ("bf16", 12, 2), ("f32", 4, 2)])
@pytest.mark.parametrize("ps", [0, 64])
@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_iteration_graph_replays_match_eager_and_oracle(dtype, hq, hkv, ps, layout):
    import torch

    import paged_kv_cache_pa_amd as pa

    D = 128 if dtype != "f32" else 64
    p = W.random_paged(81, dtype, [1, 16, 17, 200, 0, 513], hq, hkv, D, extra_blocks=6)
    rng = np.random.default_rng(82)
    S, B, NB = len(p.context_lens), p.block_size, p.num_blocks
    td = torch_dtype(dtype)
    slots = _newest_slots(p)
    kn, vn = W.randn(rng, (S, hkv, D), dtype), W.randn(rng, (S, hkv, D), dtype)
    used = set(p.block_tables[p.block_tables >= 0].tolist())
    spare = [b for b in range(NB) if b not in used]
    pairs = np.array([[p.block_tables[3, 0], spare[0]], [p.block_tables[5, 2], spare[1]]],
                     np.int32)
    chunks = np.minimum(p.context_lens, 24).astype(np.int32)
    qs = np.zeros(S + 1, np.int32)
    qs[1:] = np.cumsum(chunks)
    qp = W.randn(rng, (int(qs[-1]), hq, D), dtype)
    mcl = int(p.context_lens.max())

    k0, v0 = to_dev(in_layout(p.k_cache, layout), dtype), to_dev(in_layout(p.v_cache, layout), dtype)
    dev = dict(q=to_dev(p.q, dtype), bt=to_dev(p.block_tables), cl=to_dev(p.context_lens),
               kn=to_dev(kn, dtype), vn=to_dev(vn, dtype), slots=to_dev(slots),
               pairs=to_dev(pairs), qp=to_dev(qp, dtype), qs=to_dev(qs))
    params = pa.DecodeParams(S, hq, hkv, D, B, p.max_blocks_per_seq, NB, mcl, ps,
                             {"f32": 0, "f16": 1, "bf16": 2}[dtype], pa.LAYOUTS[layout])
    ws_bytes = pa.pa_decode_workspace_size(params)

    def buffers():
        return dict(k=k0.clone(), v=v0.clone(), k2=k0.clone(), v2=v0.clone(),
                    out=torch.empty(p.q.shape, dtype=td, device=k0.device),
                    out2=torch.empty(p.q.shape, dtype=td, device=k0.device),
                    outp=torch.empty(qp.shape, dtype=td, device=k0.device),
                    ws=torch.empty(max(1, ws_bytes // 4), dtype=torch.float32, device=k0.device))

    def iteration(b):
        pa.pa_copy_blocks(b["k"], b["v"], dev["pairs"], layout=layout)
        pa.pa_cache_write(dev["kn"], dev["vn"], b["k"], b["v"], dev["slots"], layout=layout)
        pa.pa_decode(dev["q"], b["k"], b["v"], dev["bt"], dev["cl"], p.scale, b["out"],
                     max_context_len=mcl, partition_size=ps, workspace=b["ws"], layout=layout)
        pa.pa_decode_append(dev["q"], dev["kn"], dev["vn"], b["k2"], b["v2"], dev["bt"],
                            dev["cl"], p.scale, b["out2"], max_context_len=mcl,
                            partition_size=ps, workspace=b["ws"], layout=layout)
        if dtype != "f32":       # prefill runs in 16-bit types only
            pa.pa_prefill(dev["qp"], b["k"], b["v"], dev["bt"], dev["cl"], dev["qs"], p.scale,
                          b["outp"], layout=layout)

    # eager reference
    ref = buffers()
    iteration(ref)
    torch.cuda.synchronize()
    skip = {"ws"} | ({"outp"} if dtype == "f32" else set())
    want = {name: to_host(t, dtype) for name, t in ref.items() if name not in skip}
    expect = _oracle_iteration(p, layout, dtype, pairs, kn, vn, slots, qp, qs)

    # capture (after one eager call on a side stream, so every lazily
    # initialised piece of state exists before the capture starts)
    g_buf = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        iteration(buffers())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        iteration(g_buf)
    torch.cuda.synchronize()

    nan_rows = to_dev(W.nan_fill((S, hkv, D), dtype), dtype)
    for replay in range(4):
        # eager poison of everything the graph writes
        for name in ("out", "out2", "outp"):
            g_buf[name].fill_(float("nan"))       # (outp stays NaN for f32: not in want)
        for kk, vv in (("k", "v"), ("k2", "v2")):
            pa.pa_cache_write(nan_rows, nan_rows, g_buf[kk], g_buf[vv], dev["slots"],
                              layout=layout)
        dst = torch.from_numpy(pairs[:, 1]).long().to(k0.device)   # the copies' targets
        g_buf["k"][dst] = float("nan")
        g_buf["v"][dst] = float("nan")
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, w in want.items():
            got = to_host(g_buf[name], dtype)
            assert same_bits(got, w), (replay, name)
            if name in ("k", "v", "k2", "v2"):
                assert same_bits(got, expect[name]), (replay, name, "oracle")
            else:
                assert_fp_close(f64(got, dtype), expect[name], dtype, f"replay {replay} {name}")
